"""Build libhs2.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each kernel's register, scratch, LDS and occupancy figures (the compiler's
kernel-resource-usage remarks) are written to _build/resource_usage.json, so
that a spill the compiler introduces after an edit is seen rather than only
felt as a slower kernel."""
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhs2.so")
RESOURCES = os.path.join(BUILD, "resource_usage.json")
SOURCES = ["hs2_api.cpp", "k_rows.hip", "k_decode.hip", "k_select.hip", "k_prefill.hip", "k_project.hip",
           "k_block.hip", "k_index.hip", "k_probe.hip", "hs2_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-Wall", "-Wno-unused-function",
          # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Rpass-analysis=kernel-resource-usage"]

_REMARK = "[-Rpass-analysis=kernel-resource-usage]"
_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds"}


def _resources(text: str) -> dict:
    """kernel (mangled name) -> its resource figures, from the remarks"""
    out, cur = {}, None
    for line in text.splitlines():
        if _REMARK not in line:
            continue
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass", line)
        if m and cur is not None and m.group(1) in _FIELDS:
            v = m.group(2)
            cur[_FIELDS[m.group(1)]] = int(v) if v.isdigit() else v
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    res = _resources(text)
    # the remarks and the source lines the compiler quotes under them are not printed
    lines, skip = [], 0
    for l in text.splitlines():
        if _REMARK in l:
            skip = 2 if "Function Name" in l else 0
            continue
        if skip:
            skip -= 1
            continue
        if "not a recognized feature" not in l:
            lines.append(l)
    out = "\n".join(lines)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out)
    return obj, res


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    res = {}
    for src, (_, r) in zip(SOURCES, done):
        for k, v in r.items():
            res[k] = dict(v, source=src)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
