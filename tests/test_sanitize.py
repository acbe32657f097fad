"""CPU sanitizer tier: the C oracle and the library's host layer (argument
validation, workspace sizing, status strings) rebuilt with AddressSanitizer
and UndefinedBehaviorSanitizer (gcc, host code only), then the oracle's pins
and the C-ABI validation tests run against those builds in a child process
with the ASan runtime preloaded. Any sanitizer report aborts the child and
fails the test. The HIP kernels are linked in unchanged (device code is not
sanitized; no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"


def _child(script: str, runtime: str):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    print(r.stdout.strip().splitlines()[-1])


def test_oracle_pins_under_asan_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp"] + SAN +
         [os.path.join(ROOT, "oracle", "hs2_oracle.c"), "-o", lib, "-lm"])
    script = (
        "import sys; sys.path.insert(0, '.')\n"
        "import oracle\n"
        f"oracle._LIB_PATH = {lib!r}\n"
        f"assert oracle.lib()._name == {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_oracle.py']))\n")
    _child(script, runtime)


def test_host_layer_under_asan_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from token_level_top_amd import build as tbuild
    objs = []
    for src in tbuild.SOURCES:
        if src == "hs2_api.cpp":
            continue
        obj = os.path.join(tbuild.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            os.makedirs(tbuild.BUILD, exist_ok=True)
            tbuild._compile(src)
        objs.append(obj)
    api = str(tmp_path / "hs2_api_san.o")
    lib = str(tmp_path / "libhs2_san.so")
    csrc = os.path.join(ROOT, "token_level_top_amd", "csrc")
    _run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I",
          os.path.join(ROOT, "include"), "-I", csrc, "-w"] + SAN +
         ["-c", os.path.join(csrc, "hs2_api.cpp"), "-o", api])
    _run(["g++", "-shared", "-fsanitize=address,undefined", api] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    script = (
        "import sys; sys.path.insert(0, '.')\n"
        "import token_level_top_amd as t\n"
        f"t.LIB_PATH = {lib!r}\n"
        f"assert t.lib()._name == {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
    _child(script, runtime)
