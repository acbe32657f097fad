#!/usr/bin/env python3
"""Throughput of the HySparse2 attention hot path on one MI355X.

One step = the whole path for one batch of synthetic inputs:
  decode workloads  -- hs2_decode_step: full layer over the cache (split-K
                       attention + token scores + window/top-k selection) and
                       the reusing sparse layers;
  prefill workloads -- hs2_full_attn_select (pass 1, pass 2 with streaming
                       top-k, final selection) then hs2_sparse_attn over all
                       reusing layers.
Inputs are generated on the host (hs2_inputs), copied to HBM before timing,
and every output buffer and workspace is allocated before the timed region.

Prints one JSON line. `value` is query tokens per second for the whole step.
`roofline` prices the dominant kernel (decode: split-K attention, HBM-bound;
prefill: pass-1 attention, MFMA-bound) from its algorithmic bytes or flops per
launch and its average duration, measured with hipEvents recorded on the
launch stream by the library's timing hook during the timed steps.
`cpu_baseline` times the double-precision CPU oracle on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query tok/s, full attn+top-1024 select+sparse reuse @128k; % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}

# kernel classes of the library's timing hook (include/hs2.h)
KC = {"decode_split_attn": 0, "combine": 1, "decode_score": 2, "select_hist": 3, "select_collect": 4,
      "select_final": 5, "sparse_attn": 6, "prep_kv": 7, "attn_fwd": 8, "score_stream": 9,
      "window_pass": 10, "fill": 11, "kv_project": 12, "block_score": 13, "block_select": 14,
      "decode_rescore": 15}
# kernel source file each priced kernel lives in (for the traffic record's freshness check)
KSRC = {"decode_split_attn": "k_decode.hip", "attn_fwd": "k_prefill.hip", "score_stream": "k_prefill.hip",
        "kv_project": "k_project.hip"}


def device_name() -> str:
    """The GPU the line was measured on (name and ISA)."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return f"{p.name} ({getattr(p, 'gcnArchName', '?')}, {p.multi_processor_count} CUs)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kv_bytes(kv: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[kv]


def causal_pairs(wl) -> int:
    # sum over queries of (p + 1), p = q_pos0 + i
    n, p0 = wl.n_q, wl.q_pos0
    return wl.B * (n * p0 + n * (n + 1) // 2)


def logit_bytes(wl, h: int) -> float:
    """Bytes per key of the decode logits between the split and score kernels
    in the timed step (no score vector requested): fp32 for fp32 caches, else
    an 8-bit code per head plus the fp32 maxima of each 32-key block (h/8
    bytes a key)."""
    return 4 * h if wl.kv_dtype == "f32" else h + h / 8


def path_roofline_seconds(wl, blocks: bool = False, h_full: int = 0) -> float:
    """Lower bound on one step from the method's algorithmic work (HBM or MFMA).
    blocks: the HySparse v1 variant, whose two branches attend to min(p+1, W)
    and min(p+1, K) rows. h_full: query heads of the full layer when it has
    fewer than the sparse layers (0: the same)."""
    hf = h_full or wl.H
    b = kv_bytes(wl.kv_dtype)
    sb = 4 if wl.kv_dtype == "fp8" else 0
    S = wl.window + wl.k_global
    if wl.decode:
        # K + V read once, the logits written and read once, the score written and read once
        full = wl.B * wl.n_ctx * (2 * (wl.d * b + sb) + 2 * logit_bytes(wl, hf) + 8) / (HBM_PEAK_GBS * 1e9)
        sparse = wl.n_sparse * wl.B * S * 2 * (wl.d * b + sb) / (HBM_PEAK_GBS * 1e9)
        return full + sparse
    peak = MFMA_PEAK_TFLOPS["f32" if wl.q_dtype == "f32" else "bf16"] * 1e12
    full = 6 * wl.d * hf * causal_pairs(wl) / peak
    # every query attends to min(p+1, S) selected rows in each sparse layer
    if blocks:
        sel = sum(min(wl.q_pos0 + i + 1, wl.window) + min(wl.q_pos0 + i + 1, wl.k_global)
                  for i in range(wl.n_q)) * wl.B
    else:
        sel = sum(min(wl.q_pos0 + i + 1, S) for i in range(wl.n_q)) * wl.B
    sparse = wl.n_sparse * 4 * wl.d * wl.H * sel / peak
    return full + sparse


def dominant(wl):
    """(timing class, bound, algorithmic units per launch, unit label)."""
    if wl.decode:
        b = kv_bytes(wl.kv_dtype)
        sb = 4 if wl.kv_dtype == "fp8" else 0
        per_key = 2 * (wl.d * b + sb) + logit_bytes(wl, wl.H)  # K + V rows read, logits written
        return "decode_split_attn", "hbm", int(wl.B * wl.n_ctx * per_key), "GB/s"
    return "attn_fwd", "mfma", 4 * wl.d * wl.H * causal_pairs(wl), "TFLOP/s"


def traffic_record(name: str, workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken for this kernel on this workload with the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{name}@{workload_name}")
        src = os.path.join(ROOT, "token_level_top_amd", "csrc", KSRC[name])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if not rec or rec.get("src_sha") != sha:
            return None
        return rec
    except Exception:
        return None


def cpu_baseline(wl, x, seconds: float, blocks: bool = False, xi=None):
    import numpy as np
    import oracle
    oracle.lib()
    cores = oracle.num_threads()
    rng = np.random.default_rng(12345)
    rows_all = np.arange(wl.B * wl.n_q)
    order = rng.permutation(rows_all)
    done = 0
    t0 = time.perf_counter()
    for r in order:
        r = int(r)
        if xi is not None:
            ref = oracle.index_select(xi.qi, xi.qs, xi.w, xi.ki, xi.ks, wl.q_pos0, wl.window, wl.k_global, [r])
            oracle.sparse(x.q.contiguous(), x.k, x.v, x.k_scale, x.v_scale, ref["idx"], x.sm_scale, [r])
            for l in range(wl.n_sparse):
                oracle.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, ref["idx"], x.sm_scale, [r])
        elif blocks:
            kb = wl.k_global // 64
            ref = oracle.block_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, 64, kb, x.sm_scale, [r])
            for l in range(wl.n_sparse):
                oracle.block_sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, ref["block_idx"], 64,
                                    wl.window, np.full((wl.B * wl.n_q, wl.H, 2), 0.5), wl.q_pos0, x.sm_scale, [r])
        else:
            ref = oracle.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global,
                                     x.sm_scale, [r])
            for l in range(wl.n_sparse):
                oracle.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, ref["idx"], x.sm_scale,
                              [r])
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    what = "sequences" if wl.decode else "query rows (uniform over positions)"
    return {"value": done / el, "unit": "query tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {wl.B * wl.n_q} {what}: full attention + score + select + "
                      f"{wl.n_sparse} sparse layers, fp64, {el:.1f} s"}


def copy_calibration(mib: int, dev) -> None:
    """A plain device copy of `mib` MiB, twice: the reference the HBM byte
    counters of a profiled run are scaled by."""
    if mib <= 0:
        return
    import torch
    src = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def mfma_probe(args) -> int:
    """Attainable dense bf16 matrix-core rate on this GPU, the ceiling the
    MFMA-bound kernels are read against: hs2_probe_mfma issues nothing but
    v_mfma_f32_32x32x16_bf16 on register operands (8 independent chains a
    wave), one workgroup a CU, with one and with two waves on each SIMD, on
    constant operands (the sink checked against its exact value) and on
    N(0,1) bf16 operands (the matrix cores' power draw, and so the clock they
    hold, depends on the operand bits). hipEvents around each launch, median
    of steps."""
    import torch
    import token_level_top_amd as hs2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_blocks, iters = 1024, 2000
    res = {"metric": "dense bf16 MFMA rate (attainable ceiling)", "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "data": "synthetic", "instruction": "v_mfma_f32_32x32x16_bf16",
           "peak": MFMA_PEAK_TFLOPS["bf16"], "cases": []}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gen = torch.Generator(device=dev).manual_seed(13)
    normal_ops = torch.randn(64, 16, device=dev, generator=gen).to(torch.bfloat16)
    for operands in ("constant", "normal"):
        ops = normal_ops if operands == "normal" else None
        for wps in (1, 2):
            sink = torch.empty(n_blocks * 256 * wps, dtype=torch.float32, device=dev)
            for _ in range(args.warmup):
                hs2.probe_mfma(wps, n_blocks, iters, 1.0, ops, sink)
            times = []
            for _ in range(args.steps):
                e0.record()
                hs2.probe_mfma(wps, n_blocks, iters, 1.0, ops, sink)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            if ops is None and not bool((sink == 128.0 * iters).all()):
                raise RuntimeError("MFMA probe sink holds a wrong value")
            ms = sorted(times)[len(times) // 2]
            flops = n_blocks * 4 * wps * iters * 8 * 32768
            tf = flops / (ms / 1e3) / 1e12
            res["cases"].append({"operands": operands, "waves_per_simd": wps, "ms": round(ms, 4),
                                 "tflops": round(tf, 1), "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)})
            log(f"MFMA probe, {operands} operands, {wps} wave(s) per SIMD: {ms:.3f} ms, {tf:.1f} TFLOP/s")
    print(json.dumps(res), flush=True)
    return 0


def stream_probe(args) -> int:
    """Attainable streaming rate on this GPU, the reference the decode split
    kernel is read against: hs2_probe_stream reads a 4 GiB source once (the
    64 x 128k bf16 cache's K + V) in 4 KiB chunks dealt round-robin over 2048
    workgroups (the split kernel's grid), with no writes and with a 4 KiB copy
    written after every 8 chunks read (the split kernel's 64 bytes of logits
    per 512 bytes of K and V). hipEvents around each launch, median of steps."""
    import torch
    import token_level_top_amd as hs2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src_bytes = 64 * 131072 * 512
    src = torch.empty(src_bytes, dtype=torch.uint8, device=dev)
    src.view(torch.int32).random_(0, 1 << 30, generator=torch.Generator(device=dev).manual_seed(5))
    dst = torch.empty(src_bytes // 8, dtype=torch.uint8, device=dev)
    res = {"metric": "streaming HBM rate (reference for the decode split kernel)", "unit": "TB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "data": "synthetic", "src_bytes": src_bytes, "cases": []}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_blocks = 2048
    sink = torch.empty(n_blocks * 256, dtype=torch.int32, device=dev)
    for rpw in (0, 8):
        d = dst if rpw else None
        for _ in range(args.warmup):
            hs2.probe_stream(src, d, rpw, n_blocks, sink)
        times = []
        for _ in range(args.steps):
            e0.record()
            hs2.probe_stream(src, d, rpw, n_blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        moved = src_bytes + (src_bytes // rpw if rpw else 0)
        res["cases"].append({"reads_per_write": rpw, "n_blocks": n_blocks, "ms": round(ms, 4),
                             "bytes_moved": moved, "tb_per_s": round(moved / (ms / 1e3) / 1e12, 3)})
        log(f"stream probe, {'no writes' if not rpw else f'one write per {rpw} reads'}: {ms:.3f} ms")
    print(json.dumps(res), flush=True)
    return 0


def gather_probe(args) -> int:
    """Attainable random-row gather rate on this GPU, the reference the sparse
    layers' row rate is read against (a sparse layer gathers a K row and a V
    row per index entry, so its row rate is twice its index rate):
    hs2_probe_gather reads 8192 x 1152 rows at random positions -- as fast as
    the memory system returns them, nothing else done with them -- out of a
    source of 16 MiB (the 32k prefill's K + V, which the memory-side cache
    holds) and of 64 MiB, 256-byte rows (bf16, d = 128) and 128-byte rows with
    a 4-byte scale each (FP8). The 256-byte cases are also read as runs of 64
    consecutive rows at random 64-row-aligned starts, the access pattern of the
    block-level variant's sparse layer (64-token blocks). hipEvents around each
    launch, median of steps."""
    import torch
    import token_level_top_amd as hs2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(11)
    n_idx = 8192 * 1152
    res = {"metric": "random-row gather rate (reference for the sparse layers)", "unit": "G rows/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "data": "synthetic", "rows_per_launch": n_idx,
           "cases": []}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sink = torch.empty(524288, dtype=torch.int32, device=dev)
    for mib in (16, 64):
        for row_bytes, with_scale, run in ((256, False, 1), (128, True, 1), (256, False, 64)):
            n_rows = mib * 1024 * 1024 // row_bytes
            src = torch.randint(0, 255, (n_rows, row_bytes), dtype=torch.uint8, device=dev, generator=g)
            scale = torch.rand(n_rows, device=dev, generator=g) if with_scale else None
            starts = torch.randint(0, n_rows // run, (n_idx // run,), device=dev, generator=g) * run
            idx = (starts[:, None] + torch.arange(run, device=dev)[None, :]).reshape(-1).to(torch.int32).contiguous()
            for _ in range(args.warmup):
                hs2.probe_gather(src, idx, scale, sink)
            times = []
            for _ in range(args.steps):
                e0.record()
                hs2.probe_gather(src, idx, scale, sink)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = sorted(times)[len(times) // 2]
            rb = row_bytes + (4 if with_scale else 0)
            res["cases"].append({"source_mib": mib, "row_bytes": rb, "run_rows": run, "ms": round(ms, 4),
                                 "g_rows_per_s": round(n_idx / (ms / 1e3) / 1e9, 2),
                                 "gathered_gb_per_s": round(n_idx * rb / (ms / 1e3) / 1e9, 1)})
            log(f"gather probe {mib} MiB source, {rb}-byte rows in runs of {run}: {ms:.3f} ms")
            del src, idx, scale
    print(json.dumps(res), flush=True)
    return 0


def bench_kv_project(args, cache: str) -> int:
    """KV Bridging projections alone (hs2_kv_project): the hidden state of a
    32768-token prefill chunk, hidden 2048 (the pages' model width), projected
    into K and V of 4 bridged full layers, d = 128, cache in bf16 or FP8.
    One step = one call; value = hidden-state tokens per second."""
    import ctypes
    import numpy as np
    import torch
    import token_level_top_amd as hs2
    from hs2_inputs import make_projection_inputs

    T, hidden, J, d = 32768, 2048, 4, 128
    name = f"kv_project_{T // 1024}k_hidden{hidden}_j{J}_{cache}"
    log(f"workload {name}: generating inputs on the host")
    h, w = make_projection_inputs(2024, T, hidden, J, d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hd, wd = h.to(dev), w.to(dev)
    dt = hs2.HS2_FP8_E4M3 if cache == "fp8" else hs2.HS2_BF16
    odt = torch.uint8 if cache == "fp8" else torch.bfloat16
    bufs = dict(k_out=torch.empty((J, T, d), dtype=odt, device=dev), v_out=torch.empty((J, T, d), dtype=odt,
                                                                                        device=dev))
    if cache == "fp8":
        bufs.update(k_scale=torch.empty((J, T), device=dev), v_scale=torch.empty((J, T), device=dev))

    def step():
        hs2.kv_project(hd, wd, dt, **bufs)

    copy_calibration(args.copy_calibration_mib, dev)
    L = hs2.lib()
    L.hs2_timing_enable.argtypes = [ctypes.c_uint32]
    L.hs2_timing_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ms_c, n_c = (ctypes.c_double * 16)(), (ctypes.c_int64 * 16)()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    L.hs2_timing_read(ctypes.addressof(ms_c), ctypes.addressof(n_c))
    ms_c, n_c = (ctypes.c_double * 16)(), (ctypes.c_int64 * 16)()
    L.hs2_timing_enable(1 << KC["kv_project"])
    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    L.hs2_timing_enable(0)
    if L.hs2_timing_read(ctypes.addressof(ms_c), ctypes.addressof(n_c)) != 0:
        raise RuntimeError("hs2_timing_read failed")
    ms_total = e0.elapsed_time(e1)
    kc = KC["kv_project"]
    kavg_s = ms_c[kc] / max(n_c[kc], 1) / 1e3
    flops = 2 * T * hidden * d * 2 * J
    achieved = flops / kavg_s / 1e12
    peak = MFMA_PEAK_TFLOPS["bf16"]
    out_b = 1 if cache == "fp8" else 2
    bytes_alg = T * hidden * 2 + 2 * J * d * hidden * 2 + 2 * J * T * (d * out_b + (4 if cache == "fp8" else 0))
    tr = traffic_record("kv_project", name)
    res = {"metric": "KV Bridging projection hidden-state tok/s", "value": round(T * args.steps / (ms_total / 1e3), 2),
           "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_total / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) hidden states, N(0,1/hidden) weights)",
           "config": {"workload": name, "T": T, "hidden": hidden, "n_layers": J, "d": d, "cache": cache},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4), "traffic": tr["bytes_per_launch"] if tr else None,
                        "kernel": "kv_project", "kernel_ms": round(kavg_s * 1e3, 4),
                        "algorithmic_per_launch": flops, "algorithmic_bytes_per_launch": bytes_alg}}
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        rng = np.random.default_rng(12345)
        order = rng.permutation(T)
        done, t0 = 0, time.perf_counter()
        while done < T and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.kv_project(h, w, order[done:done + 16].tolist(), quantize=cache == "fp8")
            done += 16
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": done / el, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"{done} of {T} hidden rows, all {2 * J} projections, fp64, {el:.1f} s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: decode @128k)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel class (extra steps)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB twice (reference for HBM counters)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as replays of one captured HIP graph (the kernels and their order are the "
                         "same; launch gaps go away); the per-kernel roofline timing stays eager")
    ap.add_argument("--full-heads", type=int, default=0,
                    help="query heads of the full layer (4 or 8) when fewer than the sparse layers' 16 (asymmetric "
                         "heads); 0: the same")
    ap.add_argument("--hysparse-blocks", action="store_true",
                    help="prefill workloads: the HySparse v1 block-level variant (64-token blocks, top 16, gated "
                         "128-token window branch) in place of token-level selection")
    ap.add_argument("--window-sharing", action="store_true",
                    help="prefill: sparse layers with the window shared per query block (hs2_sparse_attn_window)")
    ap.add_argument("--indexer", action="store_true",
                    help="prefill workloads: light-indexer selection (FP8 heads, see --indexer-*) in place of the full "
                         "layer, its index rows shared IndexCache-style by 1 + n_sparse sparse layers")
    ap.add_argument("--indexer-heads", type=int, default=8, help="indexer heads (4, 8 or 16)")
    ap.add_argument("--indexer-dim", type=int, default=64, help="indexer head dimension (64 or 128)")
    ap.add_argument("--kv-project", choices=["bf16", "fp8"], default=None,
                    help="instead of the attention path, time the KV Bridging projections with this cache type")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="measure the attainable dense bf16 MFMA rate (hs2_probe_mfma) instead of the path")
    ap.add_argument("--stream-probe", action="store_true",
                    help="instead of the attention path, measure the attainable streaming rate (a reference for the "
                         "decode split kernel)")
    ap.add_argument("--gather-probe", action="store_true",
                    help="instead of the attention path, measure the attainable random-row gather rate (a reference "
                         "for the sparse layers)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2
    if args.kv_project:
        return bench_kv_project(args, args.kv_project)
    if args.gather_probe:
        return gather_probe(args)
    if args.stream_probe:
        return stream_probe(args)
    if args.mfma_probe:
        return mfma_probe(args)
    blocks = args.hysparse_blocks
    indexer = args.indexer

    import torch
    import token_level_top_amd as hs2
    from hs2_inputs import make_gates, make_indexer_inputs, make_inputs, workload

    wl = workload(args.config)
    if (blocks or indexer or args.window_sharing) and wl.decode:
        print("--hysparse-blocks, --indexer and --window-sharing apply to the prefill workloads (1, 2, 4)",
              file=sys.stderr)
        return 2
    if args.window_sharing and (blocks or indexer or wl.kv_dtype == "f32"):
        print("--window-sharing applies to the token-level path with a bf16 or FP8 cache (workloads 2, 4)",
              file=sys.stderr)
        return 2
    log(f"workload {wl.name}: generating inputs on the host")
    t0 = time.perf_counter()
    x = make_inputs(wl)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; copying to the GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = lambda t: None if t is None else t.to(dev, non_blocking=False).contiguous()
    k, v, ks, vs = g(x.k), g(x.v), g(x.k_scale), g(x.v_scale)
    kvdt = {"f32": hs2.HS2_F32, "bf16": hs2.HS2_BF16, "fp8": hs2.HS2_FP8_E4M3}[wl.kv_dtype]
    S = wl.window + wl.k_global

    hf = args.full_heads or wl.H
    if args.full_heads and (blocks or indexer):
        print("--full-heads combines with the token-level path only", file=sys.stderr)
        return 2
    if wl.decode and args.full_heads:
        qf = g(x.q[:, 0, :hf])
        qs = g(x.q_sparse)                                   # [L][B][1][H][d]
        ws = torch.empty(hs2.workspace_size(hs2.OP_DECODE_STEP, wl.B, 1, wl.n_ctx, hf, wl.d, wl.window,
                                            wl.k_global, kvdt), dtype=torch.uint8, device=dev)
        nws = hs2.workspace_size(hs2.OP_SPARSE_ATTN, wl.B, 1, wl.n_ctx, wl.H, wl.d, S, 0, kvdt)
        ws_sp = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        bufs = dict(out_full=torch.empty_like(qf), lse_full=torch.empty((wl.B, hf), device=dev),
                    indices=torch.empty((wl.B, S), dtype=torch.int32, device=dev))
        idx3 = bufs["indices"].view(wl.B, 1, S)
        out_s = torch.empty_like(qs)
        lse_s = torch.empty((wl.n_sparse, wl.B, 1, wl.H), device=dev)

        def step():
            hs2.decode_step(qf, None, k, v, ks, vs, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale,
                            workspace=ws, **bufs)
            hs2.sparse_attn(qs, k, v, ks, vs, indices=idx3, sm_scale=x.sm_scale, out=out_s, lse=lse_s,
                            workspace=ws_sp)
    elif wl.decode:
        qf = g(x.q[:, 0])
        qs = g(x.q_sparse[:, :, 0])
        ws = torch.empty(hs2.workspace_size(hs2.OP_DECODE_STEP, wl.B, 1, wl.n_ctx, wl.H, wl.d, wl.window,
                                            wl.k_global, kvdt), dtype=torch.uint8, device=dev)
        bufs = dict(out_full=torch.empty_like(qf), lse_full=torch.empty((wl.B, wl.H), device=dev),
                    out_sparse=torch.empty_like(qs), lse_sparse=torch.empty((wl.n_sparse, wl.B, wl.H), device=dev),
                    indices=torch.empty((wl.B, S), dtype=torch.int32, device=dev))

        def step():
            hs2.decode_step(qf, qs, k, v, ks, vs, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale,
                            workspace=ws, **bufs)
    elif indexer:
        HI, DI = args.indexer_heads, args.indexer_dim
        xi = make_indexer_inputs(2026, wl.B, wl.n_q, wl.q_pos0, wl.n_ctx, HI, DI, n_needles=16)
        qi, qsc, qw, ki, ksc = (g(t) for t in (xi.qi, xi.qs, xi.w, xi.ki, xi.ks))
        ws_i = torch.empty(hs2.workspace_size(hs2.OP_INDEX_SELECT, wl.B, wl.n_q, wl.n_ctx, 0, DI, 0, 0, 0),
                           dtype=torch.uint8, device=dev)
        qs_all = g(torch.cat([x.q.unsqueeze(0), x.q_sparse], 0))    # the F layer's queries, then the S layers'
        nws = hs2.workspace_size(hs2.OP_SPARSE_ATTN, wl.B, wl.n_q, wl.n_ctx, wl.H, wl.d, S, 0, kvdt)
        ws_sp = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        idx = torch.empty((wl.B, wl.n_q, S), dtype=torch.int32, device=dev)
        out_s = torch.empty_like(qs_all)

        def step():
            hs2.index_select(qi, qsc, qw, ki, ksc, q_pos0=wl.q_pos0, window=wl.window, k_global=wl.k_global,
                             indices=idx, workspace=ws_i)
            hs2.sparse_attn(qs_all, k, v, ks, vs, indices=idx, sm_scale=x.sm_scale, out=out_s, want_lse=False,
                            workspace=ws_sp)
    elif blocks:
        KB = wl.k_global // hs2.BLOCK
        q = g(x.q)
        qs = g(x.q_sparse)
        ws_full = torch.empty(hs2.workspace_size(hs2.OP_BLOCK_ATTN_SELECT, wl.B, wl.n_q, wl.n_ctx, wl.H, wl.d, 0, 0,
                                                 kvdt), dtype=torch.uint8, device=dev)
        ws_sp = torch.empty(hs2.workspace_size(hs2.OP_BLOCK_SPARSE_ATTN, wl.B, wl.n_q, wl.n_ctx, wl.H, wl.d,
                                               wl.window, KB, hs2._QDT[q.dtype]), dtype=torch.uint8, device=dev)
        gates = g(make_gates(7, (wl.n_sparse, wl.B, wl.n_q, wl.H, 2)))
        out = torch.empty_like(q)
        lse = torch.empty((wl.B, wl.n_q, wl.H), device=dev)
        bidx = torch.empty((wl.B, wl.n_q, KB), dtype=torch.int32, device=dev)
        out_s = torch.empty_like(qs)

        def step():
            hs2.block_attn_select(q, k, v, ks, vs, q_pos0=wl.q_pos0, k_blocks=KB, sm_scale=x.sm_scale, out=out,
                                  lse=lse, block_idx=bidx, want_scores=False, workspace=ws_full)
            hs2.block_sparse_attn(qs, k, v, ks, vs, block_idx=bidx, q_pos0=wl.q_pos0, window=wl.window, gates=gates,
                                  sm_scale=x.sm_scale, out=out_s, workspace=ws_sp)
    else:
        q = g(x.q[:, :, :hf])
        qs = g(x.q_sparse)
        ws_full = torch.empty(hs2.workspace_size(hs2.OP_FULL_ATTN_SELECT, wl.B, wl.n_q, wl.n_ctx, hf, wl.d,
                                                 wl.window, wl.k_global, kvdt), dtype=torch.uint8, device=dev)
        if args.window_sharing:
            nws = hs2.workspace_size(hs2.OP_SPARSE_ATTN_WINDOW, wl.B, wl.n_q, wl.n_ctx, wl.H, wl.d, wl.window,
                                     wl.k_global, kvdt)
        else:
            nws = hs2.workspace_size(hs2.OP_SPARSE_ATTN, wl.B, wl.n_q, wl.n_ctx, wl.H, wl.d, S, 0, kvdt)
        ws_sp = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((wl.B, wl.n_q, hf), device=dev)
        idx = torch.empty((wl.B, wl.n_q, S), dtype=torch.int32, device=dev)
        out_s = torch.empty_like(qs)
        lse_s = torch.empty((wl.n_sparse, wl.B, wl.n_q, wl.H), device=dev)

        def step():
            hs2.full_attn_select(q, k, v, ks, vs, q_pos0=wl.q_pos0, window=wl.window, k_global=wl.k_global,
                                 sm_scale=x.sm_scale, out=out, lse=lse, indices=idx, workspace=ws_full)
            if args.window_sharing:
                hs2.sparse_attn_window(qs, k, v, ks, vs, indices=idx, q_pos0=wl.q_pos0, window=wl.window,
                                       sm_scale=x.sm_scale, out=out_s, lse=lse_s, workspace=ws_sp)
            else:
                hs2.sparse_attn(qs, k, v, ks, vs, indices=idx, sm_scale=x.sm_scale, out=out_s, lse=lse_s,
                                workspace=ws_sp)

    copy_calibration(args.copy_calibration_mib, dev)

    L = hs2.lib()
    import ctypes
    L.hs2_timing_enable.argtypes = [ctypes.c_uint32]
    L.hs2_timing_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def read_timing():
        ms = (ctypes.c_double * 16)()
        n = (ctypes.c_int64 * 16)()
        rc = L.hs2_timing_read(ctypes.addressof(ms), ctypes.addressof(n))
        if rc != 0:
            raise RuntimeError("hs2_timing_read failed")
        return list(ms), list(n)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    read_timing()

    dom, bound, units, unit = dominant(wl.with_(H=hf))
    if indexer:  # the indexer pass: 2 * HI * dI flops per candidate pair, on the bf16 matrix cores
        cand = sum(max(0, wl.q_pos0 + i - wl.window + 1) for i in range(wl.n_q)) * wl.B
        dom, bound, units, unit = "score_stream", "mfma", 2 * args.indexer_heads * args.indexer_dim * cand, "TFLOP/s"
    L.hs2_timing_enable(1 << KC[dom])
    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    L.hs2_timing_enable(0)
    ms_total = e0.elapsed_time(e1)
    ms, n = read_timing()
    ms_eager = ms_total / args.steps
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        log(f"timing {args.steps} graph replays")
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    tokens = wl.B * wl.n_q
    value = tokens * args.steps / (ms_total / 1e3)
    kavg_s = ms[KC[dom]] / max(n[KC[dom]], 1) / 1e3
    if bound == "hbm":
        achieved, peak = units / kavg_s / 1e9, HBM_PEAK_GBS
    else:
        achieved = units / kavg_s / 1e12
        peak = MFMA_PEAK_TFLOPS["f32" if wl.q_dtype == "f32" else "bf16"]
    wname = (wl.name + ("_hysparse_blocks" if blocks else "") + ("_indexer" if indexer else "")
             + (f"_full_heads{hf}" if args.full_heads else "")
             + ("_window_sharing" if args.window_sharing and not wl.decode else ""))
    tr = traffic_record(dom, wname)
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": tr["bytes_per_launch"] if tr else None,
            "kernel": dom, "kernel_ms": round(kavg_s * 1e3, 4),
            "algorithmic_per_launch": units}
    t_roof = path_roofline_seconds(wl, blocks, args.full_heads)
    if indexer:
        peak_b = MFMA_PEAK_TFLOPS["bf16"] * 1e12
        sel = sum(min(wl.q_pos0 + i + 1, S) for i in range(wl.n_q)) * wl.B
        t_roof = units / peak_b + (1 + wl.n_sparse) * 4 * wl.d * wl.H * sel / peak_b
    metric = METRIC
    if blocks:
        metric = ("query tok/s, HySparse v1 block variant: full attn + 64-token block top-16 + gated 128-token "
                  "window branch")
    if indexer:
        metric = (f"query tok/s, light-indexer selection ({args.indexer_heads} FP8 heads x {args.indexer_dim}) + "
                  "IndexCache F + S x n_sparse sparse layers")
    res = {"metric": metric, "value": round(value, 2), "unit": "query tok/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32" if wl.q_dtype == "f32" else "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V with planted needles)",
           "config": {"workload": wname, "B": wl.B, "H_full": hf, "n_q": wl.n_q, "q_pos0": wl.q_pos0, "n_ctx": wl.n_ctx,
                      "H": wl.H, "d": wl.d, "kv_storage": wl.kv_dtype, "window": wl.window,
                      "k_global": wl.k_global, "n_sparse": wl.n_sparse},
           "roofline": roof,
           "path_roofline": {"t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof * 1e3 / ms_step, 4)},
           "launch": "hip_graph" if args.graph else "eager", "device": device_name()}
    if args.graph:
        res["eager_ms_per_step"] = round(ms_eager, 4)
    if args.breakdown:
        L.hs2_timing_enable(0xFFFF if blocks else 0xFFF | 1 << KC["decode_rescore"])
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        L.hs2_timing_enable(0)
        ms, n = read_timing()
        names = {v_: k_ for k_, v_ in KC.items()}
        res["breakdown_ms_per_step"] = {names[c]: round(ms[c] / 3, 4) for c in range(16) if n[c]}
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds, blocks, xi if indexer else None)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
