"""GPU parity at the five workloads' full sizes, through the same C-ABI calls
and shapes the benchmark times. The oracle checks sampled rows: every
sequence of the decode workloads, all rows of the tiny prefill, 512 seeded
rows (all needle rows + uniform rows) of the 32k prefill and 512 seeded rows
(the 32 cluster-target rows + 480 uniform rows) of the 256k chunked prefill.
Needle recovery runs at every workload's full shape."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import checked_rows, make_inputs, workload
from tests.hs2_check import check_index_rows, decode_scores_close, lse_close, rows_close, to_np

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


def say(*a):
    print("[gpu-full]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import token_level_top_amd as t
    t.lib()
    return t


def g(t):
    return None if t is None else t.cuda().contiguous()


def oracle_rows(orc, x, wl, rows, chunk=64):
    """The oracle's full layer on `rows`, in chunks (a progress line each)."""
    parts = []
    for c0 in range(0, len(rows), chunk):
        part = rows[c0:c0 + chunk]
        parts.append(orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global,
                                     x.sm_scale, part, want_scores=True))
        say(f"  oracle rows {c0 + len(part)} of {len(rows)}")
    return {k: np.concatenate([p[k] for p in parts]) for k in ("out", "lse", "idx", "kth", "scores")}


@pytest.mark.parametrize("cfg", [3, 5])
def test_decode_full_size(hs2, orc, cfg):
    wl = workload(cfg)
    say("generate", wl.name)
    x = make_inputs(wl)
    say("decode step on the GPU")
    r = hs2.decode_step(g(x.q[:, 0]), g(x.q_sparse[:, :, 0]), g(x.k), g(x.v), g(x.k_scale), g(x.v_scale),
                        window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale, want_scores=True)
    torch.cuda.synchronize()
    rows = list(range(wl.B))
    say("oracle on", len(rows), "sequences")
    ref = oracle_rows(orc, x, wl, rows, chunk=16)
    tol = RTOL[wl.kv_dtype]
    rows_close(r["out_full"], ref["out"], tol, "decode out")
    lse_close(r["lse_full"], ref["lse"], tol, "decode lse")
    decode_scores_close(r["scores"], ref["scores"], wl.kv_dtype)
    check_index_rows(r["indices"], ref["idx"], ref["scores"], ref["kth"], wl.window)
    gidx = to_np(r["indices"]).astype(np.int32)
    for l in range(wl.n_sparse):
        s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, x.sm_scale, rows)
        rows_close(r["out_sparse"][l], s["out"], tol, f"decode sparse layer {l} out")
        lse_close(r["lse_sparse"][l], s["lse"], tol, f"decode sparse layer {l} lse")
    # the step as timed (no score vector: 8-bit logit codes, bounds, exact
    # rescoring of the candidates), against the same oracle rows
    say("decode step without the score vector")
    r8 = hs2.decode_step(g(x.q[:, 0]), g(x.q_sparse[:, :, 0]), g(x.k), g(x.v), g(x.k_scale), g(x.v_scale),
                         window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(r8["out_full"], r["out_full"]) and torch.equal(r8["lse_full"], r["lse_full"])
    ov, mn, sw = check_index_rows(r8["indices"], ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  8-bit codes: overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    same = to_np(r8["indices"]) == gidx
    if not same.all():
        gidx8 = to_np(r8["indices"]).astype(np.int32)
        for l in range(wl.n_sparse):
            s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx8, x.sm_scale, rows)
            rows_close(r8["out_sparse"][l], s["out"], tol, f"decode (8-bit codes) sparse layer {l} out")
    else:
        for l in range(wl.n_sparse):
            assert torch.equal(r8["out_sparse"][l], r["out_sparse"][l])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_uniform,n_target", [(1, 2048, None), (2, 256, None), (4, 480, 32)])
def test_prefill_full_size(hs2, orc, cfg, n_uniform, n_target):
    wl = workload(cfg)
    say("generate", wl.name)
    x = make_inputs(wl)
    needles = x.needles if n_target is None else x.needles[:n_target]
    rows = checked_rows(wl, needles, n_uniform)
    say("prefill on the GPU;", len(rows), "rows checked")
    kw = dict(q_pos0=wl.q_pos0, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale)
    out, lse, idx = hs2.full_attn_select(g(x.q), g(x.k), g(x.v), g(x.k_scale), g(x.v_scale), **kw)
    so, sl = hs2.sparse_attn(g(x.q_sparse), g(x.k), g(x.v), g(x.k_scale), g(x.v_scale), indices=idx,
                             sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    ref = oracle_rows(orc, x, wl, rows)
    tol = RTOL[wl.kv_dtype]
    ri = torch.tensor(rows)
    rows_close(out[0, ri], ref["out"], tol, "prefill out")
    lse_close(lse[0, ri], ref["lse"], tol, "prefill lse")
    check_index_rows(idx[0, ri], ref["idx"], ref["scores"], ref["kth"], wl.window)
    gidx = to_np(idx[0, ri]).astype(np.int32)
    for l in range(wl.n_sparse):
        s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, x.sm_scale, rows)
        rows_close(so[l, 0, ri], s["out"], tol, f"prefill sparse layer {l} out")
        lse_close(sl[l, 0, ri], s["lse"], tol, f"prefill sparse layer {l} lse")
    # every index row of the whole launch is well formed (window, order, causality)
    full = to_np(idx[0]).astype(np.int64)
    p = wl.q_pos0 + np.arange(wl.n_q)
    win = full[:, :wl.window]
    nw = np.minimum(wl.window, p + 1)
    expect_win = np.where(np.arange(wl.window)[None, :] < nw[:, None],
                          p[:, None] - nw[:, None] + 1 + np.arange(wl.window)[None, :], -1)
    assert np.array_equal(win, expect_win)
    glb = full[:, wl.window:]
    valid = glb >= 0
    n_cand = np.maximum(0, p - wl.window + 1)
    assert np.array_equal(valid.sum(axis=1), np.minimum(wl.k_global, n_cand))
    has = valid.any(axis=1)
    assert (np.where(valid, glb, -1).max(axis=1)[has] <= (p - wl.window)[has]).all()
    d = np.diff(np.where(valid, glb, np.iinfo(np.int64).max), axis=1)
    assert (d[valid[:, 1:]] > 0).all()
    say(f"  all {wl.n_q} index rows well formed")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_needle_recovery(hs2, cfg):
    """Planted needles are recovered by the GPU's selection at every
    workload's full shape: the literal 3*q/|q| needles at the tiny workload,
    needles three times a typical key norm elsewhere -- 256 rows of the 32k
    prefill (one needle each; a 512-row tail of queries), 32 per sequence of
    the 128k decode, 32 clusters of 8 identical FP8 keys in the 256k chunked
    prefill (every key of a cluster ties with the others), 64 per sequence by
    depth in the 1M FP8 decode."""
    wl = workload(cfg)
    if cfg == 2:
        wl = wl.with_(n_q=512, q_pos0=32768 - 512)
    norm = "R18a" if cfg == 1 else "R18b"
    x = make_inputs(wl, needle_norm=norm)
    say("needles", wl.name, norm, len(x.needles))
    kv = (g(x.k), g(x.v), g(x.k_scale), g(x.v_scale))
    if wl.decode:
        r = hs2.decode_step(g(x.q[:, 0]), g(x.q_sparse[:, :, 0]), *kv, window=wl.window, k_global=wl.k_global,
                            sm_scale=x.sm_scale)
        idx = to_np(r["indices"])[:, None, :]
    else:
        _, _, ii = hs2.full_attn_select(g(x.q), *kv, q_pos0=wl.q_pos0, window=wl.window, k_global=wl.k_global,
                                        sm_scale=x.sm_scale)
        idx = to_np(ii)
    torch.cuda.synchronize()
    keys = sum(n.length for n in x.needles)
    hit = sum(all((n.j + t) in idx[n.b, n.i, wl.window:] for t in range(n.length)) for n in x.needles)
    say(f"  {hit} of {len(x.needles)} needles ({keys} planted keys) recovered")
    assert hit == len(x.needles), f"{hit} of {len(x.needles)} needles recovered"
