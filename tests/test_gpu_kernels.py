"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and end in ragged tails.

Every call goes through the C ABI (libhs2.so via the ctypes binding)."""
import math
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_inputs, workload
from tests.hs2_check import check_index_rows, decode_scores_close, lse_close, rows_close, to_np

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import token_level_top_amd as t
    t.lib()
    return t


def dev(x):
    return None if x is None else x.cuda()


# ------------------------------------------------------------------ select

def test_select_topk_bit_exact(hs2, orc):
    rng = np.random.default_rng(1)
    rows, L, k = 12, 20000, 1024
    s = rng.random((rows, L), dtype=np.float32)
    s[1] = 0.5                                        # all tied: overflows the candidate buffer
    s[2, ::3] = np.float32(0.999)                     # thousands tied above the threshold
    s[3] = rng.standard_exponential(L).astype(np.float32) ** 4
    s[4] = 0.0
    s[5, :] = np.float32(1e-38) * rng.random(L, dtype=np.float32)   # subnormals
    s[6] = np.float32(-0.0)
    n_cand = np.array([L, L, L, L, L, L, L, 0, 1, 1023, 1024, 1025], np.int32)
    say("select_topk rows", rows, "len", L, "k", k)
    got = hs2.select_topk(torch.from_numpy(s).cuda(), k, torch.from_numpy(n_cand).cuda())
    torch.cuda.synchronize()
    ref = orc.select_scores_f32(s, n_cand.astype(np.int64), k)
    assert np.array_equal(to_np(got), ref)


def test_select_topk_bin_ranking_paths(hs2, orc):
    """The final step's branches: keys of the threshold bin ranked directly
    (random rows), more than 512 keys in that bin without overflowing the
    candidate list (digit search; 1500 exact ties straddle the k-th), every
    candidate kept (700 equal scores, n_cand = 700), rows not 16-byte aligned
    (odd row length: scalar loads), and a row of more than 1024 chunks of 8192
    (positions sorted instead of placed by runs)."""
    rng = np.random.default_rng(11)
    rows, L, k = 4, 20001, 1024
    s = (rng.random((rows, L), dtype=np.float32) * 0.5).astype(np.float32)
    hi = rng.choice(L, 2000, replace=False)
    s[0, hi[:500]] = 0.9 + 0.09 * rng.random(500, dtype=np.float32)
    s[0, hi[500:]] = np.float32(0.75)
    s[1, :] = np.float32(0.3)
    s[3] = rng.standard_exponential(L).astype(np.float32)
    n_cand = np.array([L, 700, L, L - 3], np.int32)
    say("select_topk bin paths", rows, L, k)
    got = hs2.select_topk(torch.from_numpy(s).cuda(), k, torch.from_numpy(n_cand).cuda())
    torch.cuda.synchronize()
    ref = orc.select_scores_f32(s, n_cand.astype(np.int64), k)
    assert np.array_equal(to_np(got), ref)
    Lx = 8192 * 1025 + 1
    sx = rng.random((1, Lx), dtype=np.float32)
    say("select_topk long row", Lx)
    got = hs2.select_topk(torch.from_numpy(sx).cuda(), k)
    torch.cuda.synchronize()
    ref = orc.select_scores_f32(sx, [Lx], k)
    assert np.array_equal(to_np(got), ref)


@pytest.mark.parametrize("L,k", [(131072, 1024), (300, 256), (9000, 2048), (70000, 1), (9001, 1024)])
def test_select_topk_shapes(hs2, orc, L, k):
    rng = np.random.default_rng(L + k)
    rows = 5
    s = (rng.standard_normal((rows, L)).astype(np.float32) ** 2)
    s[0, 100:200] = s[0, 50]                          # exact ties
    say("select_topk", rows, L, k)
    got = hs2.select_topk(torch.from_numpy(s).cuda(), k)
    torch.cuda.synchronize()
    ref = orc.select_scores_f32(s, [L] * rows, k)
    assert np.array_equal(to_np(got), ref)


# ------------------------------------------------------------------ sparse

def _rand_index_rows(rng, n_tok, n_sel, n_ctx, fill):
    idx = np.full((n_tok, n_sel), -1, np.int32)
    for t in range(n_tok):
        m = int(fill if fill else rng.integers(0, n_sel + 1))
        m = min(m, n_ctx)
        idx[t, :m] = np.sort(rng.choice(n_ctx, size=m, replace=False))
    return idx


@pytest.mark.parametrize("cfg,n_q,n_ctx,n_sel,fill", [
    (1, 7, 3000, 384, 0),          # f32, H=4, d=64, split path, random fill incl. empty rows
    (2, 5, 4100, 1152, 1152),      # bf16, H=16, d=128, split path
    (4, 6, 5000, 1152, 0),         # fp8 KV, split path
    (2, 1100, 2000, 200, 0),       # bf16, one workgroup per token (no split)
    (2, 1030, 6000, 2300, 0),      # bf16, no split, index rows longer than one LDS index chunk
    (2, 40, 9000, 4096, 0),        # bf16, split path, the longest index rows
    (4, 3, 3000, 2300, 2300),      # FP8, 18 splits per token
    (4, 1023, 5000, 1152, 0),      # FP8, one workgroup per token (no split)
])
def test_sparse_matches_oracle(hs2, orc, cfg, n_q, n_ctx, n_sel, fill):
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=n_ctx - n_q, n_ctx=n_ctx, n_needles=0, needles="none",
                             n_sparse=2)
    x = make_inputs(wl)
    rng = np.random.default_rng(n_q * 7 + n_sel)
    idx = _rand_index_rows(rng, n_q, n_sel, n_ctx, fill)
    say("sparse", wl.name, n_q, n_ctx, n_sel)
    out, lse = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                               indices=torch.from_numpy(idx).reshape(1, n_q, n_sel).cuda(), sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(n_q))
    for l in range(2):
        r = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, idx, x.sm_scale, rows)
        empty = (idx < 0).all(axis=1)
        rows_close(out[l, 0][~torch.from_numpy(empty)], r["out"][~empty], RTOL[wl.kv_dtype], "sparse out")
        assert (to_np(out[l, 0])[empty] == 0).all()
        lse_close(lse[l, 0], r["lse"], RTOL[wl.kv_dtype])


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("cfg,B,n_ctx,n_sparse", [
    (3, 3, 5003, 2),        # bf16
    (5, 2, 9000, 2),        # fp8
    (1, 2, 4099, 1),        # f32, H=4, d=64, K=256
    (3, 2, 100, 1),         # shorter than the window: no candidates
    (3, 2, 700, 1),         # fewer candidates than k_global
    (3, 2, 3000, 9),        # nine sparse layers, one launch and combine each
])
@pytest.mark.parametrize("want_scores", [True, False])
def test_decode_step_matches_oracle(hs2, orc, cfg, B, n_ctx, n_sparse, want_scores):
    """want_scores: the score vector is returned (bf16 / FP8: 16-bit logit
    codes); without it the step runs as timed (8-bit codes, score bounds and
    exact rescoring of the candidates)."""
    wl = workload(cfg).with_(B=B, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=n_sparse, needles="decode",
                             n_needles=8 if n_ctx > 2000 else 0, decode=True)
    x = make_inputs(wl)
    say("decode", wl.name, B, n_ctx, "with" if want_scores else "without", "the score vector")
    r = hs2.decode_step(dev(x.q[:, 0]).contiguous(), dev(x.q_sparse[:, :, 0]).contiguous(), dev(x.k), dev(x.v),
                        dev(x.k_scale), dev(x.v_scale), window=wl.window, k_global=wl.k_global,
                        sm_scale=x.sm_scale, want_scores=want_scores)
    torch.cuda.synchronize()
    rows = list(range(B))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global, x.sm_scale,
                          rows, want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(r["out_full"], ref["out"], tol, "decode out")
    lse_close(r["lse_full"], ref["lse"], tol)
    # token scores: fp32 logits (fp32 cache) or the 16-bit logit codes
    if want_scores:
        decode_scores_close(r["scores"], ref["scores"], wl.kv_dtype)
    ov, mn, sw = check_index_rows(r["indices"], ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    # sparse layers, judged on the GPU's own index set
    gidx = to_np(r["indices"]).astype(np.int32)
    for l in range(n_sparse):
        s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, x.sm_scale, rows)
        rows_close(r["out_sparse"][l], s["out"], tol, "decode sparse out")
        lse_close(r["lse_sparse"][l], s["lse"], tol)


@pytest.mark.parametrize("want_scores", [True, False])
@pytest.mark.parametrize("B,n_ctx", [(2, 5003), (1, 20000)])
def test_decode_peaked_attention_logit_codes_clamp(hs2, orc, B, n_ctx, want_scores):
    """Softmax scale 12/sqrt(d) on N(0,1) bf16 inputs: base-2 logits with a
    spread of about 17, so a 32-key block of one head spans more than 64 in the
    exponent and the decode kernel's 16-bit logit codes clamp. The score vector
    stays within its bound (relative 4e-4, clamped terms below 2^-64 of the
    block maximum) and the index rows within the swap rule, although the
    K-th score is many orders of magnitude below the largest."""
    wl = workload(3).with_(B=B, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=1, needles="decode",
                           n_needles=8, decode=True)
    x = make_inputs(wl)
    sm = 12.0 / math.sqrt(wl.d)
    # the case must clamp: some (block, head) spans more than 64 base-2 units
    qf = x.q[:, 0].to(torch.float64)                      # [B][H][d]
    kf = x.k.to(torch.float64)                            # [B][n_ctx][d]
    lg = torch.einsum("bhd,bjd->bjh", qf, kf) * (sm * math.log2(math.e))
    nb = n_ctx // 32
    blk = lg[:, :nb * 32].reshape(B, nb, 32, wl.H)
    span = (blk.max(dim=2).values - blk.min(dim=2).values).max().item()
    say(f"peaked decode B={B} n_ctx={n_ctx}: widest block span {span:.1f} (codes clamp beyond 64)")
    assert span > 64.0, span
    r = hs2.decode_step(dev(x.q[:, 0]).contiguous(), dev(x.q_sparse[:, :, 0]).contiguous(), dev(x.k), dev(x.v),
                        dev(x.k_scale), dev(x.v_scale), window=wl.window, k_global=wl.k_global,
                        sm_scale=sm, want_scores=want_scores)
    torch.cuda.synchronize()
    rows = list(range(B))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global, sm,
                          rows, want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(r["out_full"], ref["out"], tol, "peaked decode out")
    lse_close(r["lse_full"], ref["lse"], tol)
    if want_scores:
        decode_scores_close(r["scores"], ref["scores"], wl.kv_dtype, "peaked score vector")
    sc = np.asarray(ref["scores"], dtype=np.float64)
    say(f"  K-th score / largest score: {float((np.asarray(ref['kth']) / sc.max(axis=1)).min()):.3e}")
    ov, mn, sw = check_index_rows(r["indices"], ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    gidx = to_np(r["indices"]).astype(np.int32)
    s = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, sm, rows)
    rows_close(r["out_sparse"][0], s["out"], tol, "peaked decode sparse out")
    lse_close(r["lse_sparse"][0], s["lse"], tol)


# ----------------------------------------------------------------- prefill

@pytest.mark.parametrize("cfg,n_q,q_pos0,n_ctx,kg", [
    (1, 700, 0, 700, 256),           # f32, H=4, d=64
    (2, 1000, 0, 1000, 300),         # bf16, H=16, d=128
    (4, 77, 3000, 3077, 1024),       # fp8 KV, chunk at an offset, ragged block
    (2, 130, 0, 130, 1024),          # shorter than window + k
    (2, 48, 9952, 10000, 1024),      # > 4096 candidates per token: compaction while streaming
    (4, 40, 12000, 12040, 1024),     # fp8 with clustered (tied) needles, streaming compaction
    (1, 96, 5000, 5096, 256),        # f32, H=4: 8 tokens per wave, streaming compaction
    (2, 300, 500, 800, 0),           # window only (k_global = 0)
])
def test_full_attn_select_matches_oracle(hs2, orc, cfg, n_q, q_pos0, n_ctx, kg):
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, k_global=kg, n_needles=4 if kg else 0)
    x = make_inputs(wl)
    say("prefill", wl.name, n_q, q_pos0, n_ctx)
    out, lse, idx = hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                         q_pos0=q_pos0, window=wl.window, k_global=kg, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(n_q))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, q_pos0, wl.window, kg, x.sm_scale, rows,
                          want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(out[0], ref["out"], tol, "prefill out")
    lse_close(lse[0], ref["lse"], tol)
    ov, mn, sw = check_index_rows(idx[0], ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")


def test_prefill_and_decode_are_deterministic(hs2):
    wl = workload(2).with_(n_q=300, n_ctx=1500, q_pos0=1200, n_needles=2)
    x = make_inputs(wl)
    say("determinism")
    a = hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), q_pos0=1200, window=128, k_global=1024,
                             sm_scale=x.sm_scale)
    b = hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), q_pos0=1200, window=128, k_global=1024,
                             sm_scale=x.sm_scale)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # decode over 7 selection chunks per row: the chunks' candidate runs land in
    # whatever order their atomics resolve, the results may not depend on it
    wd = workload(3).with_(B=4, n_ctx=50000, q_pos0=49999, n_needles=4, n_sparse=2)
    xd = make_inputs(wd)
    say("determinism decode", wd.name, wd.B, wd.n_ctx)
    for ws in (True, False):
        runs = [hs2.decode_step(dev(xd.q[:, 0]), dev(xd.q_sparse[:, :, 0]), dev(xd.k), dev(xd.v), window=128,
                                k_global=1024, sm_scale=xd.sm_scale, want_scores=ws) for _ in range(3)]
        torch.cuda.synchronize()
        for r in runs[1:]:
            for key in ("indices", "scores", "out_full", "lse_full", "out_sparse", "lse_sparse"):
                if key == "scores" and not ws:
                    continue
                assert torch.equal(r[key], runs[0][key]), key


@pytest.mark.parametrize("cfg", [2, 4])
def test_results_do_not_depend_on_workspace_contents(hs2, cfg):
    """Workspace bytes left by earlier calls never reach the results: a prefill
    and a decode step give bit-identical outputs with the workspace zeroed and
    with every byte 0xFF (an unwritten candidate slot would then read as the
    largest key), three calls each."""
    wl = workload(cfg).with_(B=1, n_q=64, q_pos0=6000, n_ctx=6064, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    kv = (dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale))
    B, n_q, H, d = x.q.shape
    kvdt = hs2._KVDT[x.k.dtype]
    say("workspace contents", wl.name)
    n = hs2.workspace_size(hs2.OP_FULL_ATTN_SELECT, B, n_q, wl.n_ctx, H, d, 128, 1024, kvdt)
    runs = []
    for fill in (0, 255, 255, 0, 255):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        r = hs2.full_attn_select(dev(x.q), *kv, q_pos0=wl.q_pos0, window=128, k_global=1024, sm_scale=x.sm_scale,
                                 workspace=ws)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in r])
    for r in runs[1:]:
        for u, v in zip(runs[0], r):
            assert torch.equal(u, v)
    qf, qs = dev(x.q[:, -1]).contiguous(), dev(x.q_sparse[:, :, -1]).contiguous()
    n = hs2.workspace_size(hs2.OP_DECODE_STEP, B, 1, wl.n_ctx, H, d, 128, 1024, kvdt)
    runs = []
    for fill in (0, 255, 255):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        r = hs2.decode_step(qf, qs, *kv, window=128, k_global=1024, sm_scale=x.sm_scale, want_scores=True,
                            workspace=ws)
        torch.cuda.synchronize()
        runs.append({k: v.clone() for k, v in r.items() if v is not None})
    for r in runs[1:]:
        for k in runs[0]:
            assert torch.equal(runs[0][k], r[k]), k


def test_prefill_all_tied_scores(hs2, orc):
    """Zero queries give every key the same score: the lowest positions win."""
    wl = workload(2).with_(n_q=64, q_pos0=6000, n_ctx=6064, n_needles=0, needles="none")
    x = make_inputs(wl)
    x.q[0, ::3] = 0
    say("prefill all tied")
    out, lse, idx = hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), q_pos0=wl.q_pos0, window=128,
                                         k_global=1024, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    g = to_np(idx[0])
    for i in range(0, 64, 3):
        assert g[i, 128:].tolist() == list(range(1024))
    rows = list(range(64))
    ref = orc.full_select(x.q, x.k, x.v, None, None, wl.q_pos0, 128, 1024, x.sm_scale, rows, want_scores=True)
    check_index_rows(idx[0], ref["idx"], ref["scores"], ref["kth"], 128)
    rows_close(out[0], ref["out"], 1e-2)


@pytest.mark.parametrize("cfg", [3, 5])
@pytest.mark.parametrize("want_scores", [True, False])
def test_decode_all_tied_scores(hs2, orc, cfg, want_scores):
    """A zero query gives every key of its sequence the same score, so every
    candidate ties: the lowest positions win. Without the score vector the
    collect step then keeps more candidates than its list holds, and the
    overflow path runs (exact scores for the whole row, whole-row selection);
    the other sequence takes the ordinary path in the same launch."""
    wl = workload(cfg).with_(B=2, n_q=1, q_pos0=8999, n_ctx=9000, n_sparse=1, needles="none", n_needles=0,
                             decode=True)
    x = make_inputs(wl)
    x.q[0] = 0
    say("decode all tied", wl.name, "with" if want_scores else "without", "the score vector")
    r = hs2.decode_step(dev(x.q[:, 0]).contiguous(), dev(x.q_sparse[:, :, 0]).contiguous(), dev(x.k), dev(x.v),
                        dev(x.k_scale), dev(x.v_scale), window=128, k_global=1024, sm_scale=x.sm_scale,
                        want_scores=want_scores)
    torch.cuda.synchronize()
    g = to_np(r["indices"])
    assert g[0, 128:].tolist() == list(range(1024))
    assert g[0, :128].tolist() == list(range(9000 - 128, 9000))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, 128, 1024, x.sm_scale, [0, 1],
                          want_scores=True)
    ov, mn, sw = check_index_rows(r["indices"], ref["idx"], ref["scores"], ref["kth"], 128)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    rows_close(r["out_full"], ref["out"], RTOL[wl.kv_dtype], "tied decode out")


@pytest.mark.parametrize("cfg,B,H,d,n_q,q_pos0,n_ctx", [
    (2, 2, 16, 128, 200, 300, 500),     # two sequences in one launch
    (2, 1, 8, 64, 500, 4000, 4500),     # bf16, H=8, d=64 instantiations
    (4, 2, 4, 128, 160, 5000, 5160),    # fp8, H=4, two sequences
])
def test_prefill_batched_and_head_shapes(hs2, orc, cfg, B, H, d, n_q, q_pos0, n_ctx):
    wl = workload(cfg).with_(B=B, H=H, d=d, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=4, n_sparse=1)
    x = make_inputs(wl)
    say("prefill shapes", wl.name, B, H, d, n_q, q_pos0, n_ctx)
    kw = dict(q_pos0=q_pos0, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale)
    out, lse, idx = hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale), **kw)
    so, sl = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale), indices=idx,
                             sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(B * n_q))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, q_pos0, wl.window, wl.k_global, x.sm_scale, rows,
                          want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(out.reshape(B * n_q, H, d), ref["out"], tol, "prefill out")
    lse_close(lse.reshape(B * n_q, H), ref["lse"], tol)
    g = idx.reshape(B * n_q, -1)
    ov, mn, sw = check_index_rows(g, ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    s = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, to_np(g).astype(np.int32),
                   x.sm_scale, rows)
    rows_close(so[0].reshape(B * n_q, H, d), s["out"], tol, "prefill sparse out")
    lse_close(sl[0].reshape(B * n_q, H), s["lse"], tol)


@pytest.mark.parametrize("want_scores", [True, False])
@pytest.mark.parametrize("cfg,B,H,d,n_ctx", [
    (3, 3, 8, 64, 6000),     # bf16, H=8, d=64 instantiations of the split, score and rescore kernels
    (5, 2, 4, 128, 7001),    # FP8, H=4, ragged last block
    (3, 2, 16, 64, 4500),    # bf16, H=16, d=64
    (5, 2, 8, 128, 5100),    # FP8, H=8
])
def test_decode_head_shapes(hs2, orc, cfg, B, H, d, n_ctx, want_scores):
    """Every (H, d) form of the bf16 / FP8 decode step, with the score vector
    (16-bit logit codes) and without it (8-bit codes, bounds, exact rescoring)."""
    wl = workload(cfg).with_(B=B, H=H, d=d, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=1, needles="decode",
                             n_needles=4, decode=True)
    x = make_inputs(wl)
    say("decode shapes", wl.name, B, H, d, n_ctx, "with" if want_scores else "without", "the score vector")
    r = hs2.decode_step(dev(x.q[:, 0]).contiguous(), dev(x.q_sparse[:, :, 0]).contiguous(), dev(x.k), dev(x.v),
                        dev(x.k_scale), dev(x.v_scale), window=wl.window, k_global=wl.k_global,
                        sm_scale=x.sm_scale, want_scores=want_scores)
    torch.cuda.synchronize()
    rows = list(range(B))
    ref = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global, x.sm_scale,
                          rows, want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(r["out_full"], ref["out"], tol, "decode out")
    lse_close(r["lse_full"], ref["lse"], tol)
    if want_scores:
        decode_scores_close(r["scores"], ref["scores"], wl.kv_dtype)
    ov, mn, sw = check_index_rows(r["indices"], ref["idx"], ref["scores"], ref["kth"], wl.window)
    say(f"  overlap mean {ov:.4f} min {mn:.4f} swaps {sw}")
    gidx = to_np(r["indices"]).astype(np.int32)
    s = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, x.sm_scale, rows)
    rows_close(r["out_sparse"][0], s["out"], tol, "decode sparse out")
    lse_close(r["lse_sparse"][0], s["lse"], tol)


def test_sparse_attn_beyond_65535_tokens(hs2, orc):
    """More query tokens in one call than a grid's y dimension holds (65535):
    the sparse layer's 1-D grid covers them all; sampled rows against the
    oracle, including the last token."""
    n = 70000
    wl = workload(1).with_(B=1, n_q=n, q_pos0=0, n_ctx=n, n_needles=0, n_sparse=1)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 1, n, wl.H, wl.d, generator=g)
    k = torch.randn(1, n, wl.d, generator=g)
    v = torch.randn(1, n, wl.d, generator=g)
    idx = torch.randint(0, n, (1, n, 8), generator=g, dtype=torch.int32)
    idx[0, :, 7] = -1
    say("sparse attention over", n, "tokens")
    out, lse = hs2.sparse_attn(q.cuda(), k.cuda(), v.cuda(), indices=idx.cuda(), sm_scale=0.125)
    torch.cuda.synchronize()
    rows = [0, 65534, 65535, 65536, n - 1]
    ref = orc.sparse(q[0].contiguous(), k, v, None, None, idx[0, rows].numpy(), 0.125, rows)
    rows_close(out[0, 0, rows], ref["out"], RTOL["f32"], "sparse out")
    lse_close(lse[0, 0, rows], ref["lse"], RTOL["f32"])


@pytest.mark.parametrize("cfg,B,n_q,q_pos0,n_ctx,h_full", [
    (2, 1, 300, 700, 1000, 4),      # prefill: 4 full-layer heads, 16 sparse-layer heads
    (4, 1, 64, 3000, 3064, 8),      # FP8 cache, 8 full-layer heads
    (3, 4, 1, 9999, 10000, 4),      # decode: decode step without sparse layers, then 16-head sparse layers
])
def test_asymmetric_heads_compose(hs2, orc, cfg, B, n_q, q_pos0, n_ctx, h_full):
    """Fewer query heads in the full layer than in the sparse layers (the
    HySparse2 page's future-work direction): the index rows of an h_full-head
    full layer drive 16-head sparse layers."""
    wl = workload(cfg).with_(B=B, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    say("asymmetric heads", wl.name, B, n_q, q_pos0, n_ctx, h_full)
    qf = x.q[:, :, :h_full].contiguous()
    kv = (dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale))
    if wl.decode:
        r = hs2.decode_step(dev(qf[:, 0]), None, *kv, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale)
        idx = r["indices"].reshape(B, 1, -1)
        out_f = r["out_full"].reshape(B, 1, h_full, wl.d)
    else:
        out_f, _, idx = hs2.full_attn_select(dev(qf), *kv, q_pos0=q_pos0, window=wl.window, k_global=wl.k_global,
                                             sm_scale=x.sm_scale)
    so, sl = hs2.sparse_attn(dev(x.q_sparse), *kv, indices=idx, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(B * n_q))
    ref = orc.full_select(qf, x.k, x.v, x.k_scale, x.v_scale, q_pos0, wl.window, wl.k_global, x.sm_scale, rows,
                          want_scores=True)
    tol = RTOL[wl.kv_dtype]
    rows_close(out_f.reshape(B * n_q, h_full, wl.d), ref["out"], tol, "full out")
    g = idx.reshape(B * n_q, -1)
    check_index_rows(g, ref["idx"], ref["scores"], ref["kth"], wl.window)
    gi = to_np(g).astype(np.int32)
    for l in range(2):
        s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gi, x.sm_scale, rows)
        rows_close(so[l].reshape(B * n_q, wl.H, wl.d), s["out"], tol, f"sparse out {l}")
        lse_close(sl[l].reshape(B * n_q, wl.H), s["lse"], tol)


@pytest.mark.parametrize("cfg,n_q", [(2, 5), (4, 1100)])
def test_sparse_out_of_range_entries_are_skipped(hs2, orc, cfg, n_q):
    """Index entries outside [0, n_ctx) (past the end, or negative other than
    -1) are skipped like -1: the result equals the oracle on the same rows with
    those entries emptied, and the in-range neighbours are unaffected."""
    n_ctx, n_sel = 3000, 1152
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=n_ctx - n_q, n_ctx=n_ctx, n_needles=0, needles="none",
                             n_sparse=1)
    x = make_inputs(wl)
    rng = np.random.default_rng(11 + n_q)
    idx = _rand_index_rows(rng, n_q, n_sel, n_ctx, 0)
    bad = idx.copy()
    for t in range(n_q):
        slots = rng.choice(n_sel, size=8, replace=False)
        bad[t, slots] = rng.choice([n_ctx, n_ctx + 1, 2 ** 31 - 1, -2, -(2 ** 31), 10 * n_ctx], size=8)
    clean = np.where((bad >= 0) & (bad < n_ctx), bad, -1).astype(np.int32)
    say("sparse with out-of-range entries", wl.name, n_q)
    out, lse = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                               indices=torch.from_numpy(bad).reshape(1, n_q, n_sel).cuda(), sm_scale=x.sm_scale)
    ref_o, ref_l = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                   indices=torch.from_numpy(clean).reshape(1, n_q, n_sel).cuda(),
                                   sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    rows = list(range(n_q))
    r = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, clean, x.sm_scale, rows)
    empty = (clean < 0).all(axis=1)
    rows_close(out[0, 0][~torch.from_numpy(empty)], r["out"][~empty], RTOL[wl.kv_dtype], "sparse out")
    lse_close(lse[0, 0], r["lse"], RTOL[wl.kv_dtype])


@pytest.mark.parametrize("cfg,n_q", [(2, 3), (2, 300), (4, 40)])
def test_sparse_duplicate_entries_count_each_time(hs2, orc, cfg, n_q):
    """An index row may name a position more than once (the ABI attends to it
    as often as it appears, as the oracle does): rows drawn with replacement
    from a few hundred positions, so most positions repeat, against the oracle;
    few tokens take the split path, many the one-workgroup path."""
    n_ctx, n_sel = 3000, 1152
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=n_ctx - n_q, n_ctx=n_ctx, n_needles=0, needles="none",
                             n_sparse=1)
    x = make_inputs(wl)
    rng = np.random.default_rng(29 + n_q)
    pool = rng.choice(n_ctx, size=300, replace=False)
    idx = np.sort(rng.choice(pool, size=(n_q, n_sel), replace=True), axis=1).astype(np.int32)
    idx[:, -5:] = -1
    say("sparse with duplicate entries", wl.name, n_q)
    out, lse = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                               indices=torch.from_numpy(idx).reshape(1, n_q, n_sel).cuda(), sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    r = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, idx, x.sm_scale, list(range(n_q)))
    rows_close(out[0, 0], r["out"], RTOL[wl.kv_dtype], "sparse out (duplicates)")
    lse_close(lse[0, 0], r["lse"], RTOL[wl.kv_dtype], "sparse lse (duplicates)")


@pytest.mark.parametrize("cfg,H,d,n_q,n_sel", [(2, 4, 64, 9, 384), (2, 8, 128, 17, 1152), (4, 8, 64, 5, 700),
                                               (4, 4, 128, 33, 1152)])
def test_sparse_few_tokens_head_shapes(hs2, orc, cfg, H, d, n_q, n_sel):
    """Sparse layers for few query tokens (the split path and its combine) at
    every head count and head dimension instantiated, bf16 and FP8 caches,
    ragged index rows."""
    n_ctx = 4000
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=n_ctx - n_q, n_ctx=n_ctx, H=H, d=d, n_needles=0,
                             needles="none", n_sparse=1)
    x = make_inputs(wl)
    rng = np.random.default_rng(n_q * 13 + H + d)
    idx = _rand_index_rows(rng, n_q, n_sel, n_ctx, 0)
    say("sparse few tokens", wl.name, H, d, n_q, n_sel)
    out, lse = hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                               indices=torch.from_numpy(idx).reshape(1, n_q, n_sel).cuda(), sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    r = orc.sparse(x.q_sparse[0].contiguous(), x.k, x.v, x.k_scale, x.v_scale, idx, x.sm_scale, list(range(n_q)))
    empty = (idx < 0).all(axis=1)
    rows_close(out[0, 0][~torch.from_numpy(empty)], r["out"][~empty], RTOL[wl.kv_dtype], "sparse out")
    assert (to_np(out[0, 0])[empty] == 0).all()
    lse_close(lse[0, 0], r["lse"], RTOL[wl.kv_dtype])


@pytest.mark.parametrize("H,q_pos0", [(16, 70000), (4, 30000)])
def test_streaming_topk_repeatable_under_many_trims(hs2, orc, H, q_pos0):
    """Rows with tens of thousands of candidates, so each token's candidate
    buffer is trimmed several times while its keys stream in (16 heads at
    >= 64 Ki candidates: the form without threshold histograms; 4 heads below
    it: the form with them). Six calls, each on a workspace filled with fresh
    random bytes, must give identical index rows, and they must pass the
    oracle's index-set rule."""
    n_q = 96
    wl = workload(2).with_(H=H, n_q=n_q, q_pos0=q_pos0, n_ctx=q_pos0 + n_q, n_needles=4)
    x = make_inputs(wl)
    kv = (dev(x.k), dev(x.v), None, None)
    nws = hs2.workspace_size(hs2.OP_FULL_ATTN_SELECT, 1, n_q, wl.n_ctx, H, wl.d, 128, 1024, hs2.HS2_BF16)
    gen = torch.Generator(device="cuda").manual_seed(H)
    say("streaming top-k repeatability", H, q_pos0)
    runs = []
    for rep in range(6):
        ws = torch.randint(0, 256, (nws,), dtype=torch.uint8, device="cuda", generator=gen)
        _, _, idx = hs2.full_attn_select(dev(x.q), *kv, q_pos0=q_pos0, window=128, k_global=1024,
                                         sm_scale=x.sm_scale, workspace=ws)
        torch.cuda.synchronize()
        runs.append(idx.clone())
    for rep in range(1, 6):
        bad = (runs[rep] != runs[0]).any(dim=-1).nonzero()
        assert len(bad) == 0, f"call {rep} differs from call 0 in rows {bad[:8].tolist()}"
    rows = list(range(0, n_q, 6))
    ref = orc.full_select(x.q, x.k, x.v, None, None, q_pos0, 128, 1024, x.sm_scale, rows, want_scores=True)
    check_index_rows(runs[0][0, rows], ref["idx"], ref["scores"], ref["kth"], 128)
