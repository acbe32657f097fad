"""GPU parity of the HySparse (v1) block-level variant (hs2_block_attn_select,
hs2_block_sparse_attn) against the CPU oracle, through the C ABI.

Block choice: bit-exact against the oracle's selection applied to the GPU's
own fp32 block scores, and against the oracle's fp64 block scores equal up to
swaps of blocks whose scores lie within 1e-3 relative of the k-th one. Block
scores: within 1e-3 relative (fp32 sums of fp32 exponentials against fp64).
Outputs: rel 1e-5 (f32) / 1e-2 (bf16, FP8 caches), per row, as elsewhere."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_gates, make_inputs, workload
from tests.hs2_check import lse_close, rows_close, to_np

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}
KB = 16


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


def check_blocks(orc, g_idx, g_scores, ref, pos, kb, swap_rel=1e-3):
    """g_idx [n][kb], g_scores [n][n_blk] (GPU); ref from orc.block_select."""
    gi = to_np(g_idx).astype(np.int64)
    gs = to_np(g_scores).astype(np.float64)
    rs = ref["block_scores"]
    swaps = 0
    for t, p in enumerate(pos):
        nc = p // 64 + 1
        # scores of every causal block
        err = np.abs(gs[t, :nc] - rs[t, :nc])
        assert (err <= 1e-3 * rs[t, :nc] + 1e-9).all(), f"row {t}: block scores off by {err.max():.3e}"
        # the choice is exact on the GPU's own fp32 scores
        want = orc.select_scores_f32(gs[t:t + 1, :nc].astype(np.float32), [nc], kb)[0]
        assert gi[t].tolist() == want.tolist(), f"row {t}: choice differs from the exact top-k of its scores"
        # against the fp64 choice: only near-ties may differ
        rv = ref["block_idx"][t]
        gv, rr = gi[t][gi[t] >= 0], rv[rv >= 0]
        assert len(gv) == len(rr) == min(kb, nc)
        diff = np.setxor1d(gv, rr)
        if len(diff):
            sK = np.sort(rs[t, :nc])[::-1][min(kb, nc) - 1]
            assert (np.abs(rs[t, diff] - sK) <= swap_rel * sK).all(), f"row {t}: swapped blocks {diff}"
            swaps += len(diff) // 2
    return swaps


@pytest.mark.parametrize("cfg,n_q,q_pos0,n_ctx", [
    (1, 700, 0, 700),            # f32, H=4, d=64, from position 0 (fewer blocks than 16 early on)
    (2, 1000, 0, 1000),          # bf16, H=16, d=128
    (2, 300, 3700, 4000),        # bf16 chunk at an offset, ragged last block
    (4, 77, 3000, 3077),         # FP8 cache with clustered needles
    (2, 1, 4999, 5000),          # one query token
])
def test_block_attn_select_matches_oracle(hs2, orc, cfg, n_q, q_pos0, n_ctx):
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=4)
    x = make_inputs(wl)
    say("block select", wl.name, n_q, q_pos0, n_ctx)
    out, lse, bidx, bsc = hs2.block_attn_select(dev(x.q), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                                q_pos0=q_pos0, k_blocks=KB, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(n_q))
    ref = orc.block_select(x.q, x.k, x.v, x.k_scale, x.v_scale, q_pos0, 64, KB, x.sm_scale, rows)
    tol = RTOL[wl.kv_dtype]
    rows_close(out[0], ref["out"], tol, "block-mode out")
    lse_close(lse[0], ref["lse"], tol)
    sw = check_blocks(orc, bidx[0], bsc[0], ref, ref["pos"], KB)
    say(f"  near-tie swaps {sw}")


@pytest.mark.parametrize("cfg,B,n_q,q_pos0,n_ctx,L,window", [
    (1, 1, 500, 0, 500, 1, 128),       # f32
    (2, 2, 200, 300, 500, 2, 128),     # bf16, two sequences, two layers
    (4, 1, 60, 2000, 2060, 1, 128),    # FP8 cache
    (2, 1, 100, 900, 1000, 1, 300),    # window of 300 (three 128-row tiles)
])
def test_block_sparse_attn_matches_oracle(hs2, orc, cfg, B, n_q, q_pos0, n_ctx, L, window):
    wl = workload(cfg).with_(B=B, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=2, n_sparse=L)
    x = make_inputs(wl)
    H, d = wl.H, wl.d
    say("block sparse", wl.name, B, n_q, q_pos0, n_ctx, L, window)
    _, _, bidx, _ = hs2.block_attn_select(dev(x.q), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                          q_pos0=q_pos0, k_blocks=KB, sm_scale=x.sm_scale, want_scores=False)
    gates = make_gates(B * n_q + L, (L, B, n_q, H, 2))
    out = hs2.block_sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                block_idx=bidx, q_pos0=q_pos0, window=window, gates=dev(gates),
                                sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(B * n_q))
    gb = to_np(bidx).reshape(B * n_q, KB).astype(np.int32)
    tol = RTOL[wl.kv_dtype]
    for l in range(L):
        ref = orc.block_sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gb, 64, window,
                               gates[l].reshape(B * n_q, H, 2).numpy(), q_pos0, x.sm_scale, rows)
        rows_close(out[l].reshape(B * n_q, H, d), ref["out"], tol, f"block sparse out, layer {l}")


def test_block_variant_full_size_sampled(hs2, orc):
    """The 32k-token bf16 prefill shape (16 heads, d = 128) with two sparse
    layers; 48 sampled rows through both entry points."""
    wl = workload(2)
    x = make_inputs(wl)
    say("block variant full size", wl.name)
    out, lse, bidx, bsc = hs2.block_attn_select(dev(x.q), dev(x.k), dev(x.v), q_pos0=0, k_blocks=KB,
                                                sm_scale=x.sm_scale)
    gates = make_gates(7, (wl.n_sparse, 1, wl.n_q, wl.H, 2))
    so = hs2.block_sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), block_idx=bidx, q_pos0=0, window=128,
                               gates=dev(gates), sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted({0, 63, 64, wl.n_q - 1} | set(rng.choice(wl.n_q, 44, replace=False).tolist()))
    ref = orc.block_select(x.q, x.k, x.v, None, None, 0, 64, KB, x.sm_scale, rows)
    rows_close(out[0][rows], ref["out"], 1e-2, "block-mode out")
    lse_close(lse[0][rows], ref["lse"], 1e-2)
    check_blocks(orc, bidx[0][rows], bsc[0][rows], ref, ref["pos"], KB)
    gb = to_np(bidx[0][rows]).astype(np.int32)
    for l in range(wl.n_sparse):
        s = orc.block_sparse(x.q_sparse[l].contiguous(), x.k, x.v, None, None, gb, 64, 128,
                             gates[l, 0].numpy(), 0, x.sm_scale, rows)
        rows_close(so[l, 0][rows], s["out"], 1e-2, f"block sparse out, layer {l}")
