"""GPU parity of the light-indexer selection (hs2_index_select) and of
IndexCache reuse against the CPU oracle, through the C ABI.

Exact-arithmetic inputs (integer codes, unit scales, weights k/8) make every
score exact in fp32, so the index rows must be bit-identical to the oracle's,
ties included. On Gaussian FP8 inputs the window part must match exactly and
the global part may differ from the fp64 choice only by swaps of positions
whose scores lie within 1e-3 of the k-th score (relative to the larger of |k-th
score| and 1e-3 of the row's largest |score|: indexer scores can be near 0 or
negative). IndexCache: layers F, S, S share one index set; each attends with
its own queries (rel 1e-2, bf16)."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_indexer_inputs, make_inputs, workload
from tests.hs2_check import lse_close, rows_close, to_np

pytestmark = pytest.mark.gpu


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


def _run(hs2, x, q_pos0, window, kg):
    idx = hs2.index_select(x.qi.cuda(), x.qs.cuda(), x.w.cuda(), x.ki.cuda(), x.ks.cuda(), q_pos0=q_pos0,
                           window=window, k_global=kg)
    torch.cuda.synchronize()
    return to_np(idx).astype(np.int64)


@pytest.mark.parametrize("B,n_q,q_pos0,n_ctx,HI,dI,kg", [
    (1, 300, 200, 500, 4, 64, 64),          # ragged, early rows with fewer candidates than k
    (2, 100, 5000, 5100, 8, 128, 1024),     # > 4096 candidates per token: trims while streaming
    (1, 64, 2000, 2064, 16, 64, 256),       # 16 heads: one token per wave half
    (1, 40, 9000, 9040, 8, 64, 2048),       # the largest k
    # rows with 64 Ki candidates or more: the form without threshold histograms,
    # whose superset trims and final compaction every 16-head exact pass 2 runs
    (1, 48, 70000, 70048, 8, 64, 1024),
    (2, 20, 66000, 66020, 16, 128, 2048),
    (1, 33, 80000, 80033, 4, 64, 256),
])
def test_index_select_exact_is_bit_identical(hs2, orc, B, n_q, q_pos0, n_ctx, HI, dI, kg):
    x = make_indexer_inputs(B * n_q + HI + kg, B, n_q, q_pos0, n_ctx, HI, dI, exact=True)
    say("index select exact", B, n_q, q_pos0, n_ctx, HI, dI, kg)
    got = _run(hs2, x, q_pos0, 128, kg).reshape(B * n_q, -1)
    rows = list(range(B * n_q))
    ref = orc.index_select(x.qi, x.qs, x.w, x.ki, x.ks, q_pos0, 128, kg, rows)
    bad = np.nonzero((got != ref["idx"]).any(axis=1))[0]
    assert len(bad) == 0, f"rows {bad[:8]} differ"
    say(f"  [parity] {len(rows)} index rows bit-identical")


def _check_near_ties(got, ref, window):
    swaps = 0
    for t in range(got.shape[0]):
        assert np.array_equal(got[t, :window], ref["idx"][t, :window]), f"row {t}: window differs"
        g, r = got[t, window:], ref["idx"][t, window:]
        gv, rv = g[g >= 0], r[r >= 0]
        assert len(gv) == len(rv) and (np.diff(gv) > 0).all()
        diff = np.setxor1d(gv, rv)
        if len(diff):
            s = ref["scores"][t]
            kth = ref["kth"][t]
            fin = s[np.isfinite(s)]
            tol = 1e-3 * max(abs(kth), 1e-3 * np.abs(fin).max())
            assert (np.abs(s[diff] - kth) <= tol).all(), f"row {t}: swaps {diff[:6]} scores {s[diff][:6]} kth {kth}"
            swaps += len(diff) // 2
    say(f"  [parity] {got.shape[0]} index rows: window parts identical, {swaps} near-tie swaps")
    return swaps


@pytest.mark.parametrize("B,n_q,q_pos0,n_ctx,HI,dI,kg", [
    (1, 256, 3000, 3256, 8, 128, 1024),
    (2, 77, 6000, 6077, 4, 64, 512),
    (1, 50, 12000, 12050, 16, 128, 1024),
])
def test_index_select_gaussian_near_ties_only(hs2, orc, B, n_q, q_pos0, n_ctx, HI, dI, kg):
    x = make_indexer_inputs(7 * n_q + HI, B, n_q, q_pos0, n_ctx, HI, dI, n_needles=8)
    say("index select gaussian", B, n_q, q_pos0, n_ctx, HI, dI, kg)
    got = _run(hs2, x, q_pos0, 128, kg).reshape(B * n_q, -1)
    rows = list(range(B * n_q))
    ref = orc.index_select(x.qi, x.qs, x.w, x.ki, x.ks, q_pos0, 128, kg, rows, want_scores=True)
    sw = _check_near_ties(got, ref, 128)
    say(f"  near-tie swaps {sw}")
    for row, h, j in x.needles:
        assert j in got[row, 128:], f"needle at {j} of row {row} not selected"


def test_index_select_full_size_sampled(hs2, orc):
    """The 32k-token prefill shape with 8 indexer heads of 128 dims, k = 1024;
    64 sampled rows against the oracle."""
    n = 32768
    x = make_indexer_inputs(2026, 1, n, 0, n, 8, 128, n_needles=32)
    say("index select full size", n)
    got = _run(hs2, x, 0, 128, 1024).reshape(n, -1)
    rng = np.random.default_rng(8)
    rows = sorted({0, 127, 128, 1151, 1152, n - 1} | {r for r, _, _ in x.needles} |
                  set(rng.choice(n, 40, replace=False).tolist()))
    ref = orc.index_select(x.qi, x.qs, x.w, x.ki, x.ks, 0, 128, 1024, rows, want_scores=True)
    _check_near_ties(got[rows], ref, 128)
    for row, h, j in x.needles:
        assert j in got[row, 128:]


def test_indexcache_layers_share_one_index_set(hs2, orc):
    """IndexCache pattern F S S: the F layer's indexer rows serve all three
    layers' sparse attention, each with its own queries."""
    wl = workload(2).with_(B=1, n_q=200, q_pos0=2800, n_ctx=3000, n_needles=2, n_sparse=3)
    x = make_inputs(wl)
    xi = make_indexer_inputs(99, 1, wl.n_q, wl.q_pos0, wl.n_ctx, 8, 128)
    say("indexcache F S S", wl.name)
    idx = hs2.index_select(xi.qi.cuda(), xi.qs.cuda(), xi.w.cuda(), xi.ki.cuda(), xi.ks.cuda(), q_pos0=wl.q_pos0,
                           window=wl.window, k_global=wl.k_global)
    out, lse = hs2.sparse_attn(x.q_sparse.cuda(), x.k.cuda(), x.v.cuda(), indices=idx, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows = list(range(wl.n_q))
    gi = to_np(idx[0]).astype(np.int32)
    ri = orc.index_select(xi.qi, xi.qs, xi.w, xi.ki, xi.ks, wl.q_pos0, wl.window, wl.k_global, rows,
                          want_scores=True)
    _check_near_ties(gi.astype(np.int64), ri, wl.window)
    for l in range(3):
        s = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, None, None, gi, x.sm_scale, rows)
        rows_close(out[l, 0], s["out"], 1e-2, f"layer {l} out")
        lse_close(lse[l, 0], s["lse"], 1e-2, f"layer {l} lse")
