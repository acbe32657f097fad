"""The decode path's 16-bit logit codes, modelled on the CPU (no GPU).

The bf16 / FP8 decode kernel keeps each base-2 logit x of key j and head h as
c = min(round(1024 (M - x)), 65535), M the maximum of head h over the key's
32-key block, and the score kernel forms score_j = sum_h 2^(M - c/1024 - LSE_h).
This test builds that model with numpy from float64 logits of seeded inputs
and checks the two claims the design rests on: every coded score is within
4e-4 of the exact one (plus 1e-17 of the row maximum for clamped terms), and a
selection made on coded scores differs from the exact one only by swaps
whose exact scores lie within 1e-3 of the exact K-th score. It also shows
why the range is 64: with resolution 2^-11 and a clamp 32 below the block
maximum, peaked attention moves small scores by orders of magnitude.
"""
import math

import numpy as np
import pytest
import torch

from hs2_inputs import make_inputs, workload

STEP, CLAMP = 1.0 / 1024.0, 65535


def base2_logits(B, n_ctx, scale_mult):
    wl = workload(3).with_(B=B, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=1, needles="decode",
                           n_needles=8, decode=True)
    x = make_inputs(wl)
    sm = scale_mult / math.sqrt(wl.d)
    q = x.q[:, 0].to(torch.float64)                       # [B][H][d]
    k = x.k.to(torch.float64)                             # [B][n_ctx][d]
    lg = torch.einsum("bhd,bjd->bjh", q, k) * (sm * math.log2(math.e))
    return lg.numpy(), wl


def exact_and_coded(x2, step, clamp):
    """x2 [n][H] base-2 logits of one sequence -> (exact, coded) scores."""
    n, H = x2.shape
    mx = x2.max(axis=0)
    lse2 = np.log2(np.exp2(x2 - mx).sum(axis=0)) + mx
    exact = np.exp2(x2 - lse2).sum(axis=1)
    nb = (n + 31) // 32
    pad = np.full((nb * 32, H), -np.inf)
    pad[:n] = x2
    M = np.repeat(pad.reshape(nb, 32, H).max(axis=1), 32, axis=0)[:n]
    c = np.minimum(np.floor((M - x2) / step + 0.5), clamp)
    coded = np.exp2(M - c * step - lse2).sum(axis=1)
    return exact, coded


def swap_violations(exact, coded, n_cand, K):
    o_ex = np.lexsort((np.arange(n_cand), -exact[:n_cand]))[:K]
    o_cd = np.lexsort((np.arange(n_cand), -coded[:n_cand]))[:K]
    s_k = exact[o_ex[-1]]
    diff = np.setxor1d(o_ex, o_cd)
    return int((np.abs(exact[diff] - s_k) > 1e-3 * s_k).sum()), len(diff)


@pytest.mark.parametrize("B,n_ctx,scale_mult", [(2, 5003, 1.0), (1, 20000, 1.0), (2, 5003, 12.0), (1, 20000, 12.0)])
def test_coded_scores_within_bound_and_swap_rule(B, n_ctx, scale_mult):
    lg, wl = base2_logits(B, n_ctx, scale_mult)
    for b in range(B):
        exact, coded = exact_and_coded(lg[b], STEP, CLAMP)
        allow = 4e-4 * exact + 1e-17 * exact.max()
        assert (np.abs(coded - exact) <= allow).all(), float((np.abs(coded - exact) / allow).max())
        bad, n_diff = swap_violations(exact, coded, n_ctx - wl.window, wl.k_global)
        assert bad == 0, (bad, n_diff)


def test_peaked_attention_clamps_and_the_narrow_range_would_not_hold():
    lg, wl = base2_logits(1, 20000, 12.0)
    x2 = lg[0]
    nb = x2.shape[0] // 32
    blk = x2[:nb * 32].reshape(nb, 32, -1)
    assert (blk.max(axis=1) - blk.min(axis=1)).max() > 64.0  # the codes clamp here
    exact, coded = exact_and_coded(x2, STEP, CLAMP)
    _, narrow = exact_and_coded(x2, 1.0 / 2048.0, CLAMP)    # resolution 2^-11, clamp 32 below M
    allow = 4e-4 * exact + 1e-17 * exact.max()
    assert (np.abs(coded - exact) <= allow).all()
    assert (np.abs(narrow - exact) > 1e3 * allow).any()


# The 8-bit form of the timed decode step: codes c = min(round(16 (M - x)), 255)
# give bounds, the collect step keeps every key whose upper bound reaches the
# bin of the K-th largest lower bound, and only those are rescored exactly.
KR, KR_INV = np.float32(1.0221235), np.float32(0.9783545)  # the kernel's 2^(+-(1/32 + 2^-12)), widened


def score_bin(x):
    """The selection's histogram bin: bits 30..19 of the fp32 value."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 19) & 0xFFF


def bounds8(x2):
    """x2 [n][H] base-2 logits -> (exact, lower, upper) scores as the score kernel forms them."""
    n, H = x2.shape
    mx = x2.max(axis=0)
    lse2 = np.log2(np.exp2(x2 - mx).sum(axis=0)) + mx
    exact = np.exp2(x2 - lse2).sum(axis=1)
    nb = (n + 31) // 32
    pad = np.full((nb * 32, H), -np.inf)
    pad[:n] = x2
    M = np.repeat(pad.reshape(nb, 32, H).max(axis=1), 32, axis=0)[:n]
    c = np.minimum(np.floor((M - x2) * 16 + 0.5), 255)
    e = np.exp2(M - c / 16 - lse2)
    upper = e.sum(axis=1) * KR
    lower = np.where(c == 255, 0.0, e).sum(axis=1) * KR_INV
    return exact, lower, upper


@pytest.mark.parametrize("B,n_ctx,scale_mult", [(2, 5003, 1.0), (1, 20000, 1.0), (1, 20000, 12.0)])
def test_eight_bit_bounds_hold_and_keep_the_top_k(B, n_ctx, scale_mult):
    lg, wl = base2_logits(B, n_ctx, scale_mult)
    K = wl.k_global
    for b in range(B):
        exact, lower, upper = bounds8(lg[b])
        assert (lower <= exact * (1 + 1e-9)).all() and (exact <= upper * (1 + 1e-9)).all()
        n_cand = n_ctx - wl.window
        lo, up, ex = lower[:n_cand], upper[:n_cand], exact[:n_cand]
        tbin = score_bin(np.sort(lo)[::-1][K - 1])
        kept = score_bin(up) >= tbin
        top = np.lexsort((np.arange(n_cand), -ex))[:K]
        assert kept[top].all()
        if scale_mult == 1.0:
            assert kept.sum() <= 4096  # the candidate list holds them
