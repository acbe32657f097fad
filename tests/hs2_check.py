"""Comparison rules between the HIP path and the CPU oracle.

Outputs: per (query, head) row, max_c |o - o_ref| <= rtol * max_c |o_ref|
(elementwise relative error is meaningless on near-zero entries of averaged
N(0,1) values).
LSE: |LSE - LSE_ref| <= rtol, an absolute bound on the natural-log
normaliser, i.e. the softmax normaliser exp(LSE) itself within relative rtol.
Index sets: the window part must be identical; the global part must have the
oracle's size, be ascending and -1 padded, and hold only positions in
[0, p - window] (causal and disjoint from the window, p being the row's query
position, which is the last entry of its window); every position in the
symmetric difference with the oracle's set must have an oracle score within
`swap_rel` * s_K of the oracle's k-th score s_K (a legitimate near-tie swap).

Every check prints the margin it achieved ("[parity] ..."), so a run's log
shows the headroom left under each tolerance.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.to(torch.float32)
        return t.numpy()
    return np.asarray(t)


def _say(msg: str) -> None:
    print("[parity]", msg, flush=True)
    sys.stdout.flush()


def rows_close(got, ref, rtol: float, what: str = "out") -> float:
    """Returns the worst per-row error relative to the row's largest |ref|."""
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r).max(axis=-1)
    scale = np.abs(r).max(axis=-1)
    rel = err / np.maximum(scale, 1e-30)
    worst = float(rel.max()) if rel.size else 0.0
    bad = err > rtol * scale + 1e-30
    if bad.any():
        i = np.unravel_index(np.argmax(rel), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} rows exceed rtol {rtol}; worst row {i}: err {err[i]:.3e} "
                             f"scale {scale[i]:.3e}")
    _say(f"{what}: {err.size} rows, worst rel err {worst:.3e} (tol {rtol:g}, {worst / rtol:.3f} of it)")
    return worst


# Decode token scores. The fp32-cache path keeps fp32 logits: relative 1e-5 of
# the row maximum. The bf16 / FP8 split kernel hands the logits to the score
# kernel as 16-bit codes c = round(1024 (M - x)) below the maximum M of the
# key's 32-key block and head (x, M base-2 logits), so every term
# 2^(x - LSE) is read back within a factor 2^(+-1/2048), relative 3.4e-4, and
# a term clamped at c = 65535 is below 2^-64 of its block's largest term.
# Bound per score: 4e-4 of itself (the code rounding plus fp32 arithmetic)
# plus 1e-17 of the row maximum (H clamped terms).
SCORE_CODE_REL = 4e-4
SCORE_CODE_ABS = 1e-17


def decode_scores_close(got, ref, kv_dtype: str, what: str = "score vector") -> float:
    """Checks a decode score vector [B][n_ctx] against the oracle's; returns
    the worst error as a fraction of the allowed error."""
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    rowmax = np.maximum(r.max(axis=-1, keepdims=True), 1e-300)
    if kv_dtype == "f32":
        allow = 1e-5 * rowmax + 0 * r
    else:
        allow = SCORE_CODE_REL * r + SCORE_CODE_ABS * rowmax
    err = np.abs(g - r)
    frac = err / allow
    worst = float(frac.max()) if frac.size else 0.0
    rel = float((err / np.maximum(r, 1e-300)).max()) if r.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(np.argmax(frac), frac.shape)
        raise AssertionError(f"{what}: worst entry {i}: got {g[i]:.9e} ref {r[i]:.9e} ({worst:.2f} of the bound)")
    _say(f"{what}: {g.size} scores, worst error {worst:.3f} of the bound (largest relative error {rel:.3e})")
    return worst


def lse_close(got, ref, rtol: float, what: str = "lse") -> float:
    """|dLSE| <= rtol (absolute). Entries that are -inf on both sides (empty
    rows) agree. Returns the worst |dLSE|."""
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    both_inf = np.isneginf(g) & np.isneginf(r)
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(g - r))
    bad = ~(d <= rtol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.nan_to_num(d, nan=np.inf), 0)), d.shape)
        raise AssertionError(f"{what}: {bad.sum()} entries exceed {rtol} absolute; worst {i}: got {g[i]} "
                             f"want {r[i]}")
    worst = float(d.max()) if d.size else 0.0
    _say(f"{what}: {d.size} entries, worst |dLSE| {worst:.3e} (tol {rtol:g}, {worst / rtol:.3f} of it)")
    return worst


def check_index_rows(gpu_idx, ref_idx, ref_scores, kth, window: int, swap_rel: float = 1e-3,
                     what: str = "index rows"):
    """gpu_idx, ref_idx: [n][window+K]; ref_scores: [n][>= p+1] oracle scores
    (float64) of each row; kth: [n] oracle k-th score. Returns (mean overlap,
    min overlap, number of swapped positions)."""
    g = to_np(gpu_idx).astype(np.int64)
    r = np.asarray(ref_idx, dtype=np.int64)
    assert g.shape == r.shape
    overlaps, swaps, worst_gap = [], 0, 0.0
    for t in range(g.shape[0]):
        assert np.array_equal(g[t, :window], r[t, :window]), f"row {t}: window part differs"
        p = int(r[t, :window].max())  # the window always ends at the query position
        assert p >= 0, f"row {t}: empty window"
        gg, rr = g[t, window:], r[t, window:]
        gv, rv = gg[gg >= 0], rr[rr >= 0]
        assert len(gv) == len(rv), f"row {t}: {len(gv)} global entries, oracle has {len(rv)}"
        assert (gg[len(gv):] == -1).all(), f"row {t}: padding is not at the end"
        assert (np.diff(gv) > 0).all(), f"row {t}: global part not strictly ascending"
        if len(gv):
            assert gv[0] >= 0 and gv[-1] <= p - window, (
                f"row {t}: global entries {gv[0]}..{gv[-1]} outside [0, p - window] = [0, {p - window}]")
        diff = np.setxor1d(gv, rv)
        if len(diff):
            sK = kth[t]
            sc = ref_scores[t][diff]
            gap = np.abs(sc - sK) / max(abs(sK), 1e-300)
            assert (gap <= swap_rel).all(), (
                f"row {t}: swapped positions {diff[:8]} have scores {sc[:8]} vs s_K {sK}")
            worst_gap = max(worst_gap, float(gap.max()))
            swaps += len(diff) // 2
        if len(rv):
            overlaps.append(len(np.intersect1d(gv, rv)) / len(rv))
    ov = float(np.mean(overlaps)) if overlaps else 1.0
    mn = float(np.min(overlaps)) if overlaps else 1.0
    _say(f"{what}: {g.shape[0]} rows, overlap mean {ov:.5f} min {mn:.5f}, {swaps} near-tie swaps "
         f"(worst |s - s_K| / s_K {worst_gap:.2e}, tol {swap_rel:g})")
    return ov, mn, swaps
