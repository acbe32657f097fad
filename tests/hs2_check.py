"""Comparison rules between the HIP path and the CPU oracle.

Outputs: per (query, head) row, max_c |o - o_ref| <= rtol * max_c |o_ref|
(elementwise relative error is meaningless on near-zero entries of averaged
N(0,1) values). LSE: |dLSE| <= rtol * max(1, |LSE_ref|).
Index sets: the window part must be identical; the global part must have the
oracle's size, be ascending and -1 padded; every position in the symmetric
difference with the oracle's set must have an oracle score within
`swap_rel` * s_K of the oracle's k-th score s_K (a legitimate near-tie swap).
"""
from __future__ import annotations

import numpy as np
import torch


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.to(torch.float32)
        return t.numpy()
    return np.asarray(t)


def rows_close(got, ref, rtol: float, what: str = "out") -> float:
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r).max(axis=-1)
    scale = np.abs(r).max(axis=-1)
    bad = err > rtol * scale + 1e-30
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(scale, 1e-30)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} rows exceed rtol {rtol}; worst row {i}: err {err[i]:.3e} "
                             f"scale {scale[i]:.3e}")
    return float((err / np.maximum(scale, 1e-30)).max())


def lse_close(got, ref, rtol: float) -> float:
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(g) & np.isneginf(r)
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(g - r))
    tol = rtol * np.maximum(1.0, np.abs(np.where(both_inf, 0.0, r)))
    bad = ~(d <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, d, 0)), d.shape)
        raise AssertionError(f"lse: {bad.sum()} entries exceed rtol {rtol}; worst {i}: got {g[i]} want {r[i]}")
    return float(np.max(d / tol)) if d.size else 0.0


def check_index_rows(gpu_idx, ref_idx, ref_scores, kth, window: int, swap_rel: float = 1e-3):
    """gpu_idx, ref_idx: [n][window+K]; ref_scores: [n][>= p+1] oracle scores
    (float64) of each row; kth: [n] oracle k-th score. Returns (mean overlap,
    min overlap, number of swapped positions)."""
    g = to_np(gpu_idx).astype(np.int64)
    r = np.asarray(ref_idx, dtype=np.int64)
    assert g.shape == r.shape
    overlaps, swaps = [], 0
    for t in range(g.shape[0]):
        assert np.array_equal(g[t, :window], r[t, :window]), f"row {t}: window part differs"
        gg, rr = g[t, window:], r[t, window:]
        gv, rv = gg[gg >= 0], rr[rr >= 0]
        assert len(gv) == len(rv), f"row {t}: {len(gv)} global entries, oracle has {len(rv)}"
        assert (gg[len(gv):] == -1).all(), f"row {t}: padding is not at the end"
        assert (np.diff(gv) > 0).all(), f"row {t}: global part not strictly ascending"
        diff = np.setxor1d(gv, rv)
        if len(diff):
            sK = kth[t]
            sc = ref_scores[t][diff]
            assert (np.abs(sc - sK) <= swap_rel * sK).all(), (
                f"row {t}: swapped positions {diff[:8]} have scores {sc[:8]} vs s_K {sK}")
            swaps += len(diff) // 2
        if len(rv):
            overlaps.append(len(np.intersect1d(gv, rv)) / len(rv))
    if not overlaps:
        return 1.0, 1.0, swaps
    return float(np.mean(overlaps)), float(np.min(overlaps)), swaps
