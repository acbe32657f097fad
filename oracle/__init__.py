"""Python face of the CPU oracle (oracle/hs2_oracle.c).

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the benchmark's
CPU-baseline leg use this package. It imports nothing from the HIP library
and the HIP library imports nothing from it.

Arrays are CPU torch tensors or numpy arrays in their storage formats
(float32, bfloat16, uint8 FP8 codes + float32 per-token scales); the C code
widens them to double itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_hs2.so")
_lib = None

F32, BF16, FP8 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_d = ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_full_select.argtypes = [_p, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i64, _i, _i,
                                      _i, _i, _d, _p, _i64, _p, _p, _p, _p, _p]
        L.orc_full_select.restype = _i
        L.orc_sparse.argtypes = [_p, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i, _i, _p, _i, _d,
                                 _p, _i64, _p, _p]
        L.orc_sparse.restype = _i
        L.orc_select_scores_f32.argtypes = [_p, _i64, _i64, _p, _i, _p]
        L.orc_select_scores_f32.restype = _i
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = _d
        L.orc_e4m3_encode.argtypes = [_d]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_kv_project.argtypes = [_p, _i64, _i, _p, _i, _i, _p, _i64, _p, _p, _p]
        L.orc_kv_project.restype = _i
        L.orc_block_select.argtypes = [_p, _i64, _i64, _p, _i, _i, _p, _p]
        L.orc_block_select.restype = _i
        L.orc_index_select.argtypes = [_p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i, _i, _i, _i, _p, _i64, _p, _p,
                                       _p]
        L.orc_index_select.restype = _i
        L.orc_num_threads.restype = _i
        L.orc_set_threads.argtypes = [_i]
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.device.type == "cpu" and t.is_contiguous()
        return t.data_ptr()
    assert isinstance(t, np.ndarray) and t.flags["C_CONTIGUOUS"]
    return t.ctypes.data


def _dt(t: torch.Tensor) -> int:
    return _DT[t.dtype]


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def full_select(q, k, v, k_scale, v_scale, q_pos0: int, window: int, k_global: int,
                sm_scale: float, rows: Sequence[int], want_scores: bool = False,
                select: bool = True):
    """Full attention + score + selection for flat query rows `rows`.

    q: [B][n_q][H][d]; k, v: [B][n_ctx][d]. Returns dict with out [n][H][d],
    lse [n][H] (float64), idx [n][window+k_global] int32, kth [n] and, if
    asked, scores [n][n_ctx] (-1 beyond the causal limit)."""
    B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = len(rows_a)
    out = np.zeros((n, H, d), np.float64)
    lse = np.zeros((n, H), np.float64)
    S = window + k_global
    idx = np.zeros((n, S), np.int32) if select else None
    kth = np.zeros((n,), np.float64)
    sc = np.zeros((n, n_ctx), np.float64) if want_scores else None
    rc = lib().orc_full_select(_ptr(q), _dt(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                               _dt(k), B, n_q, q_pos0, n_ctx, H, d, window, k_global, sm_scale,
                               _ptr(rows_a), n, _ptr(out), _ptr(lse), _ptr(idx), _ptr(sc),
                               _ptr(kth))
    if rc != 0:
        raise ValueError("oracle full_select: invalid arguments")
    return {"out": out, "lse": lse, "idx": idx, "kth": kth, "scores": sc, "rows": rows_a}


def sparse(q, k, v, k_scale, v_scale, idx, sm_scale: float, rows: Sequence[int]):
    """Sparse attention of query rows `rows` of q ([B][n_q][H][d]) over the
    positions in idx[r] (one index row per entry of `rows`; < 0 skipped)."""
    B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    idx_a = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    assert idx_a.shape[0] == len(rows_a)
    n = len(rows_a)
    out = np.zeros((n, H, d), np.float64)
    lse = np.zeros((n, H), np.float64)
    rc = lib().orc_sparse(_ptr(q), _dt(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _dt(k),
                          B, n_q, n_ctx, H, d, _ptr(idx_a), idx_a.shape[1], sm_scale,
                          _ptr(rows_a), n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle sparse: invalid arguments")
    return {"out": out, "lse": lse}


def select_scores_f32(scores: np.ndarray, n_cand: Sequence[int], k: int) -> np.ndarray:
    """Top-k (score desc, position asc) of each row's first n_cand[r] entries,
    written ascending and padded with -1."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    rows, stride = s.shape
    nc = np.ascontiguousarray(np.asarray(n_cand, dtype=np.int64))
    out = np.zeros((rows, k), np.int32)
    rc = lib().orc_select_scores_f32(_ptr(s), rows, stride, _ptr(nc), k, _ptr(out))
    if rc != 0:
        raise ValueError("oracle select: invalid arguments")
    return out


def e4m3_encode(x: float) -> int:
    """Nearest OCP E4M3FN code, ties to even, saturating at +-448."""
    return int(lib().orc_e4m3_encode(float(x)))


def kv_project(h, w, rows: Sequence[int], quantize: bool = False):
    """KV Bridging projections of the hidden rows `rows`.
    h [T][hidden] bf16, w [J][2][d][hidden] bf16 (CPU). Returns x [J][2][n][d]
    float64 and, with quantize, codes uint8 [J][2][n][d] and scales [J][2][n]."""
    T, hidden = h.shape
    J, two, d, hid2 = w.shape
    if two != 2 or hid2 != hidden:
        raise ValueError("w must be [J][2][d][hidden]")
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = len(r)
    x = np.zeros((J, 2, n, d), np.float64)
    codes = np.zeros((J, 2, n, d), np.uint8) if quantize else None
    scales = np.zeros((J, 2, n), np.float64) if quantize else None
    rc = lib().orc_kv_project(_ptr(h.contiguous()), T, hidden, _ptr(w.contiguous()), J, d, _ptr(r), n, _ptr(x),
                              _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle kv_project: invalid arguments")
    return {"x": x, "codes": codes, "scales": scales}


def block_select_scores(scores: np.ndarray, pos: Sequence[int], block: int, k_blocks: int):
    """Block scores (sum of each block's causal token scores) and the top
    k_blocks blocks of each row (ascending, -1 padded). scores [n][stride] fp64."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    n, stride = s.shape
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    n_blk = (stride + block - 1) // block
    bs = np.zeros((n, n_blk), np.float64)
    bi = np.zeros((n, k_blocks), np.int32)
    rc = lib().orc_block_select(_ptr(s), n, stride, _ptr(p), block, k_blocks, _ptr(bs), _ptr(bi))
    if rc != 0:
        raise ValueError("oracle block_select: invalid arguments")
    return bs, bi


def block_select(q, k, v, k_scale, v_scale, q_pos0: int, block: int, k_blocks: int, sm_scale: float,
                 rows: Sequence[int]):
    """HySparse (v1) full layer for flat query rows `rows`: exact attention (out,
    lse), token scores, block scores and the selected blocks."""
    r = full_select(q, k, v, k_scale, v_scale, q_pos0, 1, 0, sm_scale, rows, want_scores=True, select=False)
    n_q = q.shape[1]
    pos = q_pos0 + r["rows"] % n_q
    bs, bi = block_select_scores(r["scores"], pos, block, k_blocks)
    return {"out": r["out"], "lse": r["lse"], "scores": r["scores"], "block_scores": bs, "block_idx": bi,
            "pos": pos, "rows": r["rows"]}


def block_index_rows(pos: Sequence[int], block_idx: np.ndarray, block: int, window: int):
    """Index rows of the two branches: the window max(0, p-window+1)..p (padded
    with -1 to `window` entries) and the positions <= p of the selected blocks
    (block by block, -1 for empty blocks and positions past p)."""
    pos = np.asarray(pos, dtype=np.int64)
    n, kb = block_idx.shape
    win = np.full((n, window), -1, np.int32)
    blk = np.full((n, kb * block), -1, np.int32)
    for r in range(n):
        p = int(pos[r])
        nw = min(p + 1, window)
        win[r, :nw] = np.arange(p - nw + 1, p + 1)
        for t in range(kb):
            c = int(block_idx[r, t])
            if c < 0:
                continue
            js = np.arange(c * block, (c + 1) * block)
            blk[r, t * block:(t + 1) * block] = np.where(js <= p, js, -1)
    return win, blk


def block_sparse(q, k, v, k_scale, v_scale, block_idx, block: int, window: int, gates, q_pos0: int,
                 sm_scale: float, rows: Sequence[int]):
    """One HySparse (v1) sparse layer for flat query rows `rows` (reading R25):
    attention over the selected blocks and, separately, over the sliding window,
    each with its own softmax, fused as out = g[..., 0] o_blocks + g[..., 1] o_window.
    block_idx [n][k_blocks] per entry of rows; gates [B*n_q][H][2]."""
    rows_a = np.asarray(rows, dtype=np.int64)
    n_q = q.shape[1]
    pos = q_pos0 + rows_a % n_q
    win, blk = block_index_rows(pos, np.asarray(block_idx), block, window)
    ow = sparse(q, k, v, k_scale, v_scale, win, sm_scale, rows_a)
    ob = sparse(q, k, v, k_scale, v_scale, blk, sm_scale, rows_a)
    g = np.asarray(gates, dtype=np.float64)[rows_a]
    out = g[..., 0:1] * ob["out"] + g[..., 1:2] * ow["out"]
    return {"out": out, "out_blocks": ob["out"], "out_window": ow["out"], "lse_blocks": ob["lse"],
            "lse_window": ow["lse"], "win_idx": win, "blk_idx": blk}


def index_select(qi, qs, w, ki, ks, q_pos0: int, window: int, k_global: int, rows: Sequence[int],
                 want_scores: bool = False):
    """Light-indexer scores and the window + top-k index rows for flat query
    rows `rows`. qi [B][n_q][HI][dI] uint8 E4M3 codes, qs [B][n_q][HI] fp32,
    w [B][n_q][HI] fp32, ki [B][n_ctx][dI] uint8 codes, ks [B][n_ctx] fp32."""
    B, n_q, HI, dI = qi.shape
    n_ctx = ki.shape[1]
    rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = len(rows_a)
    idx = np.zeros((n, window + k_global), np.int32)
    kth = np.zeros((n,), np.float64)
    sc = np.zeros((n, n_ctx), np.float64) if want_scores else None
    rc = lib().orc_index_select(_ptr(qi.contiguous()), _ptr(qs.contiguous()), _ptr(w.contiguous()),
                                _ptr(ki.contiguous()), _ptr(ks.contiguous()), B, n_q, q_pos0, n_ctx, HI, dI, window,
                                k_global, _ptr(rows_a), n, _ptr(sc), _ptr(idx), _ptr(kth))
    if rc != 0:
        raise ValueError("oracle index_select: invalid arguments")
    return {"idx": idx, "kth": kth, "scores": sc, "rows": rows_a}

