"""HySparse2 attention hot path on AMD MI355X: Python binding of libhs2.so.

The functions below only marshal arguments (device pointers, sizes, the
current HIP stream) into the C ABI of include/hs2.h; every step of the
computation runs in the library's HIP kernels. PyTorch supplies device
memory and streams. There is no fallback: if libhs2.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhs2.so")

HS2_OK, HS2_ERR_INVALID_ARG, HS2_ERR_UNSUPPORTED, HS2_ERR_WORKSPACE, HS2_ERR_HIP = range(5)
HS2_F32, HS2_BF16, HS2_FP8_E4M3 = 0, 1, 2
OP_FULL_ATTN_SELECT, OP_DECODE_STEP, OP_SPARSE_ATTN, OP_SELECT_TOPK = 0, 1, 2, 3
OP_BLOCK_ATTN_SELECT, OP_BLOCK_SPARSE_ATTN, OP_INDEX_SELECT, OP_SPARSE_ATTN_WINDOW = 4, 5, 6, 7

_p, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "hs2_abi_version": ([], _i),
    "hs2_status_string": ([_i], ctypes.c_char_p),
    "hs2_workspace_size": ([_i, _i, _i64, _i64, _i, _i, _i, _i, _i], _sz),
    "hs2_full_attn_select": ([_p, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i64, _i, _i, _i, _i, _f,
                              _p, _p, _p, _p, _sz, _p], _i),
    "hs2_sparse_attn": ([_p, _i, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i, _i, _p, _i, _f, _p, _p,
                         _p, _sz, _p], _i),
    "hs2_decode_step": ([_p, _p, _i, _i, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _f, _p, _p,
                         _p, _p, _p, _p, _p, _sz, _p], _i),
    "hs2_sparse_attn_window": ([_p, _i, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i64, _i, _i, _p, _i, _i, _f, _p,
                                _p, _p, _sz, _p], _i),
    "hs2_probe_gather": ([_p, _i64, _i, _p, _p, _i64, _p, _i64, _p], _i),
    "hs2_probe_mfma": ([_i, _i, _i, _f, _p, _p, _i64, _p], _i),
    "hs2_probe_stream": ([_p, _i64, _p, _i64, _i, _i, _p, _i64, _p], _i),
    "hs2_test_reverse_grid": ([_i], _i),
    "hs2_sparse_attn_noalloc": ([_p, _i, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i, _i, _p, _i, _f, _p, _p,
                                 _p], _i),
    "hs2_select_topk": ([_p, _i64, _i64, _p, _i, _p, _p, _sz, _p], _i),
    "hs2_kv_project": ([_p, _i64, _i, _p, _i, _i, _i, _p, _p, _p, _p, _p], _i),
    "hs2_block_attn_select": ([_p, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i64, _i, _i, _i, _i, _f, _p, _p,
                               _p, _p, _p, _sz, _p], _i),
    "hs2_index_select": ([_p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i, _i, _i, _i, _p, _p, _sz, _p], _i),
    "hs2_block_sparse_attn": ([_p, _i, _i, _p, _p, _p, _p, _i, _i, _i64, _i64, _i64, _i, _i, _p, _i, _i, _i,
                               _p, _f, _p, _p, _sz, _p], _i),
}

_lib = None


class HS2Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} (code {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libhs2.so (built by token_level_top_amd/build.py). Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python token_level_top_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().hs2_status_string(code).decode()


def abi_version() -> int:
    return lib().hs2_abi_version()


_QDT = {torch.float32: HS2_F32, torch.bfloat16: HS2_BF16}
_KVDT = {torch.float32: HS2_F32, torch.bfloat16: HS2_BF16, torch.uint8: HS2_FP8_E4M3}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to libhs2 must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != HS2_OK:
        raise HS2Error(fn, rc)


def workspace_size(op: int, B: int, n_q: int, n_ctx: int, H: int, d: int, window: int, k_global: int,
                   kv_dtype: int) -> int:
    n = lib().hs2_workspace_size(op, B, n_q, n_ctx, H, d, window, k_global, kv_dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("hs2_workspace_size: invalid arguments")
    return n


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def full_attn_select(q, k, v, k_scale=None, v_scale=None, *, q_pos0: int, window: int, k_global: int,
                     sm_scale: float, out=None, lse=None, indices=None, workspace=None, stream=None):
    """hs2_full_attn_select. q [B][n_q][H][d]; k, v [B][n_ctx][d].
    Returns (out [B][n_q][H][d], lse [B][n_q][H] fp32, indices [B][n_q][window+k_global] int32)."""
    B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if lse is None else lse
    if indices is None:
        indices = torch.empty((B, n_q, window + k_global), dtype=torch.int32, device=dev)
    kvdt = _KVDT[k.dtype]
    ws = _workspace(workspace_size(OP_FULL_ATTN_SELECT, B, n_q, n_ctx, H, d, window, k_global, kvdt), dev,
                    workspace)
    rc = lib().hs2_full_attn_select(_ptr(q), _QDT[q.dtype], _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                                    kvdt, B, n_q, q_pos0, n_ctx, H, d, window, k_global, sm_scale, _ptr(out),
                                    _ptr(lse), _ptr(indices), _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(stream))
    _check("hs2_full_attn_select", rc)
    return out, lse, indices


def sparse_attn(q, k, v, k_scale=None, v_scale=None, *, indices, sm_scale: float, out=None, lse=None,
                want_lse: bool = True, workspace=None, stream=None):
    """hs2_sparse_attn. q [L][B][n_q][H][d]; indices [B][n_q][n_sel].
    Returns (out [L][B][n_q][H][d], lse [L][B][n_q][H] or None)."""
    L, B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    n_sel = indices.shape[-1]
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((L, B, n_q, H), dtype=torch.float32, device=dev)
    kvdt = _KVDT[k.dtype]
    ws = _workspace(workspace_size(OP_SPARSE_ATTN, B, n_q, n_ctx, H, d, n_sel, 0, kvdt), dev, workspace)
    rc = lib().hs2_sparse_attn(_ptr(q), _QDT[q.dtype], L, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), kvdt,
                               B, n_q, n_ctx, H, d, _ptr(indices), n_sel, sm_scale, _ptr(out), _ptr(lse),
                               _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check("hs2_sparse_attn", rc)
    return out, lse


def sparse_attn_window(q, k, v, k_scale=None, v_scale=None, *, indices, q_pos0: int, window: int, sm_scale: float,
                       out=None, lse=None, want_lse: bool = True, workspace=None, stream=None):
    """hs2_sparse_attn_window: sparse layers over full-layer index rows
    [B][n_q][window + k_global] with the window shared per query block.
    q [L][B][n_q][H][d]. Returns (out [L][B][n_q][H][d], lse [L][B][n_q][H] or None)."""
    L, B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    k_global = indices.shape[-1] - window
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((L, B, n_q, H), dtype=torch.float32, device=dev)
    kvdt = _KVDT[k.dtype]
    ws = _workspace(workspace_size(OP_SPARSE_ATTN_WINDOW, B, n_q, n_ctx, H, d, window, k_global, kvdt), dev,
                    workspace)
    rc = lib().hs2_sparse_attn_window(_ptr(q), _QDT[q.dtype], L, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), kvdt,
                                      B, n_q, q_pos0, n_ctx, H, d, _ptr(indices), window, k_global, sm_scale,
                                      _ptr(out), _ptr(lse), _ptr(ws), ws.numel() if ws is not None else 0,
                                      _stream(stream))
    _check("hs2_sparse_attn_window", rc)
    return out, lse


def probe_gather(src, idx, scale=None, sink=None, stream=None):
    """hs2_probe_gather: src [n_rows][row_bytes] uint8 (128 or 256 bytes a row),
    idx [n_idx] int32, scale [n_rows] fp32 or None. Returns the sink tensor."""
    n_rows, row_bytes = src.shape
    sink = torch.empty(524288, dtype=torch.int32, device=src.device) if sink is None else sink
    rc = lib().hs2_probe_gather(_ptr(src), n_rows, row_bytes, _ptr(scale), _ptr(idx), idx.numel(), _ptr(sink),
                                sink.numel(), _stream(stream))
    _check("hs2_probe_gather", rc)
    return sink


def probe_stream(src, dst=None, reads_per_write: int = 0, n_blocks: int = 2048, sink=None, stream=None):
    """hs2_probe_stream: src and dst uint8 tensors (sizes multiples of 4096).
    Returns the sink tensor (n_blocks * 256 words)."""
    sink = torch.empty(n_blocks * 256, dtype=torch.int32, device=src.device) if sink is None else sink
    rc = lib().hs2_probe_stream(_ptr(src), src.numel(), _ptr(dst), 0 if dst is None else dst.numel(),
                                reads_per_write, n_blocks, _ptr(sink), sink.numel(), _stream(stream))
    _check("hs2_probe_stream", rc)
    return sink


def probe_mfma(waves_per_simd: int, n_blocks: int, iters: int, one: float = 1.0, ops=None, sink=None,
               stream=None):
    """hs2_probe_mfma: ops None (constant operands) or [64, 16] bf16 (lane l's A
    fragment in ops[l, :8], its B fragment in ops[l, 8:]). Returns the sink
    tensor (n_blocks * 256 * waves_per_simd floats)."""
    n = n_blocks * 256 * waves_per_simd
    sink = torch.empty(n, dtype=torch.float32, device="cuda") if sink is None else sink
    if ops is not None:
        assert ops.dtype == torch.bfloat16 and ops.numel() == 64 * 16 and ops.is_contiguous()
    rc = lib().hs2_probe_mfma(waves_per_simd, n_blocks, iters, one, _ptr(ops), _ptr(sink), sink.numel(),
                              _stream(stream))
    _check("hs2_probe_mfma", rc)
    return sink


def set_reverse_grid(on: bool) -> None:
    """hs2_test_reverse_grid: later calls' kernels deal their work in reverse
    order (a test hook; results must not change)."""
    _check("hs2_test_reverse_grid", lib().hs2_test_reverse_grid(1 if on else 0))


def sparse_attn_noalloc(q, k, v, k_scale=None, v_scale=None, *, indices, sm_scale: float, out=None, lse=None,
                        want_lse: bool = True, stream=None):
    """hs2_sparse_attn_noalloc: sparse_attn without a workspace (the library's
    per-GPU scratch array holds the split partials). Same shapes and returns."""
    L, B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    n_sel = indices.shape[-1]
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((L, B, n_q, H), dtype=torch.float32, device=dev)
    rc = lib().hs2_sparse_attn_noalloc(_ptr(q), _QDT[q.dtype], L, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                                       _KVDT[k.dtype], B, n_q, n_ctx, H, d, _ptr(indices), n_sel, sm_scale,
                                       _ptr(out), _ptr(lse), _stream(stream))
    _check("hs2_sparse_attn_noalloc", rc)
    return out, lse


def decode_step(q_full, q_sparse, k, v, k_scale=None, v_scale=None, *, window: int, k_global: int,
                sm_scale: float, want_scores: bool = False, out_full=None, lse_full=None, out_sparse=None,
                lse_sparse=None, indices=None, scores=None, workspace=None, stream=None):
    """hs2_decode_step. q_full [B][H][d]; q_sparse [L][B][H][d] (L may be 0).
    Returns dict of out_full, lse_full, out_sparse, lse_sparse, indices, scores."""
    B, H, d = q_full.shape
    n_ctx = k.shape[1]
    L = q_sparse.shape[0] if q_sparse is not None else 0
    dev = q_full.device
    out_full = torch.empty_like(q_full) if out_full is None else out_full
    lse_full = torch.empty((B, H), dtype=torch.float32, device=dev) if lse_full is None else lse_full
    if L and out_sparse is None:
        out_sparse = torch.empty_like(q_sparse)
    if L and lse_sparse is None:
        lse_sparse = torch.empty((L, B, H), dtype=torch.float32, device=dev)
    if indices is None:
        indices = torch.empty((B, window + k_global), dtype=torch.int32, device=dev)
    if want_scores and scores is None:
        scores = torch.empty((B, n_ctx), dtype=torch.float32, device=dev)
    kvdt = _KVDT[k.dtype]
    ws = _workspace(workspace_size(OP_DECODE_STEP, B, 1, n_ctx, H, d, window, k_global, kvdt), dev, workspace)
    rc = lib().hs2_decode_step(_ptr(q_full), _ptr(q_sparse) if L else None, _QDT[q_full.dtype], L, _ptr(k),
                               _ptr(v), _ptr(k_scale), _ptr(v_scale), kvdt, B, n_ctx, H, d, window, k_global,
                               sm_scale, _ptr(out_full), _ptr(lse_full), _ptr(out_sparse) if L else None,
                               _ptr(lse_sparse) if L else None, _ptr(indices), _ptr(scores), _ptr(ws),
                               ws.numel(), _stream(stream))
    _check("hs2_decode_step", rc)
    return {"out_full": out_full, "lse_full": lse_full, "out_sparse": out_sparse, "lse_sparse": lse_sparse,
            "indices": indices, "scores": scores}


def select_topk(scores, k: int, n_cand=None, out=None, workspace=None, stream=None):
    """hs2_select_topk. scores [rows][row_len] fp32 (>= 0); n_cand [rows] int32 or None.
    Returns out [rows][k] int32 (ascending positions, -1 padded)."""
    rows, row_len = scores.shape
    dev = scores.device
    out = torch.empty((rows, k), dtype=torch.int32, device=dev) if out is None else out
    ws = _workspace(workspace_size(OP_SELECT_TOPK, rows, 0, row_len, 0, 0, 0, k, 0), dev, workspace)
    rc = lib().hs2_select_topk(_ptr(scores), rows, row_len, _ptr(n_cand), k, _ptr(out), _ptr(ws), ws.numel(),
                               _stream(stream))
    _check("hs2_select_topk", rc)
    return out


def kv_project(h, w, kv_dtype: int = HS2_BF16, k_out=None, v_out=None, k_scale=None, v_scale=None, stream=None):
    """hs2_kv_project. h [T][hidden] bf16, w [J][2][d][hidden] bf16 (K then V).
    Returns k, v [J][T][d] (bf16, or uint8 E4M3 codes) and, for FP8, the scales [J][T] fp32."""
    T, hidden = h.shape
    J, two, d, hid2 = w.shape
    if two != 2 or hid2 != hidden:
        raise ValueError("w must be [J][2][d][hidden]")
    dev = h.device
    odt = torch.uint8 if kv_dtype == HS2_FP8_E4M3 else torch.bfloat16
    k_out = torch.empty((J, T, d), dtype=odt, device=dev) if k_out is None else k_out
    v_out = torch.empty((J, T, d), dtype=odt, device=dev) if v_out is None else v_out
    if kv_dtype == HS2_FP8_E4M3:
        k_scale = torch.empty((J, T), dtype=torch.float32, device=dev) if k_scale is None else k_scale
        v_scale = torch.empty((J, T), dtype=torch.float32, device=dev) if v_scale is None else v_scale
    rc = lib().hs2_kv_project(_ptr(h), T, hidden, _ptr(w), J, d, kv_dtype, _ptr(k_out), _ptr(v_out), _ptr(k_scale),
                              _ptr(v_scale), _stream(stream))
    _check("hs2_kv_project", rc)
    return {"k": k_out, "v": v_out, "k_scale": k_scale, "v_scale": v_scale}


BLOCK = 64  # tokens per block of the block-level (HySparse v1) selection


def block_attn_select(q, k, v, k_scale=None, v_scale=None, *, q_pos0: int, k_blocks: int, sm_scale: float,
                      out=None, lse=None, block_idx=None, block_scores=None, want_scores: bool = True,
                      workspace=None, stream=None):
    """hs2_block_attn_select. Returns (out, lse, block_idx [B][n_q][k_blocks] int32,
    block_scores [B][n_q][ceil(n_ctx/64)] fp32 or None)."""
    B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if lse is None else lse
    if block_idx is None:
        block_idx = torch.empty((B, n_q, k_blocks), dtype=torch.int32, device=dev)
    if block_scores is None and want_scores:
        block_scores = torch.empty((B, n_q, (n_ctx + BLOCK - 1) // BLOCK), dtype=torch.float32, device=dev)
    kvdt = _KVDT[k.dtype]
    ws = _workspace(workspace_size(OP_BLOCK_ATTN_SELECT, B, n_q, n_ctx, H, d, 0, 0, kvdt), dev, workspace)
    rc = lib().hs2_block_attn_select(_ptr(q), _QDT[q.dtype], _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), kvdt,
                                     B, n_q, q_pos0, n_ctx, H, d, BLOCK, k_blocks, sm_scale, _ptr(out), _ptr(lse),
                                     _ptr(block_idx), _ptr(block_scores), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream))
    _check("hs2_block_attn_select", rc)
    return out, lse, block_idx, block_scores


def block_sparse_attn(q, k, v, k_scale=None, v_scale=None, *, block_idx, q_pos0: int, window: int, gates,
                      sm_scale: float, out=None, workspace=None, stream=None):
    """hs2_block_sparse_attn. q [L][B][n_q][H][d]; block_idx [B][n_q][k_blocks];
    gates [L][B][n_q][H][2] fp32. Returns out [L][B][n_q][H][d]."""
    L, B, n_q, H, d = q.shape
    n_ctx = k.shape[1]
    k_blocks = block_idx.shape[-1]
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    qdt = _QDT[q.dtype]
    ws = _workspace(workspace_size(OP_BLOCK_SPARSE_ATTN, B, n_q, n_ctx, H, d, window, k_blocks, qdt), dev,
                    workspace)
    rc = lib().hs2_block_sparse_attn(_ptr(q), qdt, L, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _KVDT[k.dtype],
                                     B, n_q, q_pos0, n_ctx, H, d, _ptr(block_idx), BLOCK, k_blocks, window,
                                     _ptr(gates), sm_scale, _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
                                     _stream(stream))
    _check("hs2_block_sparse_attn", rc)
    return out


def index_select(q_idx, q_scale, weights, k_idx, k_scale, *, q_pos0: int, window: int, k_global: int,
                 indices=None, workspace=None, stream=None):
    """hs2_index_select. q_idx [B][n_q][HI][dI] uint8 E4M3 codes, q_scale and
    weights [B][n_q][HI] fp32, k_idx [B][n_ctx][dI] uint8, k_scale [B][n_ctx].
    Returns indices [B][n_q][window+k_global] int32."""
    B, n_q, HI, dI = q_idx.shape
    n_ctx = k_idx.shape[1]
    dev = q_idx.device
    if indices is None:
        indices = torch.empty((B, n_q, window + k_global), dtype=torch.int32, device=dev)
    ws = _workspace(workspace_size(OP_INDEX_SELECT, B, n_q, n_ctx, 0, dI, 0, 0, 0), dev, workspace)
    rc = lib().hs2_index_select(_ptr(q_idx), _ptr(q_scale), _ptr(weights), _ptr(k_idx), _ptr(k_scale), B, n_q,
                                q_pos0, n_ctx, HI, dI, window, k_global, _ptr(indices), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream))
    _check("hs2_index_select", rc)
    return indices

