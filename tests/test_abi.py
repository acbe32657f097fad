"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/hs2.h declares, sizes workspaces and rejects bad arguments
before it touches any device memory."""
import ctypes
import os
import re

import pytest

import token_level_top_amd as hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned address that is never dereferenced
MIS = 0x10004           # misaligned


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hs2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 19
    L = hs2.lib()
    for n in names:
        assert hasattr(L, n), n
    assert hs2.abi_version() == 1
    assert hs2.status_string(2) == "unsupported dtype or shape"


def test_workspace_sizes():
    ws = hs2.workspace_size
    d3 = ws(hs2.OP_DECODE_STEP, 64, 1, 131072, 16, 128, 128, 1024, hs2.HS2_BF16)
    assert d3 >= 64 * 131072 * 16 * 4            # fp32 logits of every key and head
    assert ws(hs2.OP_SELECT_TOPK, 4, 0, 1000, 0, 0, 0, 16, 0) > 0
    assert ws(hs2.OP_SPARSE_ATTN, 1, 4096, 5000, 16, 128, 1152, 0, hs2.HS2_BF16) == 0   # no split
    assert ws(hs2.OP_SPARSE_ATTN, 64, 1, 5000, 16, 128, 1152, 0, hs2.HS2_BF16) > 0
    with pytest.raises(ValueError):
        ws(8, 1, 1, 1, 16, 128, 128, 1024, 1)
    # the window-sharing sparse layers: band copies of n_q + window + 62 rows
    # (rounded to 64) whatever n_ctx is, plus one partial record per token
    w1 = ws(hs2.OP_SPARSE_ATTN_WINDOW, 1, 8192, 262144, 16, 128, 128, 1024, hs2.HS2_FP8_E4M3)
    w2 = ws(hs2.OP_SPARSE_ATTN_WINDOW, 1, 8192, 9000, 16, 128, 128, 1024, hs2.HS2_FP8_E4M3)
    assert w1 == w2 and w1 >= 8192 * 16 * 130 * 4 + 2 * (2 * 8384 * 128)
    with pytest.raises(ValueError):
        ws(hs2.OP_SPARSE_ATTN_WINDOW, 1, 10, 100, 16, 128, 0, 1024, 1)   # window < 1


def _full(**kw):
    a = dict(q=FAKE, qdt=1, k=FAKE, v=FAKE, ks=None, vs=None, kvdt=1, B=1, n_q=10, q_pos0=0, n_ctx=10, H=16,
             d=128, W=128, K=1024, scale=0.1, out=FAKE, lse=FAKE, idx=FAKE, ws=None, wsb=0, st=None)
    a.update(kw)
    return hs2.lib().hs2_full_attn_select(*a.values())


def test_full_attn_select_validation():
    E = hs2
    assert _full(q=None) == E.HS2_ERR_INVALID_ARG
    assert _full(q=MIS) == E.HS2_ERR_INVALID_ARG
    assert _full(n_q=11) == E.HS2_ERR_INVALID_ARG           # q_pos0 + n_q > n_ctx
    assert _full(q_pos0=-1) == E.HS2_ERR_INVALID_ARG
    assert _full(W=0) == E.HS2_ERR_INVALID_ARG
    assert _full(K=-1) == E.HS2_ERR_INVALID_ARG
    assert _full(scale=0.0) == E.HS2_ERR_INVALID_ARG
    assert _full(scale=float("nan")) == E.HS2_ERR_INVALID_ARG
    assert _full(kvdt=2) == E.HS2_ERR_INVALID_ARG           # fp8 without scales
    assert _full(ks=FAKE, vs=FAKE) == E.HS2_ERR_INVALID_ARG  # scales with a bf16 cache
    assert _full(kvdt=7) == E.HS2_ERR_INVALID_ARG
    assert _full(n_ctx=2 ** 31, n_q=1, q_pos0=0) == E.HS2_ERR_INVALID_ARG
    assert _full(H=12) == E.HS2_ERR_UNSUPPORTED
    assert _full(d=96) == E.HS2_ERR_UNSUPPORTED
    assert _full(qdt=0) == E.HS2_ERR_UNSUPPORTED            # f32 queries with a bf16 cache
    assert _full(K=4096) == E.HS2_ERR_UNSUPPORTED
    assert _full() == E.HS2_ERR_WORKSPACE                   # valid, but no workspace
    need = hs2.workspace_size(hs2.OP_FULL_ATTN_SELECT, 1, 10, 10, 16, 128, 128, 1024, 1)
    assert _full(ws=FAKE, wsb=need - 1) == E.HS2_ERR_WORKSPACE
    assert _full(ws=MIS, wsb=need) == E.HS2_ERR_WORKSPACE


def _decode(**kw):
    a = dict(qf=FAKE, qs=FAKE, qdt=1, L=2, k=FAKE, v=FAKE, ks=None, vs=None, kvdt=1, B=2, n_ctx=1000, H=16,
             d=128, W=128, K=1024, scale=0.1, of=FAKE, lf=FAKE, os_=FAKE, ls=None, idx=FAKE, sc=None, ws=None,
             wsb=0, st=None)
    a.update(kw)
    return hs2.lib().hs2_decode_step(*a.values())


def test_decode_step_validation():
    E = hs2
    assert _decode(qs=None) == E.HS2_ERR_INVALID_ARG         # n_sparse > 0 needs sparse queries
    assert _decode(L=0) == E.HS2_ERR_INVALID_ARG             # ... and none when n_sparse == 0
    assert _decode(L=0, qs=None, os_=None) == E.HS2_ERR_WORKSPACE
    assert _decode(idx=None) == E.HS2_ERR_INVALID_ARG
    assert _decode(sc=MIS) == E.HS2_ERR_INVALID_ARG
    assert _decode(B=0) == E.HS2_ERR_INVALID_ARG
    assert _decode(kvdt=2, ks=FAKE, vs=FAKE) == E.HS2_ERR_WORKSPACE
    assert _decode(kvdt=2, ks=FAKE, vs=FAKE, qdt=0) == E.HS2_ERR_UNSUPPORTED
    assert _decode() == E.HS2_ERR_WORKSPACE


def test_sparse_and_select_validation():
    L = hs2.lib()
    # q, qdt, n_layers, k, v, ks, vs, kvdt, B, n_q, n_ctx, H, d, idx, n_sel, scale, out, lse, ws, wsb, stream
    args = [FAKE, 1, 2, FAKE, FAKE, None, None, 1, 64, 1, 5000, 16, 128, FAKE, 1152, 0.1, FAKE, None, None, 0,
            None]
    assert L.hs2_sparse_attn(*args) == hs2.HS2_ERR_WORKSPACE
    bad = list(args)
    bad[14] = 0
    assert L.hs2_sparse_attn(*bad) == hs2.HS2_ERR_INVALID_ARG
    bad = list(args)
    bad[14] = 5000
    assert L.hs2_sparse_attn(*bad) == hs2.HS2_ERR_UNSUPPORTED
    bad = list(args)
    bad[13] = None
    assert L.hs2_sparse_attn(*bad) == hs2.HS2_ERR_INVALID_ARG
    # scores, rows, row_len, n_cand, k, out, ws, wsb, stream
    assert L.hs2_select_topk(FAKE, 4, 100, None, 8, FAKE, None, 0, None) == hs2.HS2_ERR_WORKSPACE
    assert L.hs2_select_topk(FAKE, 4, 100, None, 0, FAKE, None, 0, None) == hs2.HS2_ERR_INVALID_ARG
    assert L.hs2_select_topk(FAKE, 4, 100, None, 4096, FAKE, None, 0, None) == hs2.HS2_ERR_UNSUPPORTED
    assert L.hs2_select_topk(None, 4, 100, None, 8, FAKE, None, 0, None) == hs2.HS2_ERR_INVALID_ARG


def test_kv_project_validation():
    L = hs2.lib()
    # h, T, hidden, w, n_layers, d, kv_dtype, k_out, v_out, k_scale, v_scale, stream
    args = [FAKE, 1000, 2048, FAKE, 4, 128, hs2.HS2_BF16, FAKE, FAKE, None, None, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_kv_project(*a)

    assert call(a5=96) == hs2.HS2_ERR_UNSUPPORTED              # d not in {64, 128}
    assert call(a2=48) == hs2.HS2_ERR_UNSUPPORTED              # hidden % 32 != 0
    assert call(a6=hs2.HS2_F32) == hs2.HS2_ERR_INVALID_ARG     # not a cache type
    assert call(a6=hs2.HS2_FP8_E4M3) == hs2.HS2_ERR_INVALID_ARG  # FP8 without scales
    assert call(a6=hs2.HS2_FP8_E4M3, a9=FAKE, a10=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a0=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(a7=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a1=-1) == hs2.HS2_ERR_INVALID_ARG
    assert call(a4=16385) == hs2.HS2_ERR_INVALID_ARG          # grid limit
    assert call(a2=2 ** 22) == hs2.HS2_ERR_INVALID_ARG        # 256-row hidden block >= 2 GiB
    # empty work enqueues nothing, even with null buffers
    assert call(a1=0, a0=None, a7=None) == hs2.HS2_OK
    assert call(a4=0, a3=None) == hs2.HS2_OK


def test_block_variant_validation():
    L = hs2.lib()
    E = hs2
    # q, qdt, k, v, ks, vs, kvdt, B, n_q, q_pos0, n_ctx, H, d, block, k_blocks, scale, out, lse, idx, scores, ws,
    # wsb, stream
    sel = [FAKE, 1, FAKE, FAKE, None, None, 1, 1, 100, 0, 100, 16, 128, 64, 16, 0.1, FAKE, FAKE, FAKE, None,
           None, 0, None]

    def call_sel(**kw):
        a = list(sel)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_block_attn_select(*a)

    assert call_sel() == E.HS2_ERR_WORKSPACE
    assert call_sel(a13=32) == E.HS2_ERR_UNSUPPORTED          # block must be 64
    assert call_sel(a14=65) == E.HS2_ERR_UNSUPPORTED          # at most 64 blocks (4096 tokens)
    assert call_sel(a14=0) == E.HS2_ERR_INVALID_ARG
    assert call_sel(a18=None) == E.HS2_ERR_INVALID_ARG
    assert call_sel(a19=MIS) == E.HS2_ERR_INVALID_ARG
    assert call_sel(a8=101) == E.HS2_ERR_INVALID_ARG          # q_pos0 + n_q > n_ctx
    assert hs2.workspace_size(E.OP_BLOCK_ATTN_SELECT, 1, 32768, 32768, 16, 128, 0, 0, 1) >= 32768 * 512 * 8
    # q, qdt, L, k, v, ks, vs, kvdt, B, n_q, q_pos0, n_ctx, H, d, idx, block, k_blocks, window, gates, scale,
    # out, ws, wsb, stream
    sp = [FAKE, 1, 2, FAKE, FAKE, None, None, 1, 1, 100, 0, 100, 16, 128, FAKE, 64, 16, 128, FAKE, 0.1, FAKE,
          None, 0, None]

    def call_sp(**kw):
        a = list(sp)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_block_sparse_attn(*a)

    assert call_sp(a2=0) == E.HS2_OK                          # no layers: nothing enqueued, no workspace needed
    assert call_sp(a18=None) == E.HS2_ERR_INVALID_ARG         # gates
    assert call_sp(a17=0) == E.HS2_ERR_INVALID_ARG            # window
    assert call_sp(a17=5000) == E.HS2_ERR_UNSUPPORTED
    assert call_sp(a15=16) == E.HS2_ERR_UNSUPPORTED
    assert call_sp(a2=-1) == E.HS2_ERR_INVALID_ARG
    assert hs2.workspace_size(E.OP_BLOCK_SPARSE_ATTN, 1, 100, 100, 16, 128, 128, 16, 1) == 0


def test_index_select_validation():
    L = hs2.lib()
    E = hs2
    # qi, qs, w, ki, ks, B, n_q, q_pos0, n_ctx, HI, dI, window, k_global, idx, ws, wsb, stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 100, 0, 100, 8, 128, 128, 1024, FAKE, None, 0, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_index_select(*a)

    assert call() == E.HS2_ERR_WORKSPACE
    assert call(a9=6) == E.HS2_ERR_UNSUPPORTED                # indexer heads
    assert call(a10=96) == E.HS2_ERR_UNSUPPORTED              # indexer head dim
    assert call(a12=4096) == E.HS2_ERR_UNSUPPORTED            # k_global > 2048
    assert call(a11=0) == E.HS2_ERR_INVALID_ARG
    assert call(a1=None) == E.HS2_ERR_INVALID_ARG
    assert call(a3=MIS) == E.HS2_ERR_INVALID_ARG
    assert call(a7=1) == E.HS2_ERR_INVALID_ARG                 # q_pos0 + n_q > n_ctx
    assert hs2.workspace_size(E.OP_INDEX_SELECT, 1, 32768, 32768, 0, 128, 0, 0, 0) >= 32768 * 4096 * 8


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        hs2.select_topk(torch.zeros(2, 10), 3)


def test_batch_limits_of_the_launch_grid():
    """Sequences (and selection rows) ride on a launch's second grid
    dimension: more than 65535 is refused on the host, before any enqueue."""
    L = hs2.lib()
    E = hs2
    big = 65536
    assert _full(B=big, n_q=1, n_ctx=10) == E.HS2_ERR_UNSUPPORTED
    assert _full(B=65535, n_q=1, n_ctx=10) == E.HS2_ERR_WORKSPACE   # the limit itself is accepted
    assert _decode(B=big) == E.HS2_ERR_UNSUPPORTED
    assert _decode(B=65535) == E.HS2_ERR_WORKSPACE
    assert L.hs2_select_topk(FAKE, big, 100, None, 8, FAKE, None, 0, None) == E.HS2_ERR_UNSUPPORTED
    assert L.hs2_select_topk(FAKE, 65535, 100, None, 8, FAKE, None, 0, None) == E.HS2_ERR_WORKSPACE
    idx_args = [FAKE, FAKE, FAKE, FAKE, FAKE, big, 1, 0, 100, 8, 128, 128, 1024, FAKE, None, 0, None]
    assert L.hs2_index_select(*idx_args) == E.HS2_ERR_UNSUPPORTED
    sel = [FAKE, 1, FAKE, FAKE, None, None, 1, big, 1, 0, 100, 16, 128, 64, 16, 0.1, FAKE, FAKE, FAKE, None,
           None, 0, None]
    assert L.hs2_block_attn_select(*sel) == E.HS2_ERR_UNSUPPORTED


def test_sparse_attn_noalloc_validation():
    """The no-allocation variant checks its arguments like hs2_sparse_attn
    (no workspace) before it touches the device."""
    L = hs2.lib()
    E = hs2
    # q, qdt, n_layers, k, v, ks, vs, kvdt, B, n_q, n_ctx, H, d, idx, n_sel, scale, out, lse, stream
    args = [FAKE, 1, 2, FAKE, FAKE, None, None, 1, 64, 1, 5000, 16, 128, FAKE, 1152, 0.1, FAKE, None, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_sparse_attn_noalloc(*a)

    assert call(a14=0) == E.HS2_ERR_INVALID_ARG
    assert call(a14=5000) == E.HS2_ERR_UNSUPPORTED
    assert call(a13=None) == E.HS2_ERR_INVALID_ARG
    assert call(a0=MIS) == E.HS2_ERR_INVALID_ARG
    assert call(a11=12) == E.HS2_ERR_UNSUPPORTED
    assert call(a2=0) == E.HS2_OK              # no layers: nothing enqueued, no device touched


def test_sparse_attn_window_validation():
    L = hs2.lib()
    E = hs2
    # q, qdt, n_layers, k, v, ks, vs, kvdt, B, n_q, q_pos0, n_ctx, H, d, idx, window, k_global, scale, out, lse,
    # ws, wsb, stream
    args = [FAKE, 1, 2, FAKE, FAKE, None, None, 1, 1, 100, 900, 1000, 16, 128, FAKE, 128, 1024, 0.1, FAKE, None,
            None, 0, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_sparse_attn_window(*a)

    assert call() == E.HS2_ERR_WORKSPACE
    assert call(a10=901) == E.HS2_ERR_INVALID_ARG            # q_pos0 + n_q > n_ctx
    assert call(a10=-1) == E.HS2_ERR_INVALID_ARG
    assert call(a15=0) == E.HS2_ERR_INVALID_ARG              # window
    assert call(a16=-1) == E.HS2_ERR_INVALID_ARG
    assert call(a16=4096) == E.HS2_ERR_UNSUPPORTED           # k_global > 2048
    assert call(a14=None) == E.HS2_ERR_INVALID_ARG           # indices needed when k_global > 0
    assert call(a0=MIS) == E.HS2_ERR_INVALID_ARG
    assert call(a1=0, a7=0) == E.HS2_ERR_UNSUPPORTED         # fp32 cache
    assert call(a8=65536) == E.HS2_ERR_UNSUPPORTED           # batch limit
    assert call(a2=0) == E.HS2_ERR_WORKSPACE                 # no layers, but still no workspace


def test_probe_gather_validation():
    L = hs2.lib()
    # src, n_rows, row_bytes, scale, idx, n_idx, sink, sink_words, stream
    args = [FAKE, 1000, 256, None, FAKE, 5000, FAKE, 524288, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_probe_gather(*a)

    assert call(a2=192) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a0=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(a0=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a1=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a7=100) == hs2.HS2_ERR_INVALID_ARG          # sink too small for the grid


def test_probe_mfma_validation():
    L = hs2.lib()
    # waves_per_simd, n_blocks, iters, one, ops, sink, sink_words, stream
    args = [1, 1024, 100, 1.0, None, FAKE, 1024 * 256, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_probe_mfma(*a)

    assert call(a0=3) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a0=0) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a1=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a1=65536) == hs2.HS2_ERR_INVALID_ARG
    assert call(a2=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a2=(1 << 20) + 1) == hs2.HS2_ERR_INVALID_ARG
    assert call(a5=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(a5=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a4=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a6=1024 * 256 - 1) == hs2.HS2_ERR_INVALID_ARG
    assert call(a0=2) == hs2.HS2_ERR_INVALID_ARG            # two waves a SIMD need twice the sink


def test_probe_stream_validation():
    L = hs2.lib()
    # src, src_bytes, dst, dst_bytes, reads_per_write, n_blocks, sink, sink_words, stream
    args = [FAKE, 1 << 20, FAKE, 1 << 17, 8, 64, FAKE, 64 * 256, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.hs2_probe_stream(*a)

    assert call(a0=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(a0=MIS) == hs2.HS2_ERR_INVALID_ARG
    assert call(a1=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a1=4097) == hs2.HS2_ERR_INVALID_ARG          # whole 4 KiB chunks
    assert call(a3=100) == hs2.HS2_ERR_INVALID_ARG
    assert call(a2=None) == hs2.HS2_ERR_INVALID_ARG          # writes need dst
    assert call(a3=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a4=-1) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a4=3) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a4=16) == hs2.HS2_ERR_UNSUPPORTED
    assert call(a3=1 << 32) == hs2.HS2_ERR_INVALID_ARG
    assert call(a5=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(a5=65537) == hs2.HS2_ERR_INVALID_ARG
    assert call(a6=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(a7=64 * 256 - 1) == hs2.HS2_ERR_INVALID_ARG  # sink too small for the grid
