"""Guard bands around every output and workspace buffer.

Each buffer the library writes (outputs, LSE, index rows, score vectors and
the workspace) is carved out of a larger allocation whose bytes before and
after it hold a sentinel pattern; after the call the bands must be intact, so
a kernel writing past its buffer's end (or before its start) is caught even
where the stray write would not change a compared value. Results inside the
buffers are also checked against the same call on plain allocations."""
import sys

import numpy as np
import pytest
import torch

import token_level_top_amd as hs2_mod
from hs2_inputs import make_inputs, workload

pytestmark = pytest.mark.gpu

BAND = 4096      # guard bytes on each side (a multiple of 256 keeps alignment)
SENT = 0xA5


def say(*a):
    print("[gpu-canary]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    hs2_mod.lib()
    return hs2_mod


class Guarded:
    """A device buffer of `shape`/`dtype` (or `nbytes` raw bytes) with
    sentinel-filled guard bands on both sides."""

    def __init__(self, shape=None, dtype=torch.uint8, nbytes=None):
        esz = torch.tensor([], dtype=dtype).element_size()
        n = nbytes if nbytes is not None else int(np.prod(shape)) * esz
        self.n = (n + 255) // 256 * 256
        self.raw = torch.full((BAND + self.n + BAND,), SENT, dtype=torch.uint8, device="cuda")
        inner = self.raw[BAND:BAND + self.n]
        if nbytes is not None:
            self.t = inner
        else:
            self.t = inner[:n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        lo = self.raw[:BAND].cpu().numpy()
        hi = self.raw[BAND + self.n:].cpu().numpy()
        bad_lo = np.nonzero(lo != SENT)[0]
        bad_hi = np.nonzero(hi != SENT)[0]
        assert len(bad_lo) == 0, f"{what}: {len(bad_lo)} bytes written before the buffer (offsets {bad_lo[-4:] - BAND})"
        assert len(bad_hi) == 0, f"{what}: {len(bad_hi)} bytes written past the end (offsets {bad_hi[:4]})"


def g(t):
    return None if t is None else t.cuda().contiguous()


@pytest.mark.parametrize("cfg,n_q,q_pos0,n_ctx", [(2, 300, 1000, 1300), (4, 77, 5000, 5077), (1, 200, 0, 200)])
def test_prefill_guard_bands(hs2, cfg, n_q, q_pos0, n_ctx):
    wl = workload(cfg).with_(n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    say("prefill guard bands", wl.name, n_q, q_pos0, n_ctx)
    B, H, d, S = 1, wl.H, wl.d, wl.n_sel
    kv = (g(x.k), g(x.v), g(x.k_scale), g(x.v_scale))
    kw = dict(q_pos0=q_pos0, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale)
    kvdt = hs2._KVDT[x.k.dtype]
    out = Guarded((B, n_q, H, d), x.q.dtype)
    lse = Guarded((B, n_q, H), torch.float32)
    idx = Guarded((B, n_q, S), torch.int32)
    ws = Guarded(nbytes=hs2.workspace_size(hs2.OP_FULL_ATTN_SELECT, B, n_q, n_ctx, H, d, wl.window, wl.k_global,
                                           kvdt))
    hs2.full_attn_select(g(x.q), *kv, out=out.t, lse=lse.t, indices=idx.t, workspace=ws.t, **kw)
    for b, what in ((out, "out"), (lse, "lse"), (idx, "indices"), (ws, "workspace")):
        b.check(what)
    ref_o, ref_l, ref_i = hs2.full_attn_select(g(x.q), *kv, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.t, ref_o) and torch.equal(lse.t, ref_l) and torch.equal(idx.t, ref_i)
    # the sparse layers over those rows
    so = Guarded((2, B, n_q, H, d), x.q.dtype)
    sl = Guarded((2, B, n_q, H), torch.float32)
    sws = Guarded(nbytes=max(256, hs2.workspace_size(hs2.OP_SPARSE_ATTN, B, n_q, n_ctx, H, d, S, 0, kvdt)))
    hs2.sparse_attn(g(x.q_sparse), *kv, indices=idx.t, sm_scale=x.sm_scale, out=so.t, lse=sl.t, workspace=sws.t)
    for b, what in ((so, "sparse out"), (sl, "sparse lse"), (sws, "sparse workspace")):
        b.check(what)
    say("  bands intact")


@pytest.mark.parametrize("cfg,B,n_ctx,n_sparse", [(3, 3, 5003, 2), (5, 2, 9000, 3), (1, 2, 4099, 1)])
def test_decode_guard_bands(hs2, cfg, B, n_ctx, n_sparse):
    wl = workload(cfg).with_(B=B, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=n_sparse, n_needles=4,
                             needles="decode", decode=True)
    x = make_inputs(wl)
    say("decode guard bands", wl.name, B, n_ctx)
    H, d, S = wl.H, wl.d, wl.n_sel
    kvdt = hs2._KVDT[x.k.dtype]
    qdt = x.q.dtype
    bufs = {
        "out_full": Guarded((B, H, d), qdt), "lse_full": Guarded((B, H), torch.float32),
        "out_sparse": Guarded((n_sparse, B, H, d), qdt), "lse_sparse": Guarded((n_sparse, B, H), torch.float32),
        "indices": Guarded((B, S), torch.int32), "scores": Guarded((B, n_ctx), torch.float32),
        "workspace": Guarded(nbytes=hs2.workspace_size(hs2.OP_DECODE_STEP, B, 1, n_ctx, H, d, wl.window,
                                                       wl.k_global, kvdt)),
    }
    args = (g(x.q[:, 0]), g(x.q_sparse[:, :, 0]), g(x.k), g(x.v), g(x.k_scale), g(x.v_scale))
    kw = dict(window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale, want_scores=True)
    hs2.decode_step(*args, **kw, **{k: b.t for k, b in bufs.items()})
    for k, b in bufs.items():
        b.check(k)
    ref = hs2.decode_step(*args, **kw)
    torch.cuda.synchronize()
    for k in ("out_full", "lse_full", "out_sparse", "lse_sparse", "indices", "scores"):
        assert torch.equal(bufs[k].t, ref[k]), k
    say("  bands intact")


def test_select_and_index_guard_bands(hs2):
    rng = np.random.default_rng(5)
    rows, L, k = 5, 20000, 1024
    sc = torch.from_numpy(rng.random((rows, L), dtype=np.float32)).cuda()
    out = Guarded((rows, k), torch.int32)
    ws = Guarded(nbytes=hs2.workspace_size(hs2.OP_SELECT_TOPK, rows, 0, L, 0, 0, 0, k, 0))
    hs2.select_topk(sc, k, out=out.t, workspace=ws.t)
    out.check("select out")
    ws.check("select workspace")
    from hs2_inputs import make_indexer_inputs
    B, n_q, q_pos0, n_ctx, HI, dI = 1, 100, 5000, 5100, 8, 64
    xi = make_indexer_inputs(3, B, n_q, q_pos0, n_ctx, HI, dI)
    idx = Guarded((B, n_q, 128 + 1024), torch.int32)
    iws = Guarded(nbytes=hs2.workspace_size(hs2.OP_INDEX_SELECT, B, n_q, n_ctx, 0, dI, 0, 0, 0))
    hs2.index_select(xi.qi.cuda(), xi.qs.cuda(), xi.w.cuda(), xi.ki.cuda(), xi.ks.cuda(), q_pos0=q_pos0, window=128,
                     k_global=1024, indices=idx.t, workspace=iws.t)
    idx.check("indexer indices")
    iws.check("indexer workspace")
    say("  bands intact")
