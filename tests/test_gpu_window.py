"""GPU parity of the window-sharing sparse layers (hs2_sparse_attn_window)
against the CPU oracle, through the C ABI.

The index rows come from the GPU's own full layer (hs2_full_attn_select), as
in a model; the oracle's sparse attention over those rows (window part and
global part together, one softmax) is the reference: rel 1e-2 on outputs per
(token, head) row and 1e-2 absolute on the LSE (bf16 / FP8). The window part
of an index row must not be read: rows whose window entries are overwritten
with junk give identical results."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import checked_rows, make_inputs, workload
from tests.hs2_check import lse_close, rows_close, to_np

pytestmark = pytest.mark.gpu

RTOL = {"bf16": 1e-2, "fp8": 1e-2}


def say(*a):
    print("[gpu-window]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import token_level_top_amd as t
    t.lib()
    return t


def g(t):
    return None if t is None else t.cuda().contiguous()


def _run(hs2, orc, wl, rows=None, junk_window=True):
    x = make_inputs(wl)
    kv = (g(x.k), g(x.v), g(x.k_scale), g(x.v_scale))
    _, _, idx = hs2.full_attn_select(g(x.q), *kv, q_pos0=wl.q_pos0, window=wl.window, k_global=wl.k_global,
                                     sm_scale=x.sm_scale)
    out, lse = hs2.sparse_attn_window(g(x.q_sparse), *kv, indices=idx, q_pos0=wl.q_pos0, window=wl.window,
                                      sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    n_tok = wl.B * wl.n_q
    rows = list(range(n_tok)) if rows is None else rows
    ri = torch.tensor(rows)
    gidx = to_np(idx.reshape(n_tok, -1)[ri]).astype(np.int32)
    tol = RTOL[wl.kv_dtype]
    for l in range(wl.n_sparse):
        r = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, gidx, x.sm_scale, rows)
        rows_close(out[l].reshape(n_tok, wl.H, wl.d)[ri], r["out"], tol, f"window-shared layer {l} out")
        lse_close(lse[l].reshape(n_tok, wl.H)[ri], r["lse"], tol, f"window-shared layer {l} lse")
    if junk_window:
        bad = idx.clone()
        bad[..., :wl.window] = torch.randint(-5, wl.n_ctx + 5, bad[..., :wl.window].shape, dtype=torch.int32,
                                             device=bad.device)
        o2, l2 = hs2.sparse_attn_window(g(x.q_sparse), *kv, indices=bad, q_pos0=wl.q_pos0, window=wl.window,
                                        sm_scale=x.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, out) and torch.equal(l2, lse), "the window part of the index rows was read"
    return x, idx, out, lse


@pytest.mark.parametrize("cfg,B,H,d,n_q,q_pos0,n_ctx,kg", [
    (2, 1, 16, 128, 300, 1000, 1300, 1024),   # bf16, ragged query blocks
    (2, 2, 16, 128, 200, 0, 200, 1024),       # two sequences from position 0: windows shorter than 128
    (2, 1, 8, 64, 500, 4000, 4500, 1024),     # H = 8, d = 64
    (4, 1, 16, 128, 77, 5000, 5077, 1024),    # FP8 cache, block starts not aligned to 64
    (4, 2, 4, 128, 160, 5000, 5160, 512),     # FP8, H = 4 (64 tokens per block), two sequences
    (2, 1, 16, 128, 130, 3000, 3130, 0),      # no global part: the window alone
])
def test_window_shared_matches_oracle(hs2, orc, cfg, B, H, d, n_q, q_pos0, n_ctx, kg):
    wl = workload(cfg).with_(B=B, H=H, d=d, n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, k_global=kg, n_needles=2,
                             n_sparse=2)
    say("window-shared sparse", wl.name, B, H, d, n_q, q_pos0, n_ctx, kg)
    _run(hs2, orc, wl)


@pytest.mark.parametrize("cfg,B,n_ctx", [(3, 3, 5003), (5, 2, 9000)])
def test_window_shared_few_tokens_split_path(hs2, orc, cfg, B, n_ctx):
    """One query per sequence (decode shape): the global part is split over
    workgroups and the window's record joins the combine."""
    wl = workload(cfg).with_(B=B, n_q=1, q_pos0=n_ctx - 1, n_ctx=n_ctx, n_sparse=2, needles="decode",
                             n_needles=4, decode=False)
    say("window-shared sparse, few tokens", wl.name, B, n_ctx)
    _run(hs2, orc, wl)


def test_window_shared_matches_gather_everything(hs2):
    """Against hs2_sparse_attn over the same full index rows (window gathered
    like any row): the same softmax, evaluated in another order."""
    wl = workload(4).with_(n_q=256, q_pos0=6000, n_ctx=6256, n_needles=2, n_sparse=1)
    x = make_inputs(wl)
    kv = (g(x.k), g(x.v), g(x.k_scale), g(x.v_scale))
    _, _, idx = hs2.full_attn_select(g(x.q), *kv, q_pos0=wl.q_pos0, window=128, k_global=1024, sm_scale=x.sm_scale)
    o1, l1 = hs2.sparse_attn_window(g(x.q_sparse), *kv, indices=idx, q_pos0=wl.q_pos0, window=128,
                                    sm_scale=x.sm_scale)
    o2, l2 = hs2.sparse_attn(g(x.q_sparse), *kv, indices=idx, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    rows_close(o1.reshape(-1, wl.H, wl.d), to_np(o2.reshape(-1, wl.H, wl.d)), 1e-2, "window-shared vs gathered out")
    lse_close(l1.reshape(-1, wl.H), to_np(l2.reshape(-1, wl.H)), 1e-3, "window-shared vs gathered lse")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_uniform,n_target", [(2, 256, None), (4, 480, 32)])
def test_window_shared_full_size(hs2, orc, cfg, n_uniform, n_target):
    """The 32k prefill and the 8k-at-256k chunked prefill at full size, every
    sparse layer, on the 512 seeded rows of each workload."""
    wl = workload(cfg)
    x0 = make_inputs(wl)
    needles = x0.needles if n_target is None else x0.needles[:n_target]
    rows = checked_rows(wl, needles, n_uniform)
    del x0
    say("window-shared sparse at full size", wl.name, len(rows), "rows checked")
    _run(hs2, orc, wl, rows=rows, junk_window=False)
