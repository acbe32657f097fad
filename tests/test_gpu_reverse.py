"""Workgroup-order independence: every entry point run with its kernels'
grids dealt in the usual order and in reverse (hs2_test_reverse_grid) must give
bit-identical results. A result that depended on which workgroups run first
or together (a race between workgroups through memory, an atomic whose order
leaks into an output, an LDS hazard exposed by different co-residency) would
differ. Every output is compared with torch.equal."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_gates, make_indexer_inputs, make_inputs, make_projection_inputs, workload

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
    yield t
    t.set_reverse_grid(False)


def dev(x):
    return None if x is None else x.cuda().contiguous()


def both_orders(hs2, fn):
    """fn() -> tuple/dict of tensors, run in the usual and the reversed order."""
    hs2.set_reverse_grid(False)
    a = fn()
    torch.cuda.synchronize()
    hs2.set_reverse_grid(True)
    try:
        b = fn()
        torch.cuda.synchronize()
    finally:
        hs2.set_reverse_grid(False)
    if isinstance(a, dict):
        a, b = [a[k] for k in sorted(a)], [b[k] for k in sorted(b)]
    for i, (u, v) in enumerate(zip(a, b)):
        if u is None:
            continue
        assert torch.equal(u, v), f"output {i} differs with the workgroup order reversed"


@pytest.mark.parametrize("cfg,n_q,q_pos0,n_ctx", [(2, 1500, 0, 1500), (4, 300, 2700, 3000), (1, 700, 0, 700)])
def test_full_attn_select_and_sparse(hs2, cfg, n_q, q_pos0, n_ctx):
    wl = workload(cfg).with_(n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=2)
    x = make_inputs(wl)
    kg = min(wl.k_global, 256)
    say("reverse grid: full + sparse", wl.name, n_q, n_ctx)
    full = lambda: hs2.full_attn_select(dev(x.q), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                        q_pos0=q_pos0, window=wl.window, k_global=kg, sm_scale=x.sm_scale)
    both_orders(hs2, full)
    _, _, idx = full()
    # many tokens (one workgroup a token) and few tokens (rows split, then combined)
    both_orders(hs2, lambda: hs2.sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale),
                                             indices=idx, sm_scale=x.sm_scale))
    few = idx[:, :3].contiguous()
    both_orders(hs2, lambda: hs2.sparse_attn(dev(x.q_sparse[:, :, :3]), dev(x.k), dev(x.v), dev(x.k_scale),
                                             dev(x.v_scale), indices=few, sm_scale=x.sm_scale))


@pytest.mark.parametrize("cfg", [3, 5])
def test_decode_step(hs2, cfg):
    wl = workload(cfg).with_(B=4, n_ctx=50000, q_pos0=49999, n_needles=4, n_sparse=2)
    x = make_inputs(wl)
    say("reverse grid: decode", wl.name)
    both_orders(hs2, lambda: hs2.decode_step(dev(x.q[:, 0]), dev(x.q_sparse[:, :, 0]), dev(x.k), dev(x.v),
                                             dev(x.k_scale), dev(x.v_scale), window=wl.window,
                                             k_global=wl.k_global, sm_scale=x.sm_scale, want_scores=True))


def test_select_topk(hs2):
    g = torch.Generator(device="cuda").manual_seed(4)
    scores = torch.rand((6, 70000), device="cuda", generator=g)
    scores[2, :5000] = 0.5  # a block of ties
    say("reverse grid: select_topk")
    both_orders(hs2, lambda: (hs2.select_topk(scores, 1024),))


@pytest.mark.parametrize("fp8", [False, True])
def test_kv_project(hs2, fp8):
    h, w = make_projection_inputs(5, 1000, 2048, 4, 128)
    dt = hs2.HS2_FP8_E4M3 if fp8 else hs2.HS2_BF16
    say("reverse grid: kv_project", fp8)
    both_orders(hs2, lambda: hs2.kv_project(dev(h), dev(w), dt))


def test_block_variant(hs2):
    wl = workload(2).with_(n_q=1200, n_ctx=1200, q_pos0=0, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    say("reverse grid: block variant")
    sel = lambda: hs2.block_attn_select(dev(x.q), dev(x.k), dev(x.v), q_pos0=0, k_blocks=16, sm_scale=x.sm_scale,
                                        want_scores=True)
    # block scores are specified for the blocks at or before the query's
    # position only (the rest of the row is left unwritten)
    n_blk = (wl.n_ctx + 63) // 64
    causal = (torch.arange(n_blk, device="cuda")[None, :] * 64 <= torch.arange(wl.n_q, device="cuda")[:, None])

    def sel_causal():
        out, lse, bidx, bsc = sel()
        return out, lse, bidx, bsc[0][causal]

    both_orders(hs2, sel_causal)
    _, _, bidx, _ = sel()
    gates = dev(make_gates(7, (2, 1, wl.n_q, wl.H, 2)))
    both_orders(hs2, lambda: (hs2.block_sparse_attn(dev(x.q_sparse), dev(x.k), dev(x.v), block_idx=bidx, q_pos0=0,
                                                    window=128, gates=gates, sm_scale=x.sm_scale),))


@pytest.mark.parametrize("cfg,n_q,q_pos0,n_ctx", [(2, 1100, 900, 2000), (4, 300, 2700, 3000)])
def test_window_sharing(hs2, cfg, n_q, q_pos0, n_ctx):
    wl = workload(cfg).with_(n_q=n_q, q_pos0=q_pos0, n_ctx=n_ctx, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    kv = (dev(x.k), dev(x.v), dev(x.k_scale), dev(x.v_scale))
    _, _, idx = hs2.full_attn_select(dev(x.q), *kv, q_pos0=q_pos0, window=wl.window, k_global=wl.k_global,
                                     sm_scale=x.sm_scale)
    say("reverse grid: window sharing", wl.name, n_q)
    both_orders(hs2, lambda: hs2.sparse_attn_window(dev(x.q_sparse), *kv, indices=idx, q_pos0=q_pos0,
                                                    window=wl.window, sm_scale=x.sm_scale))


@pytest.mark.parametrize("B,n_q,q_pos0,n_ctx,HI,dI,kg", [
    (1, 600, 2400, 3000, 8, 64, 1024),      # threshold histograms
    (2, 20, 66000, 66020, 16, 128, 2048),   # 64 Ki candidates or more: superset trims
])
def test_index_select(hs2, B, n_q, q_pos0, n_ctx, HI, dI, kg):
    x = make_indexer_inputs(11, B, n_q, q_pos0, n_ctx, HI, dI, n_needles=4)
    say("reverse grid: light indexer", B, n_q, n_ctx, HI, kg)
    both_orders(hs2, lambda: (hs2.index_select(x.qi.cuda(), x.qs.cuda(), x.w.cuda(), x.ki.cuda(), x.ks.cuda(),
                                               q_pos0=q_pos0, window=128, k_global=kg),))
