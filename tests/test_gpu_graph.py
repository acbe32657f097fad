"""A decode step captured in a HIP graph and replayed: the library allocates
nothing, synchronises nothing and clears its scratch with kernels, so every
replay must reproduce the eager results bit for bit (the step is
deterministic). Replays alternate with unrelated eager work and with the
output buffers overwritten, so a replay that skipped or reused stale work
would show."""
import sys

import pytest
import torch

from hs2_inputs import make_inputs, workload

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


@pytest.mark.parametrize("cfg", [3, 5])
def test_decode_step_graph_replays_match_eager(hs2, cfg):
    wl = workload(cfg).with_(B=4, n_ctx=20000, q_pos0=19999, n_needles=2, n_sparse=2)
    x = make_inputs(wl)
    say("graph replay", wl.name, wl.B, wl.n_ctx)
    dev = torch.device("cuda")
    g = lambda t: None if t is None else t.to(dev).contiguous()
    k, v, ks, vs = g(x.k), g(x.v), g(x.k_scale), g(x.v_scale)
    qf, qs = g(x.q[:, 0]), g(x.q_sparse[:, :, 0])
    S = wl.window + wl.k_global
    kvdt = {"bf16": hs2.HS2_BF16, "fp8": hs2.HS2_FP8_E4M3}[wl.kv_dtype]
    ws = torch.empty(hs2.workspace_size(hs2.OP_DECODE_STEP, wl.B, 1, wl.n_ctx, wl.H, wl.d, wl.window, wl.k_global,
                                        kvdt), dtype=torch.uint8, device=dev)
    bufs = dict(out_full=torch.empty_like(qf), lse_full=torch.empty((wl.B, wl.H), device=dev),
                out_sparse=torch.empty_like(qs), lse_sparse=torch.empty((wl.n_sparse, wl.B, wl.H), device=dev),
                indices=torch.empty((wl.B, S), dtype=torch.int32, device=dev),
                scores=torch.empty((wl.B, wl.n_ctx), device=dev))

    def step():
        hs2.decode_step(qf, qs, k, v, ks, vs, window=wl.window, k_global=wl.k_global, sm_scale=x.sm_scale,
                        want_scores=True, workspace=ws, **bufs)

    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in bufs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for t in bufs.values():          # stale results must not survive a replay
            t.fill_(-7)
        ws.fill_(0xAB)
        junk.mul_(1.0001)                # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for n, t in bufs.items():
            assert torch.equal(t, ref[n]), f"replay {rep}: {n} differs from the eager step"
