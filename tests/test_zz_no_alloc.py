"""hs2_sparse_attn_noalloc (the sparse layers without a caller workspace,
for callers that cannot allocate) against hs2_sparse_attn through the C ABI:
the same kernels, so the outputs and LSEs must be bit-identical, and both
within the parity tolerance of the oracle. Two calls in a row on the
library's per-GPU scratch array, the second with a smaller input (the first
call's partials are still in the array), then a shape with no split."""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_inputs, workload
from tests.hs2_check import lse_close, rows_close

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hs2():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import token_level_top_amd as t
    t.lib()
    return t


def _case(hs2, orc, cfg, n_q, n_ctx, n_sel, seed):
    wl = workload(cfg).with_(B=1, n_q=n_q, q_pos0=n_ctx - n_q, n_ctx=n_ctx, n_needles=0, needles="none",
                             n_sparse=2)
    x = make_inputs(wl)
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, n_sel), -1, np.int32)
    for t in range(n_q):
        m = int(rng.integers(1, n_sel + 1))
        idx[t, :m] = np.sort(rng.choice(n_ctx, size=m, replace=False))
    kv = [t.cuda().contiguous() if t is not None else None for t in (x.k, x.v, x.k_scale, x.v_scale)]
    q = x.q_sparse.cuda().contiguous()
    gi = torch.from_numpy(idx).reshape(1, n_q, n_sel).cuda()
    say("no-alloc sparse", wl.name, "tokens", n_q, "n_sel", n_sel,
        "scratch bytes", hs2.workspace_size(hs2.OP_SPARSE_ATTN, 1, n_q, n_ctx, wl.H, wl.d, n_sel, 0,
                                            hs2._KVDT[x.k.dtype]))
    o_na, l_na = hs2.sparse_attn_noalloc(q, *kv, indices=gi, sm_scale=x.sm_scale)
    o_ws, l_ws = hs2.sparse_attn(q, *kv, indices=gi, sm_scale=x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), "no-alloc result differs from hs2_sparse_attn"
    rows = list(range(n_q))
    for l in range(2):
        r = orc.sparse(x.q_sparse[l].contiguous(), x.k, x.v, x.k_scale, x.v_scale, idx, x.sm_scale, rows)
        rows_close(o_na[l, 0], r["out"], RTOL[wl.kv_dtype], f"no-alloc layer {l} out")
        lse_close(l_na[l, 0], r["lse"], RTOL[wl.kv_dtype], f"no-alloc layer {l} lse")


def test_noalloc_matches_workspace_entry_twice_then_smaller(hs2, orc):
    _case(hs2, orc, 2, 64, 20000, 1152, 1)     # 64 tokens x 5 splits of partials (2.7 MB)
    _case(hs2, orc, 4, 7, 6000, 800, 2)        # smaller, FP8 cache, on the same array
    _case(hs2, orc, 1, 3, 3000, 384, 3)        # fp32, H = 4, d = 64
    _case(hs2, orc, 2, 1100, 3000, 300, 4)     # no split: the array is not used
