"""GPU parity of the KV Bridging projections (hs2_kv_project) against the CPU
oracle, through the C ABI.

Two kinds of inputs:
  * exact: integer hidden values and weights k/16, so the fp32 accumulation is
    exact in any order; the bf16 outputs, FP8 codes and scales must then be
    bit-identical to the oracle's (its quantiser decides in fp32 too).
  * Gaussian (the realistic case): outputs within the bound the arithmetic
    gives. The kernel's fp32 sum of `hidden` exact bf16 products differs from
    the exact sum by at most gamma = hidden * 2^-24 * sum|w_c h_c| (standard
    recursive-summation bound, any order); bf16 rounding adds 2^-8 |x|.
    FP8: the kernel's code must lie between the oracle's codes for
    t -/+ dt, where dt covers gamma on x and on the row maximum.
"""
import sys

import numpy as np
import pytest
import torch

from hs2_inputs import make_projection_inputs

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


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


def _run(hs2, h, w, fp8):
    dt = hs2.HS2_FP8_E4M3 if fp8 else hs2.HS2_BF16
    r = hs2.kv_project(h.cuda(), w.cuda(), dt)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in r.items()}


def _kernel_rows(r, rows, fp8):
    """[J][2][n][d] outputs (bf16 as float64, or codes) and [J][2][n] scales."""
    k, v = r["k"][:, rows], r["v"][:, rows]
    out = torch.stack([k, v], dim=1)
    if not fp8:
        return out.double().numpy(), None
    sc = torch.stack([r["k_scale"][:, rows], r["v_scale"][:, rows]], dim=1).double().numpy()
    return out.numpy(), sc


def _gamma(h, w, rows):
    """hidden * 2^-24 * sum_c |w[j][kv][e][c] h[t][c]| per output, [J][2][n][d]."""
    ha = h[rows].double().abs().numpy()                       # [n][hidden]
    wa = w.double().abs().numpy()                              # [J][2][d][hidden]
    J, two, d, hidden = wa.shape
    s = (wa.reshape(-1, hidden) @ ha.T).reshape(J, two, d, len(rows)).transpose(0, 1, 3, 2)
    return hidden * U32 * s * 1.0001


def _e4m3(t):
    """RNE cast of fp64 values (exact fp32 or not) via torch, saturating."""
    x = torch.from_numpy(np.asarray(t, np.float64)).clamp(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def check_exact(orc, hs2, h, w, rows, fp8):
    got = _run(hs2, h, w, fp8)
    ref = orc.kv_project(h, w, rows, quantize=fp8)
    g, gs = _kernel_rows(got, rows, fp8)
    if fp8:
        assert np.array_equal(g, ref["codes"])
        assert np.array_equal(gs, ref["scales"])
    else:
        want = torch.from_numpy(ref["x"]).to(torch.bfloat16).double().numpy()
        assert np.array_equal(g, want)


def check_gauss(orc, hs2, h, w, rows, fp8, got=None):
    got = _run(hs2, h, w, fp8) if got is None else got
    ref = orc.kv_project(h, w, rows, quantize=fp8)
    x = ref["x"]
    gam = _gamma(h, w, rows)
    g, gs = _kernel_rows(got, rows, fp8)
    if not fp8:
        err = np.abs(g - x)
        bound = 2.0 ** -8 * (np.abs(x) + gam) + gam
        assert (err <= bound).all(), f"max excess {np.max(err - bound)}"
        return
    # The kernel's row maximum is within G = max_e gamma_e of the exact one, so
    # its scale fl32(amax_k / 448) is within G/448 plus three fp32 roundings.
    sref = ref["scales"]
    G = gam.max(axis=-1)
    ds = G / 448.0 + 3 * U32 * sref
    assert (np.abs(gs - sref) <= ds).all()
    # t_k = fl32(x_k / s_k) with |x_k - x| <= gamma and |s_k - s| <= ds:
    # |t_k - x/s| <= (gamma + |t| ds) / (s - ds) + 2^-24 |t|
    t = x / sref[..., None]
    dt = (gam + np.abs(t) * ds[..., None]) / (sref - ds)[..., None] + 2 * U32 * np.abs(t) + 1e-12
    lo, hi = _dec(_e4m3(t - dt)), _dec(_e4m3(t + dt))
    gv = _dec(g)
    assert ((gv >= lo) & (gv <= hi)).all()
    same = np.mean(g == ref["codes"])
    assert same > 0.99, f"only {same:.4f} of codes equal the oracle's"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("T,hidden,J", [(1000, 2048, 3), (257, 96, 1), (1, 32, 2), (512, 64, 2), (200, 192, 1),
                                         (700, 256, 2), (300, 128, 4), (513, 384, 1), (520, 2048, 8)])
def test_kv_project_exact(hs2, orc, d, fp8, T, hidden, J):
    say("kv_project exact T", T, "hidden", hidden, "J", J, "d", d, "fp8", fp8)
    zero = (0, T - 1) if T > 2 else ()
    h, w = make_projection_inputs(7 + T + hidden, T, hidden, J, d, exact=True, zero_rows=zero)
    check_exact(orc, hs2, h, w, list(range(T)), fp8)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("T,hidden,J", [(1000, 2048, 3), (300, 160, 2)])
def test_kv_project_gaussian(hs2, orc, d, fp8, T, hidden, J):
    say("kv_project gaussian T", T, "hidden", hidden, "J", J, "d", d, "fp8", fp8)
    h, w = make_projection_inputs(3 * T + hidden + d, T, hidden, J, d, zero_rows=(5,))
    check_gauss(orc, hs2, h, w, list(range(T)), fp8)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_kv_project_full_size_sampled(hs2, orc, fp8):
    """The bench's shape: a 32k-token prefill chunk, hidden 2048, four bridged
    layers, d = 128; 256 sampled rows (the first and last, both sides of every
    fourth 256-token block boundary, the rest seeded)."""
    T, hidden, J, d = 32768, 2048, 4, 128
    say("kv_project full size T", T, "hidden", hidden, "J", J, "fp8", fp8)
    h, w = make_projection_inputs(2024, T, hidden, J, d)
    rng = np.random.default_rng(99)
    rows = {0, T - 1}
    for b in range(256, T, 1024):
        rows |= {b - 1, b}
    rows |= set(rng.choice(T, 256 - len(rows), replace=False).tolist())
    rows = sorted(rows)[:256]
    check_gauss(orc, hs2, h, w, rows, fp8)
