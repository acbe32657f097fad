"""Pins for the CPU oracle: each check is fixed by mathematics, a library
routine, brute force or a hand-derived example, never by the oracle itself.

The method is defined on the HySparse2 page (sections "어떻게 동작하나",
"무엇과 다른가", "어떻게 쓰나") and, for the head-aggregated attention
distribution and the per-query top-k set, on the IndexCache page, section 3
("표기법"). The readings taken where the pages are silent (head sum, 1/sqrt(d)
scale, window includes the query token, ties to the lower position, ascending
index rows, -1 padding) are the ones the oracle's header lists.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from hs2_inputs import make_inputs, quantize_e4m3, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cache(x):
    """[n][d] float tensor -> [1][n][d] contiguous float32"""
    return x.to(torch.float32).reshape(1, *x.shape).contiguous()


def _full(orc, q, k, v, q_pos0=0, window=4, k_global=3, sm_scale=None, rows=None, scores=True,
          ks=None, vs=None):
    B, n_q, H, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if rows is None:
        rows = list(range(B * n_q))
    return orc.full_select(q.contiguous(), k.contiguous(), v.contiguous(), ks, vs, q_pos0, window,
                           k_global, sm_scale, rows, want_scores=scores)


def _sdpa64(q, k, v, mask, sm_scale):
    """float64 torch SDPA, q [n][H][d], k/v [m][d], mask [n][m] bool (True = attend)."""
    qh = q.to(torch.float64).permute(1, 0, 2)                # [H][n][d]
    kk = k.to(torch.float64).unsqueeze(0).expand(qh.shape[0], -1, -1)
    vv = v.to(torch.float64).unsqueeze(0).expand(qh.shape[0], -1, -1)
    o = F.scaled_dot_product_attention(qh, kk, vv, attn_mask=mask.unsqueeze(0), scale=sm_scale)
    logits = torch.matmul(qh, kk.transpose(1, 2)) * sm_scale
    logits = logits.masked_fill(~mask.unsqueeze(0), float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)                     # [H][n]
    return o.permute(1, 0, 2).numpy(), lse.T.numpy()


# ---------------------------------------------------------------- golden ----

def test_golden_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    n, H = g["inputs"]["n"], g["inputs"]["H"]
    q = torch.zeros(1, n, H, 1)
    q[..., 0, 0] = 1.0
    q[..., 1, 0] = -1.0
    k = torch.tensor([math.log(j + 1) for j in range(n)], dtype=torch.float32).reshape(1, n, 1)
    v = torch.arange(n, dtype=torch.float32).reshape(1, n, 1)
    r = _full(orc, q, k, v, window=g["inputs"]["window"], k_global=g["inputs"]["k_global"],
              sm_scale=g["inputs"]["sm_scale"])
    e = g["expected"]
    np.testing.assert_allclose(r["lse"], np.array(e["lse"]), atol=1e-6)
    np.testing.assert_allclose(r["out"][:, :, 0], np.array(e["out"]), atol=1e-6)
    np.testing.assert_allclose(r["scores"][3], np.array(e["scores_p3"]), atol=1e-6)
    np.testing.assert_allclose(r["scores"][2][:3], np.array(e["scores_p2"]), atol=1e-6)
    assert r["idx"].tolist() == e["idx"]


# ----------------------------------------------------- library cross-check ----

@pytest.mark.parametrize("n_q,q_pos0,n_ctx,H,d,dt", [
    (40, 0, 40, 4, 64, torch.float32),
    (33, 20, 53, 16, 128, torch.bfloat16),
    (17, 3, 70, 8, 64, torch.bfloat16),
])
def test_full_attention_matches_torch_sdpa_f64(orc, n_q, q_pos0, n_ctx, H, d, dt):
    g = torch.Generator().manual_seed(n_q * 1000 + n_ctx)
    q = torch.randn(1, n_q, H, d, generator=g).to(dt)
    k = torch.randn(1, n_ctx, d, generator=g).to(dt)
    v = torch.randn(1, n_ctx, d, generator=g).to(dt)
    sm = 1.0 / math.sqrt(d)
    r = _full(orc, q, k, v, q_pos0=q_pos0, sm_scale=sm, scores=False)
    pos = torch.arange(n_q) + q_pos0
    mask = torch.arange(n_ctx).unsqueeze(0) <= pos.unsqueeze(1)
    o_ref, lse_ref = _sdpa64(q[0], k[0], v[0], mask, sm)
    np.testing.assert_allclose(r["out"], o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)


def test_fp8_cache_matches_sdpa_on_dequantised_values(orc):
    g = torch.Generator().manual_seed(7)
    n_ctx, H, d = 50, 4, 64
    q = torch.randn(1, n_ctx, H, d, generator=g).to(torch.bfloat16)
    k32 = torch.randn(1, n_ctx, d, generator=g) * 3
    v32 = torch.randn(1, n_ctx, d, generator=g)
    kc, ks = quantize_e4m3(k32)
    vc, vs = quantize_e4m3(v32)
    kd = kc.view(torch.float8_e4m3fn).to(torch.float64) * ks.to(torch.float64).unsqueeze(-1)
    vd = vc.view(torch.float8_e4m3fn).to(torch.float64) * vs.to(torch.float64).unsqueeze(-1)
    sm = 1.0 / math.sqrt(d)
    r = _full(orc, q, kc, vc, ks=ks, vs=vs, sm_scale=sm, scores=False)
    mask = torch.arange(n_ctx).unsqueeze(0) <= torch.arange(n_ctx).unsqueeze(1)
    o_ref, lse_ref = _sdpa64(q[0], kd[0], vd[0], mask, sm)
    np.testing.assert_allclose(r["out"], o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ closed forms ----

def test_zero_query_gives_uniform_attention(orc):
    n, H, d = 30, 4, 8
    g = torch.Generator().manual_seed(1)
    q = torch.zeros(1, n, H, d)
    k = torch.randn(1, n, d, generator=g)
    v = torch.randn(1, n, d, generator=g)
    r = _full(orc, q, k, v, window=4, k_global=5)
    v64 = v[0].to(torch.float64).numpy()
    for p in range(n):
        mean = v64[:p + 1].mean(axis=0)
        for h in range(H):
            np.testing.assert_allclose(r["out"][p, h], mean, rtol=1e-12, atol=1e-13)
            assert abs(r["lse"][p, h] - math.log(p + 1)) < 1e-12
        np.testing.assert_allclose(r["scores"][p][:p + 1], H / (p + 1), rtol=1e-12)
        # all scores tie: the lowest candidate positions win
        n_cand = max(0, p - 4 + 1)
        want = list(range(min(5, n_cand))) + [-1] * (5 - min(5, n_cand))
        assert r["idx"][p][4:].tolist() == want


def test_constant_values_and_first_position(orc):
    n, H, d = 12, 2, 16
    g = torch.Generator().manual_seed(2)
    q = torch.randn(1, n, H, d, generator=g)
    k = torch.randn(1, n, d, generator=g)
    c = torch.randn(d, generator=g)
    v = c.expand(1, n, d).contiguous()
    r = _full(orc, q, k, v)
    np.testing.assert_allclose(r["out"], np.broadcast_to(c.double().numpy(), r["out"].shape),
                               rtol=1e-12, atol=1e-13)
    # p = 0: output is v_0 and LSE is the single logit
    v2 = torch.randn(1, n, d, generator=g)
    r2 = _full(orc, q, k, v2)
    np.testing.assert_allclose(r2["out"][0], np.broadcast_to(v2[0, 0].double().numpy(), (H, d)),
                               rtol=1e-12)
    s00 = (q[0, 0].double() @ k[0, 0].double()) / math.sqrt(d)
    np.testing.assert_allclose(r2["lse"][0], s00.numpy(), rtol=1e-12, atol=1e-13)


def test_two_key_closed_form(orc):
    d = 4
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, 1, d, generator=g)
    k = torch.randn(1, 2, d, generator=g)
    v = torch.randn(1, 2, d, generator=g)
    r = _full(orc, q, k, v, window=1, k_global=1)
    qd, kd, vd = q[0, 1, 0].double(), k[0].double(), v[0].double()
    s0, s1 = float(qd @ kd[0]) / 2, float(qd @ kd[1]) / 2
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(r["out"][1, 0], (w0 * vd[0] + (1 - w0) * vd[1]).numpy(), rtol=1e-12)
    assert abs(r["lse"][1, 0] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-12
    np.testing.assert_allclose(r["scores"][1][:2], [w0, 1 - w0], rtol=1e-12)


# ------------------------------------------------------------- invariants ----

def _check_rows(idx, p_of_row, W, K):
    for r, p in enumerate(p_of_row):
        row = idx[r]
        win, glb = row[:W], row[W:]
        nw = min(W, p + 1)
        assert win[:nw].tolist() == list(range(p - nw + 1, p + 1))
        assert (win[nw:] == -1).all()
        gv = glb[glb >= 0]
        n_cand = max(0, p - W + 1)
        assert len(gv) == min(K, n_cand)
        assert (glb[len(gv):] == -1).all()              # padding only at the end
        assert (np.diff(gv) > 0).all()                   # ascending, no duplicates
        if len(gv):
            assert gv.max() <= p - W                     # outside the window, causal
        sel = set(row[row >= 0].tolist())
        assert len(sel) == min(p + 1, W + K)             # window and global disjoint
        assert max(sel) <= p


def test_score_sums_to_H_and_selection_invariants(orc):
    wl = workload(1).with_(n_q=400, n_ctx=400, window=16, k_global=24, n_needles=4)
    x = make_inputs(wl)
    r = _full(orc, x.q, x.k, x.v, window=16, k_global=24)
    for p in range(wl.n_q):
        assert abs(r["scores"][p][:p + 1].sum() - wl.H) < 1e-12
    _check_rows(r["idx"], list(range(wl.n_q)), 16, 24)


def test_selection_is_threshold_on_scores(orc):
    """Every selected candidate beats every unselected one under (score desc,
    position asc); the stored K-th score is the smallest selected score."""
    wl = workload(1).with_(n_q=300, n_ctx=300, window=8, k_global=20, n_needles=0, needles="none")
    x = make_inputs(wl)
    r = _full(orc, x.q, x.k, x.v, window=8, k_global=20)
    for p in range(8, wl.n_q):
        sc = r["scores"][p][:p - 8 + 1]
        sel = r["idx"][p][8:]
        sel = sel[sel >= 0]
        mask = np.zeros(len(sc), bool)
        mask[sel] = True
        if mask.all():
            continue
        worst_in = min((sc[j], -j) for j in np.nonzero(mask)[0])
        best_out = max((sc[j], -j) for j in np.nonzero(~mask)[0])
        assert worst_in > best_out
        assert r["kth"][p] == worst_in[0]


def test_selection_brute_force_subsets(orc):
    """T <= 24: enumerate every K-subset of the candidates; exactly one has all
    members ranked above all non-members, and it must be the oracle's set."""
    g = torch.Generator().manual_seed(11)
    T, H, d, W = 22, 3, 8, 4
    q = torch.randn(1, T, H, d, generator=g)
    k = torch.randn(1, T, d, generator=g)
    k[0, 5] = k[0, 9]                                     # an exact tie
    v = torch.randn(1, T, d, generator=g)
    for K in (3, 4, 6):
        r = _full(orc, q, k, v, window=W, k_global=K)
        for p in range(W, T, 3):
            cand = list(range(0, p - W + 1))
            sc = r["scores"][p]
            good = []
            for sub in itertools.combinations(cand, min(K, len(cand))):
                rest = [j for j in cand if j not in sub]
                if all((sc[a], -a) > (sc[b], -b) for a in sub for b in rest):
                    good.append(sub)
            assert len(good) == 1
            got = [j for j in r["idx"][p][W:].tolist() if j >= 0]
            assert got == sorted(good[0])


def test_tie_goes_to_lower_position(orc):
    T, H, d, W = 12, 2, 4, 2
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, T, H, d, generator=g)
    k = torch.randn(1, T, d, generator=g)
    k[0, 2] = k[0, 6] = k[0, 1]                           # three identical keys
    q[0, -1, :, :] = k[0, 1] * 4                          # the last row favours them
    v = torch.randn(1, T, d, generator=g)
    r = _full(orc, q, k, v, window=W, k_global=2)
    sc = r["scores"][T - 1]
    assert sc[1] == sc[2] == sc[6]
    assert r["idx"][T - 1][W:].tolist() == [1, 2]


def test_results_do_not_depend_on_thread_count(orc):
    wl = workload(1).with_(n_q=256, n_ctx=256, n_needles=2)
    x = make_inputs(wl)
    n0 = orc.num_threads()
    try:
        orc.set_threads(1)
        a = _full(orc, x.q, x.k, x.v, window=16, k_global=32)
        orc.set_threads(max(2, n0))
        b = _full(orc, x.q, x.k, x.v, window=16, k_global=32)
    finally:
        orc.set_threads(n0)
    for key in ("out", "lse", "idx", "scores"):
        assert np.array_equal(a[key], b[key])


# ----------------------------------------------------------------- sparse ----

def test_sparse_equals_full_when_everything_is_selected(orc):
    """K >= number of candidates: the index row lists every visible key, so a
    sparse layer fed the full layer's own query reproduces full attention."""
    wl = workload(2).with_(n_q=90, n_ctx=90, window=16, k_global=100, n_needles=2)
    x = make_inputs(wl)
    rows = list(range(wl.n_q))
    r = _full(orc, x.q, x.k, x.v, window=16, k_global=100, rows=rows, scores=False)
    s = orc.sparse(x.q, x.k, x.v, None, None, r["idx"], x.sm_scale, rows)
    np.testing.assert_allclose(s["out"], r["out"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["lse"], r["lse"], rtol=1e-12, atol=1e-13)


def test_sparse_matches_masked_sdpa(orc):
    g = torch.Generator().manual_seed(13)
    n_ctx, H, d, S = 60, 4, 32, 12
    q = torch.randn(1, 5, H, d, generator=g)
    k = torch.randn(1, n_ctx, d, generator=g)
    v = torch.randn(1, n_ctx, d, generator=g)
    idx = np.full((5, S), -1, np.int32)
    rng = np.random.default_rng(0)
    for r in range(5):
        m = rng.integers(1, S + 1)
        idx[r, :m] = rng.choice(n_ctx, size=m, replace=False)
    sm = 0.3
    s = orc.sparse(q, k, v, None, None, idx, sm, list(range(5)))
    mask = torch.zeros(5, n_ctx, dtype=torch.bool)
    for r in range(5):
        mask[r, idx[r][idx[r] >= 0]] = True
    o_ref, lse_ref = _sdpa64(q[0], k[0], v[0], mask, sm)
    np.testing.assert_allclose(s["out"], o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s["lse"], lse_ref, rtol=1e-12)


def test_sparse_empty_row(orc):
    q = torch.randn(1, 1, 2, 4)
    k = torch.randn(1, 3, 4)
    s = orc.sparse(q, k, k.clone(), None, None, np.full((1, 5), -1, np.int32), 0.5, [0])
    assert (s["out"] == 0).all() and np.isneginf(s["lse"]).all()


# -------------------------------------------------------- select on scores ----

def _lexsort_topk(row, n, k):
    order = np.lexsort((np.arange(n), -row[:n].astype(np.float64)))
    take = sorted(order[:min(k, n)].tolist())
    return take + [-1] * (k - len(take))


def test_select_scores_f32(orc):
    rng = np.random.default_rng(3)
    rows, n, k = 12, 5000, 300
    s = rng.random((rows, n), dtype=np.float32)
    s[1] = 0.25                                           # every score tied
    s[2, ::7] = s[2, 3]                                   # many ties at one value
    s[3] = np.float32(1e-30) * np.arange(n, 0, -1)        # tiny, descending
    s[4, :] = 0.0
    n_cand = [n, n, n, n, n, 299, 300, 301, 0, 1, 4000, 17]
    got = orc.select_scores_f32(s, n_cand, k)
    for r in range(rows):
        assert got[r].tolist() == _lexsort_topk(s[r], n_cand[r], k)
    assert got[1].tolist() == list(range(k))


def test_select_scores_brute_force_small(orc):
    rng = np.random.default_rng(4)
    for trial in range(30):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 6))
        row = rng.integers(0, 4, size=n).astype(np.float32)   # many ties
        got = orc.select_scores_f32(row.reshape(1, -1), [n], k)[0]
        best = None
        for sub in itertools.combinations(range(n), min(k, n)):
            rest = [j for j in range(n) if j not in sub]
            if all((row[a], -a) > (row[b], -b) for a in sub for b in rest):
                best = sorted(sub)
        assert got.tolist() == best + [-1] * (k - len(best))


# -------------------------------------------------------------------- FP8 ----

def test_e4m3_decode_all_codes(orc):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    for c in range(256):
        got = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got) and (c & 0x7F) == 0x7F
        else:
            assert got == ref[c]
    # spot values of the format: max 448, min subnormal 2^-9, min normal 2^-6
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0xC0) == -2.0


def test_quantizer_is_round_to_nearest_even(orc):
    vals = np.array([orc.e4m3_value(c) for c in range(256)])
    finite = np.unique(vals[~np.isnan(vals)])
    g = torch.Generator().manual_seed(9)
    x = torch.randn(64, 128, generator=g) * torch.logspace(-3, 3, 64).unsqueeze(1)
    x[3] = 0.0
    codes, sc = quantize_e4m3(x)
    assert sc[3] == 1.0 and (codes[3] & 0x7F == 0).all()
    y = (x / sc.unsqueeze(1)).clamp(-448, 448).to(torch.float64).numpy()
    got = np.array([orc.e4m3_value(int(c)) for c in codes.flatten()]).reshape(y.shape)
    for a, b in zip(y.flatten()[::7], got.flatten()[::7]):
        i = np.searchsorted(finite, a)
        cands = [finite[j] for j in (i - 1, i) if 0 <= j < len(finite)]
        best = min(abs(c - a) for c in cands)
        assert abs(b - a) == best
        ties = [c for c in cands if abs(c - a) == best]
        if len(ties) == 2:   # exact half-way: even mantissa wins
            even = [c for c in ties if int(np.where(vals == c)[0][0]) % 2 == 0]
            assert b == even[0]
    # the largest magnitude in every row maps to +-448
    assert (got.__abs__().max(axis=1)[np.arange(64) != 3] == 448.0).all()


# ---------------------------------------------------------------- needles ----

def _recovered(orc, x, rows):
    wl = x.wl
    r = orc.full_select(x.q, x.k, x.v, x.k_scale, x.v_scale, wl.q_pos0, wl.window, wl.k_global,
                        x.sm_scale, rows, select=True)
    pos = {row: t for t, row in enumerate(r["rows"].tolist())}
    hit = 0
    for n in x.needles:
        row = n.b * wl.n_q + n.i
        glb = r["idx"][pos[row]][wl.window:]
        hit += all((n.j + t) in glb for t in range(n.length))
    return hit, len(x.needles)


def test_needles_config1_literal_norm_all_recovered(orc):
    wl = workload(1)
    x = make_inputs(wl, needle_norm="R18a")
    rows = sorted({n.b * wl.n_q + n.i for n in x.needles})
    hit, tot = _recovered(orc, x, rows)
    assert (hit, tot) == (16, 16)


def test_needles_strong_norm_recovered_at_4k_h16(orc):
    wl = workload(2).with_(n_q=64, q_pos0=4032, n_ctx=4096, n_needles=24)
    x = make_inputs(wl, needle_norm="R18b")
    rows = sorted({n.b * wl.n_q + n.i for n in x.needles})
    hit, tot = _recovered(orc, x, rows)
    assert hit == tot == 24


def test_clustered_needles_fp8_recovered_with_ties(orc):
    wl = workload(4).with_(n_q=16, q_pos0=3000, n_ctx=3016, n_needles=4)
    x = make_inputs(wl, needle_norm="R18b")
    # identical keys inside a cluster stay identical after quantisation
    for n in x.needles:
        blk = x.k[0, n.j:n.j + n.length]
        assert (blk == blk[0]).all()
    rows = sorted({n.b * wl.n_q + n.i for n in x.needles})
    hit, tot = _recovered(orc, x, rows)
    assert hit == tot == 4


# ------------------------------------------------------------ KV Bridging

def test_e4m3_encoder_matches_torch_cast(orc):
    """The oracle's FP8 encoder (nearest, ties to even) against torch's
    float8_e4m3fn cast of the same float32 values, inside the finite range."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.standard_normal(4000) * 30.0, rng.uniform(-448, 448, 4000),
                           rng.standard_normal(2000) * 1e-2, [0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]])
    vals = vals.astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert (got == ref).all(), (vals[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])


def test_e4m3_encoder_round_trip_and_ties(orc):
    for c in list(range(0x00, 0x7F)) + list(range(0x81, 0xFF)):
        assert orc.e4m3_encode(orc.e4m3_value(c)) == c
    for c in range(0x00, 0x7E):  # the midpoint of two neighbours goes to the even code
        mid = 0.5 * (orc.e4m3_value(c) + orc.e4m3_value(c + 1))
        assert orc.e4m3_encode(mid) == (c if c % 2 == 0 else c + 1)
    assert orc.e4m3_encode(1e6) == 0x7E and orc.e4m3_encode(-1e6) == 0xFE


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def test_kv_project_one_hot_rows_give_weight_columns(orc):
    """A hidden row e_k projects to column k of each [d][hidden] weight."""
    J, d, hidden = 2, 8, 24
    rng = np.random.default_rng(3)
    w = _bf16(rng.standard_normal((J, 2, d, hidden)))
    h = _bf16(np.eye(hidden))
    r = orc.kv_project(h, w, list(range(hidden)))
    wf = w.float().double().numpy()
    for k in range(hidden):
        assert np.array_equal(r["x"][:, :, k, :], wf[:, :, :, k])


def test_kv_project_is_linear(orc):
    """Additivity and scaling by 2 hold exactly (sums of bf16 products are exact
    in float64 at this size), pinning every term of the contraction."""
    J, d, hidden, T = 2, 16, 64, 5
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal((J, 2, d, hidden)))
    a = _bf16(rng.standard_normal((T, hidden)))
    b = _bf16(rng.standard_normal((T, hidden)))
    s = _bf16(a.float() + b.float())
    exact = (a.float() + b.float() == s.float()).all().item()
    ra, rb = orc.kv_project(a, w, range(T))["x"], orc.kv_project(b, w, range(T))["x"]
    r2 = orc.kv_project(_bf16(2 * a.float()), w, range(T))["x"]
    assert np.array_equal(r2, 2 * ra)
    if exact:
        assert np.array_equal(orc.kv_project(s, w, range(T))["x"], ra + rb)
    # additivity on rows whose sum is exactly representable
    ok = (a.float() + b.float() == s.float()).all(dim=1).numpy()
    rs = orc.kv_project(s, w, range(T))["x"]
    assert np.allclose(rs[:, :, ok], (ra + rb)[:, :, ok], rtol=0, atol=1e-9)


def test_kv_project_quantisation(orc):
    """Per-token scale = max|x| / 448: the largest element of each row codes to
    +-448, every code decodes within half a step of x / scale, and an all-zero
    row has scale 1 and zero codes."""
    J, d, hidden, T = 1, 32, 64, 6
    rng = np.random.default_rng(5)
    w = _bf16(rng.standard_normal((J, 2, d, hidden)))
    h = rng.standard_normal((T, hidden)).astype(np.float32)
    h[2] = 0.0
    r = orc.kv_project(_bf16(h), w, range(T), quantize=True)
    x, codes, sc = r["x"], r["codes"], r["scales"]
    dec = np.vectorize(orc.e4m3_value)(codes)
    grid = np.array([orc.e4m3_value(c) for c in range(0x7F)])  # the finite non-negative values
    for kind in range(2):
        for t in range(T):
            if t == 2:
                assert sc[0, kind, t] == 1.0 and (codes[0, kind, t] == 0).all()
                continue
            # the quantiser works in fp32: t = fl32(fl32(x) / scale), scale an fp32 value
            assert sc[0, kind, t] == np.float64(np.float32(sc[0, kind, t]))
            y = (x[0, kind, t].astype(np.float32) / np.float32(sc[0, kind, t])).astype(np.float64)
            assert np.isclose(np.abs(y).max(), 448.0)
            assert np.abs(dec[0, kind, t]).max() == 448.0
            # each code decodes to a representable value nearest to x / scale
            best = np.abs(np.abs(y)[:, None] - grid[None, :]).min(axis=1)
            assert np.allclose(np.abs(dec[0, kind, t] - y), best, rtol=0, atol=1e-12)


def test_kv_project_quantisation_matches_torch_fp32_cast(orc):
    """The oracle's fp32 quantiser against torch's own float8_e4m3fn cast applied
    to the same fp32 rows (scale = amax / 448 in fp32, divide, clamp, RNE cast):
    codes and scales bit-identical on Gaussian rows and on rows with ties."""
    J, d, hidden, T = 2, 64, 96, 40
    rng = np.random.default_rng(11)
    w = _bf16(rng.standard_normal((J, 2, d, hidden)) / np.sqrt(hidden))
    h = rng.standard_normal((T, hidden)).astype(np.float32)
    h[3] = 0.0
    h[7] = np.round(h[7] * 4) / 4            # coarse values: more exact midpoints
    r = orc.kv_project(_bf16(h), w, range(T), quantize=True)
    x32 = torch.from_numpy(r["x"].astype(np.float32))
    amax = x32.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    ref = (x32 / scale.unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(torch.from_numpy(r["codes"]), ref)
    assert np.array_equal(r["scales"], scale.double().numpy())


# ------------------------------------------------- HySparse (v1) block variant

def test_block_select_hand_example(orc):
    """Block scores and choices worked by hand: sums of each block's causal
    token scores, ties to the lower block, output ascending and -1 padded."""
    s = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 9, 10]], float)
    bs, bi = orc.block_select_scores(s, [9], 4, 2)
    assert bs.tolist() == [[10, 26, 19]] and bi.tolist() == [[1, 2]]
    bs, bi = orc.block_select_scores(s, [5], 4, 5)            # block 1 holds positions 4, 5 only
    assert bs.tolist() == [[10, 11, 0]] and bi.tolist() == [[0, 1, -1, -1, -1]]
    t = np.array([[1, 1, 1, 1, 2, 0, 0, 0, 1, 1, 1, 1]], float)
    _, bi = orc.block_select_scores(t, [11], 4, 2)            # sums 4, 2, 4
    assert bi.tolist() == [[0, 2]]
    _, bi = orc.block_select_scores(t, [11], 4, 1)            # tie of blocks 0 and 2: the lower wins
    assert bi.tolist() == [[0]]


def test_block_scores_hold_the_whole_attention_mass(orc):
    """Summed over a row's blocks, the block scores give sum_h sum_j p_hj = H."""
    wl = workload(1)
    x = make_inputs(wl)
    rows = [0, 1, 63, 64, 65, 700, 2047]
    r = orc.block_select(x.q, x.k, x.v, None, None, 0, 64, 16, x.sm_scale, rows)
    assert np.allclose(r["block_scores"].sum(axis=1), wl.H, rtol=0, atol=1e-9)
    # and block c's score is zero once c * 64 > p
    for i, p in enumerate(r["pos"]):
        assert (r["block_scores"][i, p // 64 + 1:] == 0).all()


def test_block_select_of_one_token_blocks_is_token_topk(orc):
    """With 1-token blocks the block choice is the top-k of the token scores
    over all causal positions, checked against a plain sort."""
    wl = workload(1)
    x = make_inputs(wl)
    rows = [5, 300, 1999]
    r = orc.block_select(x.q, x.k, x.v, None, None, 0, 1, 40, x.sm_scale, rows)
    for i, p in enumerate(r["pos"]):
        s = r["scores"][i, :p + 1]
        order = sorted(range(p + 1), key=lambda j: (-s[j], j))[:40]
        want = sorted(order) + [-1] * (40 - len(order))
        assert r["block_idx"][i].tolist() == want


def test_block_select_recovers_planted_needles(orc):
    """A strong needle key aimed at a query row puts its block among the row's
    16 selected 64-token blocks."""
    wl = workload(2).with_(n_q=64, q_pos0=4032, n_ctx=4096, n_needles=24)
    x = make_inputs(wl, needle_norm="R18b")
    rows = sorted({n.b * wl.n_q + n.i for n in x.needles})
    r = orc.block_select(x.q, x.k, x.v, None, None, wl.q_pos0, 64, 16, x.sm_scale, rows)
    where = {row: i for i, row in enumerate(rows)}
    for n in x.needles:
        assert n.j // 64 in r["block_idx"][where[n.b * wl.n_q + n.i]].tolist()


def test_block_sparse_reduces_to_full_attention(orc):
    """Gate (1, 0) with every causal block selected, and gate (0, 1) with a
    window covering the whole prefix, both give the full layer's attention."""
    wl = workload(1)
    x = make_inputs(wl)
    rows = [0, 7, 130, 1000, 2047]
    full = orc.full_select(x.q, x.k, x.v, None, None, 0, 1, 0, x.sm_scale, rows, select=False)
    n_blk = (wl.n_ctx + 63) // 64
    sel = orc.block_select(x.q, x.k, x.v, None, None, 0, 64, n_blk, x.sm_scale, rows)
    g = np.zeros((wl.B * wl.n_q, wl.H, 2))
    g[..., 0] = 1.0
    rb = orc.block_sparse(x.q, x.k, x.v, None, None, sel["block_idx"], 64, 128, g, 0, x.sm_scale, rows)
    assert np.allclose(rb["out"], full["out"], rtol=0, atol=1e-12)
    g = g[..., ::-1].copy()
    rw = orc.block_sparse(x.q, x.k, x.v, None, None, sel["block_idx"], 64, wl.n_ctx, g, 0, x.sm_scale, rows)
    assert np.allclose(rw["out"], full["out"], rtol=0, atol=1e-12)
    # the window branch alone is attention over the last 128 positions
    assert (rb["win_idx"][3] == np.arange(1000 - 127, 1001)).all()
    assert (rb["win_idx"][1][:8] == np.arange(8)).all() and (rb["win_idx"][1][8:] == -1).all()


# ----------------------------------------------------- light indexer (DSA-style)

def _e4m3_codes(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


def test_index_select_hand_example(orc):
    """Two heads picking the two coordinates of 2-d keys, weights 1 and 1/2:
    I(j) = relu(k_j[0]) + relu(k_j[1]) / 2, worked by hand; then window 2 and
    the top candidates among j <= p - 2, ties to the lower position."""
    qi = _e4m3_codes([[[[1, 0], [0, 1]]]])                    # [B=1][n_q=1][HI=2][dI=2]
    ki = _e4m3_codes([[[2, 0], [0, 2], [1, 1], [-1, 2], [0, 0], [1, 0]]])
    qs, ks = torch.ones(1, 1, 2), torch.ones(1, 6)
    w = torch.tensor([[[1.0, 0.5]]])
    r = orc.index_select(qi, qs, w, ki, ks, 5, 2, 2, [0], want_scores=True)
    assert r["scores"][0].tolist() == [2.0, 1.0, 1.5, 1.0, 0.0, 1.0]
    assert r["idx"][0].tolist() == [4, 5, 0, 2]
    r = orc.index_select(qi, qs, w, ki, ks, 5, 2, 3, [0])       # 1 and 3 tie at 1: 1 wins
    assert r["idx"][0].tolist() == [4, 5, 0, 1, 2]
    w = torch.tensor([[[-1.0, 0.5]]])                           # I = -2, 1, -0.5, 1
    r = orc.index_select(qi, qs, w, ki, ks, 5, 2, 2, [0], want_scores=True)
    assert r["scores"][0][:4].tolist() == [-2.0, 1.0, -0.5, 1.0]
    assert r["idx"][0].tolist() == [4, 5, 1, 3]
    r = orc.index_select(qi, qs, w, ki, ks, 5, 2, 1, [0])
    assert r["idx"][0].tolist() == [4, 5, 1]


def test_index_select_scales_and_relu(orc):
    """The scales multiply each head's dot product; a head whose dot product is
    negative contributes nothing whatever its weight."""
    qi = _e4m3_codes([[[[1, 1], [-1, -1]]]])
    ki = _e4m3_codes([[[1, 2], [3, 0]]])
    w = torch.tensor([[[2.0, -5.0]]])
    r = orc.index_select(qi, torch.tensor([[[0.5, 1.0]]]), w, ki, torch.tensor([[4.0, 0.25]]), 1, 1, 1, [0],
                         want_scores=True)
    # head 0: 0.5 * scale_k * (k0 + k1), head 1: negative dot, relu -> 0
    assert r["scores"][0].tolist() == [2.0 * 0.5 * 4.0 * 3.0, 2.0 * 0.5 * 0.25 * 3.0]


def test_index_select_all_zero_scores_pick_lowest_positions(orc):
    """Queries of +1 and keys of -1 everywhere: every dot product is negative,
    every score 0 whatever the weights, so the global part is the first
    k_global candidates."""
    from hs2_inputs import make_indexer_inputs
    x = make_indexer_inputs(3, 1, 4, 300, 304, 4, 64)
    qi = _e4m3_codes(np.ones((1, 4, 4, 64)).tolist())
    ki = _e4m3_codes((-np.ones((1, 304, 64))).tolist())
    r = orc.index_select(qi, torch.ones(1, 4, 4), x.w, ki, torch.ones(1, 304), 300, 128, 16, [0, 3],
                         want_scores=True)
    assert (r["scores"][0, :301] == 0).all() and (r["scores"][1, :304] == 0).all()
    assert r["idx"][0][128:].tolist() == list(range(16))
    assert r["idx"][1][:128].tolist() == list(range(303 - 127, 304))


def test_index_select_sign_and_order(orc):
    """Negating the weights negates every score exactly, and the chosen set is
    the plain sort of the scores (desc, position asc) over the candidates."""
    from hs2_inputs import make_indexer_inputs
    x = make_indexer_inputs(5, 1, 6, 500, 506, 8, 64)
    rows = [0, 5]
    a = orc.index_select(x.qi, x.qs, x.w, x.ki, x.ks, 500, 128, 40, rows, want_scores=True)
    b = orc.index_select(x.qi, x.qs, (-x.w).contiguous(), x.ki, x.ks, 500, 128, 40, rows, want_scores=True)
    for t, row in enumerate(rows):
        p = 500 + row
        assert np.array_equal(b["scores"][t, :p + 1], -a["scores"][t, :p + 1])
        for r in (a, b):
            s = r["scores"][t]
            order = sorted(range(p - 128 + 1), key=lambda j: (-s[j], j))[:40]
            assert r["idx"][t][128:].tolist() == sorted(order)


def test_index_select_recovers_planted_needles(orc):
    from hs2_inputs import make_indexer_inputs
    x = make_indexer_inputs(11, 1, 64, 4032, 4096, 4, 64, n_needles=12)
    rows = sorted({r for r, _, _ in x.needles})
    r = orc.index_select(x.qi, x.qs, x.w, x.ki, x.ks, 4032, 128, 1024, rows)
    where = {row: i for i, row in enumerate(rows)}
    for row, h, j in x.needles:
        assert j in r["idx"][where[row]][128:].tolist()


def test_sparse_duplicate_entry_is_counted_twice(orc):
    """A position listed twice gets two softmax terms: over the row [j, j] the
    weights are 1/2 each, so O = v_j and LSE = s_j + ln 2 (closed form)."""
    g = torch.Generator().manual_seed(3)
    H, d, n_ctx = 2, 4, 8
    q = torch.randn(1, 1, H, d, generator=g)
    k = torch.randn(1, n_ctx, d, generator=g)
    v = torch.randn(1, n_ctx, d, generator=g)
    j, sm = 5, 0.5
    r = orc.sparse(q, k, v, None, None, np.array([[j, j, -1]], np.int32), sm, [0])
    s_j = sm * (q[0, 0].double() @ k[0, j].double()).numpy()          # [H]
    np.testing.assert_allclose(r["out"][0], np.broadcast_to(v[0, j].double().numpy(), (H, d)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"][0], s_j + np.log(2.0), rtol=0, atol=1e-12)
