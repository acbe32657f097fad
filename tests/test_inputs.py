"""The seeded generator: determinism, storage formats and needle placement."""
import math

import torch

from hs2_inputs import WORKLOADS, checked_rows, make_inputs, workload


def test_deterministic_and_formats():
    wl = workload(4).with_(n_q=8, q_pos0=600, n_ctx=608, n_needles=3)
    a, b = make_inputs(wl), make_inputs(wl, threads=1)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.k_scale, b.k_scale), (a.q_sparse, b.q_sparse)):
        assert torch.equal(x, y)
    assert a.q.dtype == torch.bfloat16 and a.k.dtype == torch.uint8
    assert a.k_scale.shape == (1, 608) and a.q_sparse.shape == (3, 1, 8, 16, 128)
    assert ((a.k & 0x7F) != 0x7F).all()                  # no NaN codes


def test_needles_lie_outside_the_window_and_align_with_queries():
    for cfg in (1, 2):
        wl = workload(cfg).with_(n_q=512, n_ctx=512, n_needles=8)
        x = make_inputs(wl, needle_norm="R18b")
        assert len(x.needles) == 8
        for n in x.needles:
            p = wl.q_pos0 + n.i
            assert 0 <= n.j <= p - wl.window
            kv = x.k[n.b, n.j].to(torch.float64)
            qv = x.q[n.b, n.i, n.h].to(torch.float64)
            cos = float(kv @ qv / (kv.norm() * qv.norm()))
            assert cos > 0.99
            assert abs(float(kv.norm()) - 3 * math.sqrt(wl.d)) < 0.05 * 3 * math.sqrt(wl.d)


def test_depth_needles_are_spread_uniformly():
    wl = workload(5).with_(n_ctx=65536, q_pos0=65535, B=2)
    x = make_inputs(wl)
    js = sorted(n.j for n in x.needles if n.b == 0)
    span = 65535 - wl.window + 1
    assert js == [math.floor((m + 0.5) * span / 64) for m in range(64)]


def test_checked_rows_contain_needle_rows():
    wl = workload(2).with_(n_q=2048, n_ctx=2048, n_needles=16)
    x = make_inputs(wl)
    rows = checked_rows(wl, x.needles, 100)
    assert {n.i for n in x.needles} <= set(rows)
    assert len(rows) == 116


def test_workload_table_matches_the_five_settings():
    assert [WORKLOADS[c].n_ctx for c in range(1, 6)] == [2048, 32768, 131072, 262144, 1048576]
    assert all(WORKLOADS[c].window == 128 for c in range(1, 6))
    assert [WORKLOADS[c].k_global for c in range(1, 6)] == [256, 1024, 1024, 1024, 1024]
    assert [WORKLOADS[c].n_sparse for c in range(1, 6)] == [1, 2, 4, 3, 5]
