"""Seeded generation of queries, KV cache and planted needles.

Streams (numpy Philox, one SeedSequence per (workload, stream, sequence)):
  1 = full-layer queries, 2 = K, 3 = V, 10+l = queries of sparse layer l,
  50 = needle placement, 60 = rows the oracle checks.
All values are float32 N(0,1). Needles are planted in float32, then every
array is rounded once into its storage format: bf16 by round-to-nearest-even,
FP8 as OCP E4M3FN codes with a per-token fp32 scale amax/448 (1 for an
all-zero row), values clamped to +-448 before the round-to-nearest-even cast.
Both sides of every comparison consume exactly these rounded arrays.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

from .configs import Workload

E4M3_MAX = 448.0

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _rng(wl: Workload, stream: int, sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([wl.cfg_id, stream, sub])))


def _normal(wl: Workload, stream: int, sub: int, shape) -> np.ndarray:
    return _rng(wl, stream, sub).standard_normal(size=shape, dtype=np.float32)


def quantize_e4m3(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-row (last dim) FP8 quantisation. Returns (uint8 codes, float32 scales)."""
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


@dataclass
class Needle:
    b: int       # sequence
    i: int       # query row (index into n_q) the needle is aimed at
    h: int       # head whose query the needle copies
    j: int       # first key position
    length: int  # number of adjacent identical keys (1 unless clustered)


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor                    # [B][n_q][H][d]  f32 or bf16
    q_sparse: torch.Tensor             # [L][B][n_q][H][d]
    k: torch.Tensor                    # [B][n_ctx][d]  f32 / bf16 / uint8 codes
    v: torch.Tensor
    k_scale: Optional[torch.Tensor]    # [B][n_ctx] f32 (fp8 only)
    v_scale: Optional[torch.Tensor]
    needles: List[Needle] = field(default_factory=list)
    needle_norm: float = 3.0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.wl.d)


def _pick_needles(wl: Workload) -> List[Needle]:
    out: List[Needle] = []
    W = wl.window
    for b in range(wl.B):
        rng = _rng(wl, 50, b)
        used = set()
        if wl.needles == "none" or wl.n_needles == 0:
            continue
        if wl.needles == "rows":
            lo = max(0, W - wl.q_pos0)          # rows with p - W >= 0
            rows = np.arange(lo, wl.n_q)
            n = min(wl.n_needles, len(rows))
            pick = rng.choice(rows, size=n, replace=False)
            for i in sorted(int(r) for r in pick):
                p = wl.q_pos0 + i
                while True:
                    j = int(rng.integers(0, p - W + 1))
                    if j not in used:
                        break
                used.add(j)
                out.append(Needle(b, i, int(rng.integers(0, wl.H)), j, 1))
        elif wl.needles == "decode":
            p = wl.q_pos0 + wl.n_q - 1
            for _ in range(wl.n_needles):
                while True:
                    j = int(rng.integers(0, p - W + 1))
                    if j not in used:
                        break
                used.add(j)
                out.append(Needle(b, 0, int(rng.integers(0, wl.H)), j, 1))
        elif wl.needles == "depth":
            p = wl.q_pos0 + wl.n_q - 1
            n = wl.n_needles
            span = p - W + 1
            for m in range(n):
                j = int(math.floor((m + 0.5) * span / n))
                out.append(Needle(b, 0, int(rng.integers(0, wl.H)), j, 1))
        elif wl.needles == "clusters":
            L = wl.cluster_len
            lo = max(0, W + L - 1 - wl.q_pos0)
            rows = np.arange(lo, wl.n_q)
            n = min(wl.n_needles, len(rows))
            pick = rng.choice(rows, size=n, replace=False)
            for i in sorted(int(r) for r in pick):
                p = wl.q_pos0 + i
                for _ in range(1000):
                    j = int(rng.integers(0, p - W - L + 2))
                    if not any((j + t) in used for t in range(L)):
                        break
                used.update(j + t for t in range(L))
                out.append(Needle(b, i, int(rng.integers(0, wl.H)), j, L))
        else:
            raise ValueError(wl.needles)
    return out


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(wl: Workload, needle_norm: str = "R18a", threads: Optional[int] = None) -> Inputs:
    """Generate every array for workload `wl` on the host (CPU tensors).

    needle_norm "R18a": planted key = 3 * q/|q| (the workload text read literally).
    needle_norm "R18b": planted key = 3*sqrt(d) * q/|q| (three times a typical key
    norm), used where the test asks that every needle be recovered.
    """
    B, nq, H, d, nc = wl.B, wl.n_q, wl.H, wl.d, wl.n_ctx
    assert wl.q_pos0 + nq <= nc
    norm = 3.0 if needle_norm == "R18a" else 3.0 * math.sqrt(d)
    th = threads or _threads()
    qdt = _TORCH_DT[wl.q_dtype]

    def gen_q(stream):
        arr = torch.empty((B, nq, H, d), dtype=qdt)
        for b in range(B):
            arr[b] = torch.from_numpy(_normal(wl, stream, b, (nq, H, d))).to(qdt)
        return arr

    q = gen_q(1)
    q_sparse = torch.stack([gen_q(10 + l) for l in range(wl.n_sparse)]) if wl.n_sparse else \
        torch.empty((0, B, nq, H, d), dtype=qdt)
    needles = _pick_needles(wl)
    by_b = {}
    for n in needles:
        by_b.setdefault(n.b, []).append(n)

    fp8 = wl.kv_dtype == "fp8"
    kv_dt = torch.uint8 if fp8 else _TORCH_DT[wl.kv_dtype]
    k = torch.empty((B, nc, d), dtype=kv_dt)
    v = torch.empty((B, nc, d), dtype=kv_dt)
    ks = torch.empty((B, nc), dtype=torch.float32) if fp8 else None
    vs = torch.empty((B, nc), dtype=torch.float32) if fp8 else None

    def fill(job):
        b, which = job
        x = torch.from_numpy(_normal(wl, 2 if which == "k" else 3, b, (nc, d)))
        if which == "k":
            for n in by_b.get(b, []):
                qv = q[n.b, n.i, n.h].to(torch.float32)
                vec = norm * qv / qv.norm()
                x[n.j:n.j + n.length] = vec
        dst, sdst = (k, ks) if which == "k" else (v, vs)
        if fp8:
            codes, sc = quantize_e4m3(x)
            dst[b] = codes
            sdst[b] = sc
        else:
            dst[b] = x.to(kv_dt)

    jobs = [(b, w) for b in range(B) for w in ("k", "v")]
    with ThreadPoolExecutor(th) as ex:
        list(ex.map(fill, jobs))
    return Inputs(wl, q, q_sparse, k, v, ks, vs, needles, norm)


def checked_rows(wl: Workload, needles: List[Needle], n_uniform: int) -> List[int]:
    """Flat query rows (b*n_q + i) the oracle checks: every needle's target row
    plus `n_uniform` further rows drawn without replacement (stream 60)."""
    rows = sorted({n.b * wl.n_q + n.i for n in needles})
    total = wl.B * wl.n_q
    rest = np.setdiff1d(np.arange(total), np.array(rows, dtype=np.int64))
    rng = _rng(wl, 60, 0)
    n = min(n_uniform, len(rest))
    extra = rng.choice(rest, size=n, replace=False) if n else np.array([], dtype=np.int64)
    return sorted(set(rows) | {int(r) for r in extra})


def make_projection_inputs(seed: int, T: int, hidden: int, J: int, d: int, exact: bool = False,
                           zero_rows: Tuple[int, ...] = ()) -> Tuple[torch.Tensor, torch.Tensor]:
    """Hidden states h [T][hidden] and KV Bridging weights w [J][2][d][hidden],
    both bf16 (CPU). Streams 70 (h) and 71 (w) of SeedSequence([seed, stream]).

    Default: h ~ N(0,1) (a normalised hidden state), w ~ N(0, 1/hidden), so the
    projected values are about N(0,1).
    exact=True: h integers in [-3, 3] and w = k/16 with integer k in [-8, 8];
    every product is a multiple of 1/16 and every partial sum stays below
    2^24/16 for hidden < 5000, so an fp32 accumulation is exact in any order.
    Rows listed in zero_rows are all-zero."""
    g = [np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, s]))) for s in (70, 71)]
    if exact:
        assert hidden < 5000
        h = g[0].integers(-3, 4, size=(T, hidden)).astype(np.float32)
        w = g[1].integers(-8, 9, size=(J, 2, d, hidden)).astype(np.float32) / 16.0
    else:
        h = g[0].standard_normal(size=(T, hidden), dtype=np.float32)
        w = g[1].standard_normal(size=(J, 2, d, hidden), dtype=np.float32) / np.float32(math.sqrt(hidden))
    for r in zero_rows:
        h[r] = 0.0
    return torch.from_numpy(h).to(torch.bfloat16), torch.from_numpy(w).to(torch.bfloat16)


def make_gates(seed: int, shape) -> torch.Tensor:
    """Gate values in (0, 1) for the two-branch sparse layer, fp32 (CPU):
    the logistic function of N(0,1) draws (stream 72 of SeedSequence([seed, 72]))."""
    g = np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, 72])))
    z = g.standard_normal(size=shape)
    return torch.from_numpy((1.0 / (1.0 + np.exp(-z))).astype(np.float32))


@dataclass
class IndexerInputs:
    qi: torch.Tensor       # [B][n_q][HI][dI] uint8 E4M3 codes
    qs: torch.Tensor       # [B][n_q][HI] fp32 scales
    w: torch.Tensor        # [B][n_q][HI] fp32 head weights (either sign)
    ki: torch.Tensor       # [B][n_ctx][dI] uint8 E4M3 codes
    ks: torch.Tensor       # [B][n_ctx] fp32 scales
    needles: List[Tuple[int, int, int]] = field(default_factory=list)  # (flat query row, head, key position)


def make_indexer_inputs(seed: int, B: int, n_q: int, q_pos0: int, n_ctx: int, HI: int, dI: int,
                        n_needles: int = 0, window: int = 128, exact: bool = False) -> IndexerInputs:
    """Light-indexer operands (streams 80..84 of SeedSequence([seed, stream])).

    Default: queries and keys N(0,1), quantised per (token, head) and per key
    row to E4M3 with scale amax/448; weights N(0, 1/HI), so a few are negative
    per token. Needles: for a random query row and head with a positive
    weight (its largest, and only where it is at least 0.5), the key at a random
    candidate position (<= p - window) is set to 8*sqrt(dI) times the unit
    direction of that head's query.
    exact=True: codes of integers in [-2, 2], unit scales, weights k/8 with
    integer k in [-8, 8]: every dot product and weighted sum is exact in fp32
    and equal scores are common (ties then decide by position)."""
    g = [np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, s]))) for s in range(80, 85)]
    if exact:
        qv = torch.from_numpy(g[0].integers(-2, 3, size=(B, n_q, HI, dI)).astype(np.float32))
        kv = torch.from_numpy(g[1].integers(-2, 3, size=(B, n_ctx, dI)).astype(np.float32))
        w = torch.from_numpy(g[2].integers(-8, 9, size=(B, n_q, HI)).astype(np.float32) / 8.0)
        qi = qv.to(torch.float8_e4m3fn).view(torch.uint8)
        ki = kv.to(torch.float8_e4m3fn).view(torch.uint8)
        return IndexerInputs(qi, torch.ones(B, n_q, HI), w, ki, torch.ones(B, n_ctx))
    qv = torch.from_numpy(g[0].standard_normal(size=(B, n_q, HI, dI), dtype=np.float32))
    kv = torch.from_numpy(g[1].standard_normal(size=(B, n_ctx, dI), dtype=np.float32))
    w = torch.from_numpy(g[2].standard_normal(size=(B, n_q, HI), dtype=np.float32) / np.float32(math.sqrt(HI)))
    needles = []
    for _ in range(n_needles):
        b = int(g[3].integers(0, B))
        i = int(g[3].integers(0, n_q))
        p = q_pos0 + i
        if p - window < 0:
            continue
        h = int(torch.argmax(w[b, i]))
        if w[b, i, h] < 0.5:
            continue
        j = int(g[4].integers(0, p - window + 1))
        qd = qv[b, i, h]
        kv[b, j] = 8.0 * math.sqrt(dI) * qd / qd.norm()
        needles.append((b * n_q + i, h, j))
    qi, qs = quantize_e4m3(qv)
    ki, ks = quantize_e4m3(kv)
    return IndexerInputs(qi.contiguous(), qs.contiguous(), w.contiguous(), ki.contiguous(), ks.contiguous(), needles)
