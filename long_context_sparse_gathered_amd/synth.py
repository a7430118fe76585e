"""Seeded synthetic workloads for sparse decode attention.

This module only *makes inputs*: the KV cache, the decode queries, the
selected index set, the cluster assignment and the prefill mean query.  It
holds none of the attention/tail arithmetic; the HIP library and the CPU
oracle both consume exactly the arrays produced here.

Recipe (one independent generator per (sequence, KV head) unit, so that any
unit can be regenerated alone):

* rng = numpy ``default_rng([seed, s, g])``; structure draws (heavy-hitter
  positions, cluster cut points) use ``default_rng([seed, s, g, 1])``.
* key bias beta = 4 * (random unit vector); K = N(0,1) + beta; V = N(0,1).
* query heads q_h ~ N(0,1) (prior workload: q_h = m_h + N(0,1) with
  m_h = 3 * random unit vector, and mu_Q_h = the fp32 mean of 2048 prefill
  queries m_h + N(0,1)).  Selector workloads (r > 0) plant a query geometry:
  U = the Q factor of a d x r Gaussian matrix (orthonormal columns, fp32) and
  q_h = sqrt(d/r) * U z_h + 0.25 * N(0,1), z_h ~ N(0,1)^r, so that most of
  every query lies in span(U), the subspace the selector scores in.
* 8 heavy hitters at distinct positions in [n_sink, n - n_local): the row is
  replaced by t * sqrt(d) * qbar / <qbar, qbar> with t ~ U(11, 13) and qbar
  the group-mean query, so the scaled logit of qbar against it is t.
* Everything is rounded to the workload dtype (bf16 round-to-nearest-even)
  before any selection is made.
* Index set = sink [0, n_sink) + local window [n - n_local, n) + the n_top
  positions in between with the largest score max_h scale*<q_h, k_j>
  (fp64; ties go to the lower position), sorted ascending.  This is the
  selector that sits in front of the attention kernel, not part of it.
* Clusters: 'equal' = C contiguous equal segments; 'random' = C contiguous
  segments cut at C-1 distinct uniform positions in [1, n-1].

The workloads mirror the pages' decode settings (Llama-3.1-8B shape: 32 query
heads over 8 KV heads, d = 128, bf16) at 4K / 32K / 64K / 128K context.  They
stand in for the long-context benchmarks the pages evaluate on (RULER,
LongBench), whose data and model weights are not used.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from statistics import NormalDist

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    n: int
    d: int
    dtype: str          # "bf16" or "f32"
    n_sink: int
    n_local: int
    n_top: int
    tail: str           # "proxy", "sampled", "prior" or "none"
    seed: int
    C: int = 0          # clusters per unit (proxy tail)
    seg: str = "equal"  # "equal" or "random"
    n_heavy: int = 8
    b0: int = 64        # sampled tail: base draws
    eps: float = 0.05
    delta: float = 0.05
    sampler_seed: int = 4004
    n_prefill: int = 2048   # prior tail: prefill queries behind mu_Q
    muq_norm: float = 3.0
    lam: float = 1.0
    r: int = 0              # selector workloads: rank of the query subspace

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def m(self) -> int:
        return self.n_sink + self.n_local + self.n_top

    @property
    def z(self) -> float:
        """Phi^-1(1 - delta/2), the two-sided normal quantile."""
        return NormalDist().inv_cdf(1.0 - self.delta / 2.0)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _pct(n: int, frac: float) -> int:
    return int(np.ceil(n * frac - 1e-9))


WORKLOADS = {
    # single head, fp32, 4K: 4 sink + 64 local + top-128, 16 equal clusters
    "proxy_f32_b1_n4k": Workload("proxy_f32_b1_n4k", 1, 1, 1, 4096, 128, "f32", 4, 64, 128, "proxy", seed=1, C=16, seg="equal"),
    # 8B decode shape, batch 1, 32K, 1% read (328), 32 random contiguous clusters
    "proxy_bf16_b1_n32k": Workload("proxy_bf16_b1_n32k", 1, 32, 8, 32768, 128, "bf16", 4, 64, _pct(32768, 0.01) - 68, "proxy",
                   seed=2, C=32, seg="random"),
    # the same at batch 32
    "proxy_bf16_b32_n32k": Workload("proxy_bf16_b32_n32k", 32, 32, 8, 32768, 128, "bf16", 4, 64, _pct(32768, 0.01) - 68, "proxy",
                   seed=3, C=32, seg="random"),
    # sampled tail: batch 8, 64K, I_f = 4 + 128 + 1% top-k
    "sampled_bf16_b8_n64k": Workload("sampled_bf16_b8_n64k", 8, 32, 8, 65536, 128, "bf16", 4, 128, _pct(65536, 0.01), "sampled", seed=4),
    # rank-1 prior: batch 16, 128K, 3% read
    "prior_bf16_b16_n128k": Workload("prior_bf16_b16_n128k", 16, 32, 8, 131072, 128, "bf16", 4, 64, _pct(131072, 0.03) - 68, "prior", seed=5),
    # selector in front of the proxy decode: the batch-32 32K shape, queries
    # in a rank-32 subspace, 32 random contiguous clusters, 260 rows to pick
    "qgs_bf16_b32_n32k": Workload("qgs_bf16_b32_n32k", 32, 32, 8, 32768, 128, "bf16", 4, 64, _pct(32768, 0.01) - 68, "proxy",
                   seed=6, C=32, seg="random", r=32),
}


# ---------------------------------------------------------------------------
# dtype handling

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Returns (stored array, its exact fp32 value)."""
    if dtype == "bf16":
        bits = round_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    x = np.ascontiguousarray(x, dtype=np.float32)
    return x, x


def _unit_vec(rng, d):
    v = rng.standard_normal(d)
    return v / np.linalg.norm(v)


# ---------------------------------------------------------------------------
# one unit

@dataclasses.dataclass
class UnitData:
    K: np.ndarray            # [n, d] uint16 bits or float32
    V: np.ndarray            # [n, d]
    q: np.ndarray            # [G, d]
    idx: np.ndarray          # [m] int32 sorted
    cid: np.ndarray | None   # [n] int32
    mu_Q: np.ndarray | None  # [G, d] float32
    heavy: np.ndarray        # [n_heavy] positions
    U: np.ndarray | None = None   # [d, r] float32 (selector workloads)


def select_index_set(Kf: np.ndarray, qf: np.ndarray, n_sink: int, n_local: int, n_top: int,
                     scale: float) -> np.ndarray:
    """sink + local + top-k by max_h scale*<q_h,k_j> over the middle range (fp64)."""
    n = Kf.shape[0]
    lo, hi = n_sink, n - n_local
    assert 0 <= lo <= hi <= n and n_top <= hi - lo
    score = (Kf[lo:hi].astype(np.float64) @ qf.astype(np.float64).T * float(scale)).max(axis=1)
    pos = np.arange(lo, hi)
    order = np.lexsort((pos, -score))  # descending score, then ascending position
    top = pos[order[:n_top]]
    idx = np.concatenate([np.arange(0, lo), top, np.arange(hi, n)])
    return np.sort(idx).astype(np.int32)


def make_clusters(rng, n: int, C: int, seg: str) -> np.ndarray:
    if seg == "equal":
        assert n % C == 0
        return (np.arange(n) // (n // C)).astype(np.int32)
    cuts = np.sort(rng.choice(np.arange(1, n), size=C - 1, replace=False))
    return np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32)


def make_unit(w: Workload, s: int, g: int) -> UnitData:
    rng = np.random.default_rng([w.seed, s, g])
    srng = np.random.default_rng([w.seed, s, g, 1])
    n, d, G = w.n, w.d, w.G
    scale = np.float32(1.0 / np.sqrt(d))

    beta = 4.0 * _unit_vec(rng, d)
    Kf = rng.standard_normal((n, d), dtype=np.float32)
    Kf += beta.astype(np.float32)
    Vf = rng.standard_normal((n, d), dtype=np.float32)

    mu_Q = None
    if w.tail == "prior":
        mean = np.stack([w.muq_norm * _unit_vec(rng, d) for _ in range(G)])          # [G, d]
        pre = mean[:, None, :] + rng.standard_normal((G, w.n_prefill, d))           # [G, P, d]
        _, pre_f = _to_dtype(pre.astype(np.float32), w.dtype)
        mu_Q = pre_f.astype(np.float64).mean(axis=1).astype(np.float32)
        q_raw = (mean + rng.standard_normal((G, d))).astype(np.float32)
    elif w.r > 0:
        U = np.linalg.qr(rng.standard_normal((d, w.r)))[0].astype(np.float32)
        z = rng.standard_normal((G, w.r))
        q_raw = (np.sqrt(d / w.r) * z @ U.T.astype(np.float64) + 0.25 * rng.standard_normal((G, d))).astype(np.float32)
    else:
        q_raw = rng.standard_normal((G, d), dtype=np.float32)
    q, qf = _to_dtype(q_raw, w.dtype)

    heavy = np.sort(srng.choice(np.arange(w.n_sink, n - w.n_local), size=w.n_heavy, replace=False))
    qbar = qf.astype(np.float64).mean(axis=0)
    t = srng.uniform(11.0, 13.0, size=w.n_heavy)
    Kf[heavy] = (t[:, None] * np.sqrt(d) * qbar[None, :] / (qbar @ qbar)).astype(np.float32)

    K, Kf = _to_dtype(Kf, w.dtype)
    V, _ = _to_dtype(Vf, w.dtype)
    idx = select_index_set(Kf, qf, w.n_sink, w.n_local, w.n_top, scale)
    cid = make_clusters(srng, n, w.C, w.seg) if w.C > 0 else None
    return UnitData(K=K, V=V, q=q, idx=idx, cid=cid, mu_Q=mu_Q, heavy=heavy, U=U if w.r > 0 else None)


# ---------------------------------------------------------------------------
# whole workload

@dataclasses.dataclass
class Case:
    w: Workload
    q: np.ndarray            # [B, Hq, d]
    K: np.ndarray            # [B, Hkv, n, d]
    V: np.ndarray
    idx: np.ndarray          # [B, Hkv, m] int32
    cid: np.ndarray | None   # [B, Hkv, n] int32
    mu_Q: np.ndarray | None  # [B, Hq, d] float32
    U: np.ndarray | None = None   # [B, Hkv, d, r] float32 (selector workloads)

    @property
    def idx_cluster(self) -> np.ndarray:
        """cluster id of every listed row, [B, Hkv, m] (what a per-cluster selector emits)."""
        return np.take_along_axis(self.cid, self.idx.astype(np.int64), axis=2).astype(np.int32)


def make_case(w: Workload, threads: int | None = None) -> Case:
    B, Hkv, G, n, d, m = w.B, w.Hkv, w.G, w.n, w.d, w.m
    st = np.uint16 if w.dtype == "bf16" else np.float32
    K = np.empty((B, Hkv, n, d), st)
    V = np.empty((B, Hkv, n, d), st)
    q = np.empty((B, w.Hq, d), st)
    idx = np.empty((B, Hkv, m), np.int32)
    cid = np.empty((B, Hkv, n), np.int32) if w.C > 0 else None
    mu_Q = np.empty((B, w.Hq, d), np.float32) if w.tail == "prior" else None
    U = np.empty((B, Hkv, d, w.r), np.float32) if w.r > 0 else None

    def fill(u):
        s, g = divmod(u, Hkv)
        ud = make_unit(w, s, g)
        K[s, g], V[s, g] = ud.K, ud.V
        q[s, g * G:(g + 1) * G] = ud.q
        idx[s, g] = ud.idx
        if cid is not None:
            cid[s, g] = ud.cid
        if mu_Q is not None:
            mu_Q[s, g * G:(g + 1) * G] = ud.mu_Q
        if U is not None:
            U[s, g] = ud.U

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and B * Hkv > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(B * Hkv)))
    else:
        for u in range(B * Hkv):
            fill(u)
    return Case(w=w, q=q, K=K, V=V, idx=idx, cid=cid, mu_Q=mu_Q, U=U)


def index_sets(c: Case, n_top: int, threads: int | None = None) -> np.ndarray:
    """The index sets [B, Hkv, n_sink + n_local + n_top] of case c for another
    top-k count.  K, V, q and the clusters of a unit do not depend on n_top,
    so these are the lists make_case would give for w.replace(n_top=n_top)."""
    w = c.w
    m = w.n_sink + w.n_local + n_top
    idx = np.empty((w.B, w.Hkv, m), np.int32)
    scale = np.float32(1.0 / np.sqrt(w.d))

    def fill(u):
        s, g = divmod(u, w.Hkv)
        Kf = bf16_bits_to_f32(c.K[s, g]) if c.K.dtype == np.uint16 else c.K[s, g]
        qs = c.q[s, g * w.G:(g + 1) * w.G]
        qf = bf16_bits_to_f32(qs) if qs.dtype == np.uint16 else qs
        idx[s, g] = select_index_set(Kf, qf, w.n_sink, w.n_local, n_top, scale)

    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, range(w.B * w.Hkv)))
    return idx


def unit_case(w: Workload, s: int, g: int) -> Case:
    """One unit as a B=1, Hkv=1 case (same values as in the full workload)."""
    ud = make_unit(w, s, g)
    w1 = w.replace(B=1, Hq=w.G, Hkv=1)
    return Case(w=w1, q=ud.q[None], K=ud.K[None, None], V=ud.V[None, None], idx=ud.idx[None, None],
                cid=None if ud.cid is None else ud.cid[None, None],
                mu_Q=None if ud.mu_Q is None else ud.mu_Q[None],
                U=None if ud.U is None else ud.U[None, None])
