"""Clustering oracle: query-geometry projection of the keys and k-means on
it.  Plain numpy; fp64 where the method has real arithmetic, exact integers
for the sums.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does.  It
imports nothing from the product package and shares no code with it.

Source: "OpenAttention: One Percent Is Enough with Tail Proxies"
(ai-frontier-tracker summary), stage 01 of the four-stage method list (keys
projected onto the top 16 query eigenvectors are clustered with k-means; each
cluster caches a count, a mean token and a diagonal-variance token) and the
settings list (QGC rank r = 16, C = 64 clusters).

The page names the steps, not their details.  Readings (also in the design
notes):
  G1  The basis is an input: V [d, 16] with orthonormal columns, the leading
      16 columns of the query subspace basis the selector uses.
  G2  Projection z_j = V^T k_j, summed over d in index order in fp64 (every
      product of a bf16/fp32 element and an fp32 basis entry is exact), then
      held in fixed point: zq_j = rint(z_j * 2^12) as an integer (round half
      to even), clamped to |zq| <= 2^23 - 1 (|z| < 2048; larger projections
      are flagged on the GPU).  Integer coordinates make every centroid sum
      exact.
  G3  k-means (Lloyd's iteration) on zq with C centroids held in the same
      fixed point as the points.  Start: centroid k is the point of row
      floor((2k + 1) n / (2C)).  One iteration: each row goes to the centroid
      at the smallest squared distance sum_i (zq_i - c_ki)^2 (ties to the
      lower k); each centroid becomes its rows' mean rounded to the grid,
      rint(S / N) with S the exact integer sum (round half to even); a
      centroid with no rows stays where it is.  T iterations (default 10),
      stopping early once no row changes its centroid (a fixed point).
      Points and centroids are integers below 2^23, so every distance is an
      integer below 2^52 and exact in fp64 in any order; and fp64(S)/fp64(N)
      rounds to the same integer as the exact S/N (an exact quotient that is
      not a half-integer lies at least 1/(2N) from one, far above the
      division's rounding error).
  G4  The cluster id of a row is its final centroid.  The per-cluster state
      (count, key sum, value sum, squared-key sum) is then the proxy
      builder's, over these ids.
"""
from __future__ import annotations

import numpy as np

R_QGC = 16          # projection rank (settings list)
FIX_SCALE = 4096.0  # fixed-point scale of the projected coordinates
FIX_MAX = (1 << 23) - 1
T_DEFAULT = 10


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def project_fixed(K, V) -> np.ndarray:
    """G2: integer coordinates zq [n, r] (int64) of one unit's keys."""
    X, Vv = _f64(K), np.asarray(V, dtype=np.float32).astype(np.float64)
    z = np.zeros((X.shape[0], Vv.shape[1]))
    for dd in range(X.shape[1]):
        z += X[:, dd:dd + 1] * Vv[dd][None, :]
    return np.clip(np.rint(z * FIX_SCALE), -FIX_MAX, FIX_MAX).astype(np.int64)


def init_centroids(zq, C) -> np.ndarray:
    n = zq.shape[0]
    rows = (2 * np.arange(C) + 1) * n // (2 * C)
    return zq[rows].astype(np.float64)


def sq_distances(zq, cent) -> np.ndarray:
    """[n, C] squared distances (integers below 2^52: exact in fp64)."""
    zf = zq.astype(np.float64)
    D = np.zeros((zq.shape[0], cent.shape[0]))
    for i in range(zq.shape[1]):
        diff = zf[:, i:i + 1] - cent[None, :, i]
        D = D + diff * diff
    return D


def assign(zq, cent) -> np.ndarray:
    return np.argmin(sq_distances(zq, cent), axis=1).astype(np.int32)   # first minimum: lower k


def update(zq, a, cent) -> np.ndarray:
    """Each centroid = rint(exact integer sum of its rows / count); empty
    centroids stay."""
    C, r = cent.shape
    new = cent.copy()
    for k in range(C):
        m = a == k
        cnt = int(m.sum())
        if cnt:
            s = zq[m].sum(axis=0)          # int64, exact
            new[k] = np.rint(s.astype(np.float64) / float(cnt))
    return new


def kmeans(zq, C, T=T_DEFAULT):
    """G3: returns (assignment [n] int32, centroids [C, r] fp64, iterations run)."""
    cent = init_centroids(zq, C)
    a = None
    it = 0
    for it in range(1, T + 1):
        a_new = assign(zq, cent)
        if a is not None and np.array_equal(a_new, a):
            return a, cent, it - 1
        a = a_new
        cent = update(zq, a, cent)
    return a, cent, it


def objective(zq, a, cent) -> float:
    d = zq.astype(np.float64) - cent[a]
    return float((d * d).sum())


def cluster_unit(K, V16, C, T=T_DEFAULT):
    """G1-G4 for one unit: cluster ids [n] int32."""
    zq = project_fixed(K, V16)
    a, _, _ = kmeans(zq, C, T)
    return a
