"""Clustering oracle: query-geometry projection of the keys and k-means on
it.  Plain numpy in fp64.

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
      product of a bf16/fp32 element and an fp32 basis entry is exact), kept
      as fp64 coordinates.  A coordinate beyond +-2048 (a key of norm above
      2048) is clamped there and flagged on the GPU, so that the sums below
      stay within 64-bit integers.
  G3  Lloyd's k-means with C centroids.  Start: centroid k is the point of
      row floor((2k + 1) n / (2C)).  One iteration: each row goes to the
      centroid at the smallest squared distance sum_i (z_i - c_ki)^2, the
      terms added in coordinate order (ties to the lower k); each centroid
      becomes its rows' mean; a centroid with no rows stays where it is.
      T iterations (default 10), stopping early at a fixed point.
        kmeans_plain: the mean is the exactly rounded fp64 mean (an exactly
          rounded sum per coordinate, divided by the count).
        kmeans: the mean as the GPU forms it -- each coordinate rounded to
          the grid 2^-32 and summed as an exact 64-bit integer (so the sum
          is the same in any order), then (sum / count) * 2^-32 in fp64.
          It lies within 2^-33 of the plain mean; the tests measure that the
          two give the same clusters.
      (An earlier reading rounded the coordinates and the centroids to a
      2^-12 grid; on the selector workload that moved about 4% of the rows
      to other clusters than the plain iteration, so it was dropped.)
  G4  The cluster id of a row is its final centroid.  The per-cluster state
      (count, key sum, value sum, squared-key sum) is then the proxy
      builder's, over these ids.
"""
from __future__ import annotations

import math

import numpy as np

R_QGC = 16            # projection rank (settings list)
Z_MAX = 2048.0        # coordinate clamp (keeps the fixed-point sums in int64)
SUM_SCALE = 2.0 ** 32  # grid of the centroid sums (kmeans)
T_DEFAULT = 10


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def project(K, V) -> np.ndarray:
    """G2: coordinates z [n, r] (fp64) of one unit's keys."""
    X, Vv = _f64(K), np.asarray(V, dtype=np.float32).astype(np.float64)
    z = np.zeros((X.shape[0], Vv.shape[1]))
    for dd in range(X.shape[1]):
        z += X[:, dd:dd + 1] * Vv[dd][None, :]
    return np.clip(z, -Z_MAX, Z_MAX)


def init_centroids(z, C) -> np.ndarray:
    n = z.shape[0]
    rows = (2 * np.arange(C) + 1) * n // (2 * C)
    return z[rows].astype(np.float64)


def sq_distances(z, cent) -> np.ndarray:
    """[n, C] squared distances, the terms added in coordinate order."""
    D = np.zeros((z.shape[0], cent.shape[0]))
    for i in range(z.shape[1]):
        diff = z[:, i:i + 1] - cent[None, :, i]
        D = D + diff * diff
    return D


def assign(z, cent) -> np.ndarray:
    return np.argmin(sq_distances(z, cent), axis=1).astype(np.int32)   # first minimum: lower k


def update_fixed(z, a, cent) -> np.ndarray:
    """G3 (kmeans): means from exact integer sums of the coordinates on the
    2^-32 grid; empty centroids stay."""
    C = cent.shape[0]
    new = cent.copy()
    zz = np.rint(z * SUM_SCALE).astype(np.int64)      # |z| <= 2^11: exact, below 2^43
    for k in range(C):
        m = a == k
        cnt = int(m.sum())
        if cnt:
            s = zz[m].sum(axis=0)                     # int64, exact for n <= 2^20
            new[k] = (s.astype(np.float64) / float(cnt)) * (1.0 / SUM_SCALE)
    return new


def update_plain(z, a, cent) -> np.ndarray:
    """G3 (kmeans_plain): exactly rounded fp64 means; empty centroids stay."""
    C, r = cent.shape
    new = cent.copy()
    for k in range(C):
        rows = z[a == k]
        if len(rows):
            new[k] = [math.fsum(rows[:, i].tolist()) / len(rows) for i in range(r)]
    return new


def _lloyd(z, C, T, update):
    cent = init_centroids(z, C)
    a = None
    it = 0
    for it in range(1, T + 1):
        a_new = assign(z, cent)
        if a is not None and np.array_equal(a_new, a):
            return a, cent, it - 1
        a = a_new
        cent = update(z, a, cent)
    return a, cent, it


def kmeans(z, C, T=T_DEFAULT):
    """G3 as the GPU computes it: (assignment [n] int32, centroids [C, r],
    iterations run)."""
    return _lloyd(z, C, T, update_fixed)


def kmeans_plain(z, C, T=T_DEFAULT):
    """G3 with exactly rounded means (the plain iteration)."""
    return _lloyd(z, C, T, update_plain)


def objective(z, a, cent) -> float:
    d = z - cent[a]
    return float((d * d).sum())


def cluster_unit(K, V16, C, T=T_DEFAULT):
    """G1-G4 for one unit as the GPU computes it: cluster ids [n] int32."""
    a, _, _ = kmeans(project(K, V16), C, T)
    return a


def cluster_unit_plain(K, V16, C, T=T_DEFAULT):
    a, _, _ = kmeans_plain(project(K, V16), C, T)
    return a
