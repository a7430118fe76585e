"""Pins of the clustering oracle (query-geometry projection + k-means,
"OpenAttention" stage 01 and the settings list; readings G1-G4 in
oracle/qgc.py) against hand-worked values, exactly rounded sums, exact
rational arithmetic and the defining properties of Lloyd's iteration."""
import math
from fractions import Fraction

import numpy as np

from oracle import qgc


def _eye(d, r):
    V = np.zeros((d, r), np.float32)
    V[np.arange(r), np.arange(r)] = 1.0
    return V


def test_fixed_point_hand_example():
    """G2: identity basis; 1.5 -> 6144; 2^-13 * 4096 = 0.5 -> 0 and
    3 * 2^-13 * 4096 = 1.5 -> 2 (half to even); -2.25 -> -9216; 3000 is
    clamped to 2^23 - 1."""
    K = np.zeros((5, 32), np.float32)
    K[:, 0] = [1.5, 2.0 ** -13, 3 * 2.0 ** -13, -2.25, 3000.0]
    K[:, 20] = 7.0                              # outside the 16 coordinates
    zq = qgc.project_fixed(K, _eye(32, 16))
    np.testing.assert_array_equal(zq[:, 0], [6144, 0, 2, -9216, (1 << 23) - 1])
    assert (zq[:, 1:] == 0).all() and zq.dtype == np.int64


def test_projection_against_exact_sum():
    rng = np.random.default_rng(0)
    K = rng.standard_normal((10, 128)).astype(np.float32)
    V = np.linalg.qr(rng.standard_normal((128, 16)))[0].astype(np.float32)
    zq = qgc.project_fixed(K, V)
    for j in range(10):
        for i in range(16):
            exact = math.fsum(float(K[j, t]) * float(V[t, i]) for t in range(128))
            assert abs(zq[j, i] - exact * 4096.0) <= 0.5 + 1e-9


def test_separated_blobs_recovered():
    """G3: C blobs far apart, each a contiguous run of rows, so the evenly
    spaced start takes one point per blob: every row ends in its blob's
    cluster, and the centroids are the blob means."""
    rng = np.random.default_rng(1)
    C, per, r = 8, 50, 16
    centres = rng.standard_normal((C, r)) * 1e6
    zq = np.concatenate([np.rint(centres[k] + rng.standard_normal((per, r)) * 10).astype(np.int64) for k in range(C)])
    a, cent, it = qgc.kmeans(zq, C, T=10)
    np.testing.assert_array_equal(a, np.repeat(np.arange(C), per))
    assert it <= 2
    for k in range(C):
        np.testing.assert_allclose(cent[k], zq[k * per:(k + 1) * per].mean(axis=0), rtol=0, atol=0.5)


def test_fixed_point_properties_exact():
    """G3 at convergence: every centroid is its rows' exact mean rounded half
    to even to the integer grid (rational arithmetic), and every sampled row
    sits at a centroid of least exact squared distance."""
    rng = np.random.default_rng(2)
    zq = rng.integers(-200000, 200000, size=(600, 16)).astype(np.int64)
    zq[:300] += 300000
    a, cent, it = qgc.kmeans(zq, 6, T=100)
    assert it < 100
    for k in range(6):
        rows = zq[a == k]
        if len(rows):
            for i in range(16):
                assert cent[k, i] == float(round(Fraction(int(rows[:, i].sum()), len(rows))))
    cf = [[Fraction(float(x)) for x in c] for c in cent]
    for j in rng.choice(600, size=40, replace=False):
        d = [sum((Fraction(int(zq[j, i])) - cf[k][i]) ** 2 for i in range(16)) for k in range(6)]
        assert d[a[j]] == min(d)


def test_objective_never_increases():
    """Lloyd's objective does not increase from one iteration to the next,
    up to the grid rounding of the centroids (each coordinate of a centroid
    moves at most 1/2 from the exact mean: at most 16 * 1/4 per row)."""
    rng = np.random.default_rng(3)
    zq = np.rint(rng.standard_normal((400, 16)) * 5e4).astype(np.int64)
    prev = None
    for T in range(1, 8):
        a, cent, _ = qgc.kmeans(zq, 5, T=T)
        obj = qgc.objective(zq, a, cent)
        if prev is not None:
            assert obj <= prev + 4 * len(zq)
        prev = obj


def test_degenerate_cluster_counts_and_empty_centroid():
    """C = 1: one cluster.  C = n with distinct points: every row its own
    cluster.  Two identical starting points: the tie goes to the lower k and
    the other centroid, left empty, stays at its starting point."""
    rng = np.random.default_rng(4)
    zq = rng.integers(-1000, 1000, size=(12, 16)).astype(np.int64)
    a, _, _ = qgc.kmeans(zq, 1)
    assert (a == 0).all()
    a, _, _ = qgc.kmeans(zq, 12)
    np.testing.assert_array_equal(a, np.arange(12))
    zq2 = zq.copy()
    zq2[3] = zq2[9]                                # starting rows of centroids 0 and 1 (n = 12, C = 2)
    a, cent, _ = qgc.kmeans(zq2, 2, T=1)
    assert (a == 0).all()
    assert cent[1].tolist() == zq2[9].astype(float).tolist()
