"""Pins of the clustering oracle (query-geometry projection + k-means,
"OpenAttention" stage 01 and the settings list; readings G1-G4 in
oracle/qgc.py) against exactly rounded sums, exact rational arithmetic, the
defining properties of Lloyd's iteration and recovery of separated blobs; and
the measured effect of the fixed-point centroid sums (the GPU's form of the
mean) against the plain iteration with exactly rounded means."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import qgc


def _eye(d, r):
    V = np.zeros((d, r), np.float32)
    V[np.arange(r), np.arange(r)] = 1.0
    return V


def test_projection_hand_example_and_clamp():
    """G2: identity basis, so z = the first 16 key coordinates (exact), a
    coordinate beyond 2048 is clamped, dimensions past 16 are ignored."""
    K = np.zeros((4, 32), np.float32)
    K[:, 0] = [1.5, 2.0 ** -30, -2.25, 3000.0]
    K[:, 20] = 7.0
    z = qgc.project(K, _eye(32, 16))
    np.testing.assert_array_equal(z[:, 0], [1.5, 2.0 ** -30, -2.25, 2048.0])
    assert (z[:, 1:] == 0).all() and z.dtype == np.float64


def test_projection_against_exact_sum():
    rng = np.random.default_rng(0)
    K = rng.standard_normal((10, 128)).astype(np.float32)
    V = np.linalg.qr(rng.standard_normal((128, 16)))[0].astype(np.float32)
    z = qgc.project(K, V)
    for j in range(10):
        for i in range(16):
            exact = math.fsum(float(K[j, t]) * float(V[t, i]) for t in range(128))
            assert abs(z[j, i] - exact) <= 1e-13 * max(1.0, abs(exact))


@pytest.mark.parametrize("km", [qgc.kmeans, qgc.kmeans_plain])
def test_separated_blobs_recovered(km):
    """G3: C blobs far apart, each a contiguous run of rows, so the evenly
    spaced start takes one point per blob: every row ends in its blob's
    cluster, and the centroids are the blob means."""
    rng = np.random.default_rng(1)
    C, per, r = 8, 50, 16
    centres = rng.standard_normal((C, r)) * 100
    z = np.concatenate([centres[k] + rng.standard_normal((per, r)) * 0.1 for k in range(C)])
    a, cent, it = km(z, C, T=10)
    np.testing.assert_array_equal(a, np.repeat(np.arange(C), per))
    assert it <= 2
    for k in range(C):
        np.testing.assert_allclose(cent[k], z[k * per:(k + 1) * per].mean(axis=0), rtol=0, atol=1e-9)


def _exact_sq(zrow, c):
    return sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(zrow, c))


def test_fixed_point_centroids_exact_and_rows_nearest():
    """G3 (kmeans) at convergence: every centroid is its rows' mean of the
    coordinates rounded to 2^-32, to within one rounding of fp64 (rational
    arithmetic), and every sampled row sits at a centroid of least exact
    squared distance (up to the fp64 rounding of the distances)."""
    rng = np.random.default_rng(2)
    z = rng.standard_normal((600, 16)) * 3
    z[:300] += 8
    a, cent, it = qgc.kmeans(z, 6, T=100)
    assert it < 100
    for k in range(6):
        rows = z[a == k]
        if len(rows):
            for i in range(16):
                s = sum(int(v) for v in np.rint(rows[:, i] * 2.0 ** 32))
                mean = Fraction(s, len(rows)) / 2 ** 32
                assert abs(Fraction(cent[k, i]) - mean) <= abs(mean) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    for j in rng.choice(600, size=40, replace=False):
        d = [_exact_sq(z[j], cent[k]) for k in range(6)]
        assert d[a[j]] <= min(d) * (1 + Fraction(1, 10 ** 12))


def test_plain_centroids_are_exact_means():
    """G3 (kmeans_plain) at convergence: every centroid is its rows' exact
    mean to within one fp64 rounding of the division (rational arithmetic)."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal((400, 16)) * 2
    z[:150] -= 5
    a, cent, it = qgc.kmeans_plain(z, 5, T=100)
    assert it < 100
    for k in range(5):
        rows = z[a == k]
        for i in range(16):
            mean = sum(Fraction(float(v)) for v in rows[:, i]) / len(rows)
            assert abs(Fraction(cent[k, i]) - mean) <= abs(mean) * Fraction(1, 2 ** 51) + Fraction(1, 2 ** 1000)


@pytest.mark.parametrize("km", [qgc.kmeans, qgc.kmeans_plain])
def test_objective_never_increases(km):
    """Lloyd's objective does not increase from one iteration to the next (up
    to fp64 rounding)."""
    rng = np.random.default_rng(3)
    z = rng.standard_normal((400, 16)) * 5
    prev = None
    for T in range(1, 8):
        a, cent, _ = km(z, 5, T=T)
        obj = qgc.objective(z, a, cent)
        if prev is not None:
            assert obj <= prev * (1 + 1e-12)
        prev = obj


@pytest.mark.parametrize("km", [qgc.kmeans, qgc.kmeans_plain])
def test_degenerate_cluster_counts_and_empty_centroid(km):
    """C = 1: one cluster.  C = n with distinct points: every row its own
    cluster.  Two identical starting points: the tie goes to the lower k and
    the other centroid, left empty, stays at its starting point."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal((12, 16))
    a, _, _ = km(z, 1)
    assert (a == 0).all()
    a, _, _ = km(z, 12)
    np.testing.assert_array_equal(a, np.arange(12))
    z2 = z.copy()
    z2[3] = z2[9]                                  # starting rows of centroids 0 and 1 (n = 12, C = 2)
    a, cent, _ = km(z2, 2, T=1)
    assert (a == 0).all()
    assert cent[1].tolist() == z2[9].tolist()


def test_fixed_point_sums_match_the_plain_iteration_on_the_selector_workload():
    """The measured effect of the GPU's form of the mean: on units of the
    selector workload (batch-32 32K keys, C = 64, 10 passes) the k-means with
    fixed-point sums and the plain k-means with exactly rounded means put
    every row in the same cluster (n = 8192 rows per unit here, to keep the
    CPU suite short)."""
    from long_context_sparse_gathered_amd import synth
    w = synth.WORKLOADS["qgs_bf16_b32_n32k"].replace(n=8192)
    moved = []
    for s, g in [(0, 0), (5, 3)]:
        ud = synth.make_unit(w, s, g)
        z = qgc.project(ud.K, ud.U[:, :16])
        a_fix, _, _ = qgc.kmeans(z, 64, 10)
        a_pl, _, _ = qgc.kmeans_plain(z, 64, 10)
        moved.append(int((a_fix != a_pl).sum()))
    print(f"rows in another cluster than the plain iteration: {moved} of {w.n} per unit")
    assert max(moved) == 0
