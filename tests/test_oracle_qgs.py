"""Pins of the selector oracle (QGS codes and scores, ErrorGate budgets,
per-cluster selection) against facts fixed outside it: hand-worked values,
exactly rounded sums, library routines and exact designs.

Source: "OpenAttention: One Percent Is Enough with Tail Proxies", method
stages 01-03 and the settings list; the readings Q1-Q7 are in oracle/qgs.py.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import qgs


def _eye_basis(d, r):
    U = np.zeros((d, r), np.float32)
    U[np.arange(r), np.arange(r)] = 1.0
    return U


def test_codes_hand_example():
    """Q3 on a worked example: identity basis, so y = the first r key
    coordinates.  Column 0: kmax 2, codes 127, rint(-63.5) = -64,
    rint(31.75) = 32; column 1 all zero: codes 0; column 2: +-127; column 3:
    kmax 254, 127 * 125 / 254 = 62.5 rounds to the even 62 (not 63)."""
    d, r = 8, 4
    K = np.zeros((3, d), np.float32)
    K[:, 0] = [2.0, -1.0, 0.5]
    K[:, 2] = [1.0, 1.0, -1.0]
    K[:, 3] = [254.0, 125.0, -254.0]
    K[:, 5] = [9.0, -9.0, 3.0]           # outside the subspace: ignored
    code, kmax = qgs.codes(K, _eye_basis(d, r))
    np.testing.assert_array_equal(kmax, [2.0, 0.0, 1.0, 254.0])
    np.testing.assert_array_equal(code, [[127, 0, 127, 127], [-64, 0, 127, 62], [32, 0, -127, -127]])
    assert code.dtype == np.int8


def test_projection_matches_exactly_rounded_sum():
    """Q2: each projection is within a few ulps of the exactly rounded dot
    product (math.fsum), with the basis applied as U^T k (not U k)."""
    rng = np.random.default_rng(0)
    d, r, n = 128, 32, 20
    K = rng.standard_normal((n, d)).astype(np.float32)
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    U = U.astype(np.float32)
    y = qgs.project(K, U)
    for j in range(n):
        for i in range(r):
            exact = math.fsum(float(K[j, t]) * float(U[t, i]) for t in range(d))
            assert abs(y[j, i] - exact) <= 1e-13 * max(1.0, abs(exact)), (j, i)


def test_projection_products_exact_for_bf16():
    """Q2: a bf16 key element times an fp32 basis entry is exact in fp64, so a
    one-term projection reproduces the exact rational product."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal(64).astype(np.float32)
    bits = ((k.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # some bf16 values
    u = rng.standard_normal(64).astype(np.float32)
    for t in range(64):
        K = np.zeros((1, 1), np.uint16)
        K[0, 0] = bits[t]
        y = qgs.project(K, np.array([[u[t]]], np.float32))[0, 0]
        kv = float((np.uint32(bits[t]) << 16).view(np.float32))
        assert Fraction(y) == Fraction(kv) * Fraction(float(u[t]))


def test_lossless_codes_give_exact_topk():
    """Q4 + Q7: with integer keys whose coordinate maxima are 127 and an
    integer query of max 127 in the identity basis, codes and query weights
    are the values themselves, so one cluster with budget E selects exactly
    the exact top-E rows by q.k (lexsort reference, ties to the lower
    position)."""
    rng = np.random.default_rng(2)
    d = 32
    n = 300
    K = rng.integers(-126, 127, size=(n, d)).astype(np.float32)
    K[0, :] = 127.0                      # every coordinate reaches 127 in row 0 (a sink row)
    q = rng.integers(-126, 127, size=(1, d)).astype(np.float32)
    q[0, 3] = 127.0
    U = _eye_basis(d, d)
    code, kmax = qgs.codes(K, U)
    np.testing.assert_array_equal(code.astype(np.float32), K)
    wq = qgs.query_weights(q, U, kmax)
    np.testing.assert_array_equal(wq.astype(np.float32), q)
    S = qgs.scores(code, wq)
    exact = (K.astype(np.int64) @ q[0].astype(np.int64))
    cid = np.zeros(n, np.int32)
    E, n_sink, n_local = 40, 4, 16
    idx = qgs.select(S, cid, [E], n_sink, n_local)
    pos = np.arange(n_sink, n - n_local)
    order = np.lexsort((pos, -exact[pos]))
    expect = np.sort(np.concatenate([np.arange(n_sink), pos[order[:E]], np.arange(n - n_local, n)]))
    np.testing.assert_array_equal(idx, expect)
    # top-1 of the middle is numpy's argmax (first occurrence on ties)
    one = qgs.select(S, cid, [1], n_sink, n_local)
    mid = [j for j in one if n_sink <= j < n - n_local]
    assert mid == [n_sink + int(np.argmax(exact[n_sink:n - n_local]))]


def test_scores_take_the_max_over_heads():
    """Q4: the group score is the larger of the heads' integer scores."""
    code = np.array([[1, 0], [0, 1], [1, 1]], np.int8)
    wq = np.array([[3, -1], [-2, 5]], np.int32)
    np.testing.assert_array_equal(qgs.scores(code, wq), [3, 5, 3])


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_logit_moments_exact_on_orthogonal_design():
    """Q5: members k_j = mu + a * h_j with h_j the rows of a Hadamard matrix
    (columns 1..d): the members' key covariance is exactly diag(a^2), so the
    mean logit and the diagonal logit variance equal the members' logit mean
    and (population) variance, computed directly."""
    rng = np.random.default_rng(3)
    d, N = 64, 128
    H = _hadamard(N)[:, 1:d + 1]
    mu = rng.standard_normal(d)
    a = rng.uniform(0.25, 2.0, size=d)
    K = (mu[None, :] + a[None, :] * H).astype(np.float64)
    q = rng.standard_normal((3, d)).astype(np.float32)
    scale = 0.125
    Nb, S1, S2 = np.array([N]), K.sum(axis=0)[None], (K * K).sum(axis=0)[None]
    zbar, s2 = qgs.logit_moments(q, Nb, S1, S2, scale)
    logits = float(np.float32(scale)) * (K @ q.astype(np.float64).T)      # [N, 3]
    np.testing.assert_allclose(zbar[0], logits.mean(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2[0], logits.var(axis=0), rtol=1e-10)


def test_weight_error_zero_for_identical_members():
    """Q5: a cluster whose members share one key has no logit spread, so the
    proxy is exact and its weight error is 0; the other cluster carries all
    the error."""
    rng = np.random.default_rng(4)
    d = 16
    k0 = rng.standard_normal(d).astype(np.float32)
    K = np.concatenate([np.repeat(k0[None], 50, axis=0), rng.standard_normal((70, d)).astype(np.float32)])
    cid = np.array([0] * 50 + [1] * 70, np.int32)
    q = rng.standard_normal((2, d)).astype(np.float32)
    N, S1, S2 = qgs.cluster_stats(K, cid, 2)
    eps = qgs.weight_errors(q, N, S1, S2, 0.25)
    assert eps[0] == 0.0 and eps[1] > 0.0


def test_weight_error_invariant_to_replicating_members():
    """Q5: repeating every member of every cluster k times keeps means and
    variances and scales all counts alike, so eps is unchanged."""
    rng = np.random.default_rng(5)
    d, n, C = 16, 90, 3
    K = rng.standard_normal((n, d)).astype(np.float32)
    cid = rng.integers(0, C, size=n).astype(np.int32)
    q = rng.standard_normal((2, d)).astype(np.float32)
    e1 = qgs.weight_errors(q, *qgs.cluster_stats(K, cid, C), 0.3)
    e3 = qgs.weight_errors(q, *qgs.cluster_stats(np.tile(K, (3, 1)), np.tile(cid, 3), C), 0.3)
    np.testing.assert_allclose(e3, e1, rtol=1e-9)
    assert (e1 > 0).all() and e1.sum() < q.shape[0]


def test_weight_error_two_cluster_closed_form():
    """Q5 against a hand-derived value: one head, scale 1, d = 1.  Cluster 0:
    members +-1 (N = 2, mean 0, variance 1) with q = 1: zbar = 0, s2 = 1,
    e = 2 (e^{1/2} - 1), weight 2 e^{1/2}.  Cluster 1: two members at 0:
    weight 2, error 0.  eps_0 = 2 (e^{1/2} - 1) / (2 e^{1/2} + 2)."""
    K = np.array([[1.0], [-1.0], [0.0], [0.0]], np.float32)
    cid = np.array([0, 0, 1, 1], np.int32)
    eps = qgs.weight_errors(np.array([[1.0]], np.float32), *qgs.cluster_stats(K, cid, 2), 1.0)
    e = math.exp(0.5)
    assert eps[1] == 0.0
    assert abs(eps[0] - 2 * (e - 1) / (2 * e + 2)) < 1e-15


@pytest.mark.parametrize("eps,avail,E,expect", [
    ([1, 1, 1], [100, 100, 100], 10, [4, 3, 3]),            # equal remainders: lower b first
    ([0.5, 0.25, 0.25], [100, 100, 100], 7, [3, 2, 2]),      # 3.5, 1.75, 1.75
    ([10, 1, 1], [2, 100, 100], 10, [2, 4, 4]),              # cap 2, the other 8 split evenly
    ([0, 0, 0], [1, 2, 3], 4, [1, 1, 2]),                    # no error anywhere: capacity weights
    ([3, 1, 0], [5, 5, 5], 30, [5, 5, 5]),                   # budget above capacity
    ([1, 0, 2], [10, 10, 0], 6, [6, 0, 0]),                  # no capacity, no share
])
def test_allocation_hand_cases(eps, avail, E, expect):
    q, _ = qgs.allocate(np.array(eps, float), np.array(avail), E)
    np.testing.assert_array_equal(q, expect)


def test_allocation_properties():
    """Q6 on random inputs: the budget is spent up to the capacity, no cluster
    exceeds its capacity, and without caps every q_b is its quota rounded up
    or down."""
    rng = np.random.default_rng(6)
    for _ in range(300):
        C = int(rng.integers(1, 40))
        eps = rng.exponential(size=C) * (rng.random(C) < 0.8)
        avail = rng.integers(0, 30, size=C)
        E = int(rng.integers(0, 400))
        q, _ = qgs.allocate(eps, avail, E)
        assert q.sum() == min(E, avail.sum())
        assert (q <= avail).all() and (q >= 0).all()
        if (avail >= E).all() and eps.sum() > 0:
            quota = E * eps / eps.sum()
            assert (np.abs(q - quota) < 1 + 1e-9).all()


def test_select_hand_example():
    """Q7 on a worked example: n = 12, sink 2, local 2; cluster 0 = rows 0-5,
    cluster 1 = rows 6-11, row 7 in no cluster.  Cluster 0 (eligible 2-5,
    scores 5, 9, 9, 1) with q = 2 takes rows 3 and 4 (tie at 9 both taken);
    cluster 1 (eligible 6, 8, 9; scores 4, 4, 7) with q = 2 takes 9 and then
    6 (the tie at 4 goes to the lower position)."""
    S = np.array([0, 0, 5, 9, 9, 1, 4, 100, 4, 7, 0, 0])
    cid = np.array([0, 0, 0, 0, 0, 0, 1, -1, 1, 1, 1, 1])
    idx = qgs.select(S, cid, [2, 2], 2, 2)
    np.testing.assert_array_equal(idx, [0, 1, 3, 4, 6, 9, 10, 11])
    idx = qgs.select(S, cid, [1, 1], 2, 2)
    np.testing.assert_array_equal(idx, [0, 1, 3, 9, 10, 11])


def test_select_unit_shapes_and_budget():
    """The whole selector on a small random unit: the index set holds sink,
    local and exactly sum(q_b) selected rows, each in its own cluster's
    eligible range."""
    rng = np.random.default_rng(7)
    n, d, C, E = 2000, 128, 8, 60
    K = (rng.standard_normal((n, d)) + 0.5).astype(np.float32)
    cid = np.repeat(np.arange(C), n // C).astype(np.int32)
    U, _ = np.linalg.qr(rng.standard_normal((d, 32)))
    q = rng.standard_normal((4, d)).astype(np.float32)
    r = qgs.select_unit(q, K, cid, C, U.astype(np.float32), 4, 64, E, 1 / np.sqrt(d))
    idx = r["idx"]
    assert r["budget"].sum() == E
    assert len(idx) == 4 + 64 + E and (np.diff(idx) > 0).all()
    mid = idx[(idx >= 4) & (idx < n - 64)]
    for b in range(C):
        assert ((cid[mid] == b).sum()) == r["budget"][b]


def test_plain_scores_rank_like_the_logits_for_lossless_codes():
    """Q4 plain reading: keys inside span(U) whose projections sit on the code
    grid are coded without loss, so the plain score of a row is its largest
    logit over the group up to one positive factor: the top-k by plain score
    is the exact top-k by max_h <q_h, k_j> (lexsort reference, ties to the
    lower position)."""
    rng = np.random.default_rng(11)
    d, r, n, G = 64, 32, 300, 4
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    U = U.astype(np.float32)
    cgrid = rng.integers(-127, 128, size=(n, r))
    cgrid[0, :] = 127                                  # every column reaches the code maximum
    K = (cgrid.astype(np.float64) / 127.0) @ U.astype(np.float64).T     # projections = code / 127
    code, kmax = qgs.codes(K.astype(np.float64), U)
    np.testing.assert_array_equal(code.astype(np.int64), cgrid)
    q = rng.standard_normal((G, d)).astype(np.float32)
    S = qgs.scores_plain(code, q, U, kmax)
    logits = (K @ q.astype(np.float64).T).max(axis=1)
    order = np.lexsort((np.arange(n), -logits))
    top = np.sort(order[:40])
    order_s = np.lexsort((np.arange(n), -S))
    np.testing.assert_array_equal(np.sort(order_s[:40]), top)


def test_plain_and_integer_scores_agree_when_the_query_weights_are_integral():
    """When 127 * w / max|w| is already integral the integer weights are the
    plain weights up to one factor, so both readings list the same rows."""
    rng = np.random.default_rng(12)
    d, r, n = 64, 32, 400
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    U = U.astype(np.float32)
    K = rng.standard_normal((n, d)).astype(np.float32)
    code, kmax = qgs.codes(K, U)
    # a query whose projection is chosen so that w = qt * kmax is a multiple of wmax / 127
    target = rng.integers(-127, 128, size=(1, r)).astype(np.float64)
    target[0, 0] = 127
    qt = target / kmax[None, :]
    q = (qt @ U.astype(np.float64).T).astype(np.float32)
    wq = qgs.query_weights(q, U, kmax)
    S_int = qgs.scores(code, wq)
    S_pl = qgs.scores_plain(code, q, U, kmax)
    top_int = np.lexsort((np.arange(n), -S_int))[:50]
    top_pl = np.lexsort((np.arange(n), -S_pl))[:50]
    # the float query is within rounding of the target, so compare the sets away from near-ties
    gap = np.sort(S_pl)[::-1]
    if abs(gap[49] - gap[50]) > 1e-6 * abs(gap[0]):
        np.testing.assert_array_equal(np.sort(top_int), np.sort(top_pl))


def test_plain_scores_invariant_to_query_scale():
    rng = np.random.default_rng(13)
    d, r, n = 64, 32, 200
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    U = U.astype(np.float32)
    K = rng.standard_normal((n, d)).astype(np.float32)
    code, kmax = qgs.codes(K, U)
    q = rng.standard_normal((2, d)).astype(np.float32)
    a = np.lexsort((np.arange(n), -qgs.scores_plain(code, q, U, kmax)))[:30]
    b = np.lexsort((np.arange(n), -qgs.scores_plain(code, q * np.float32(4.0), U, kmax)))[:30]
    np.testing.assert_array_equal(a, b)


def test_integer_query_weights_move_few_listed_rows_on_the_selector_workload():
    """The measured effect of rounding the query weights (reading Q4) on units
    of the selector workload (n = 8192 rows here, 260 rows picked): the rows
    listed by the integer scores against the plain fp64 scores, same budgets.
    The selector notes record the numbers (2-4 of 260 on full 32K units)."""
    from long_context_sparse_gathered_amd import synth
    w = synth.WORKLOADS["qgs_bf16_b32_n32k"].replace(n=8192)
    sc = np.float32(1.0 / np.sqrt(w.d))
    moved = []
    for s, g in [(0, 0), (3, 5), (9, 1), (17, 6)]:
        ud = synth.make_unit(w, s, g)
        a = qgs.select_unit(ud.q, ud.K, ud.cid, w.C, ud.U, w.n_sink, w.n_local, w.n_top, sc)
        b = qgs.select_unit_plain(ud.q, ud.K, ud.cid, w.C, ud.U, w.n_sink, w.n_local, w.n_top, sc)
        np.testing.assert_array_equal(a["budget"], b["budget"])
        moved.append(len(np.setdiff1d(b["idx"], a["idx"])))
    print(f"listed rows that the integer query weights move: {moved} of {w.n_top} per unit")
    assert max(moved) <= 0.03 * w.n_top
