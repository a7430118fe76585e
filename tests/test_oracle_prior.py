"""Pins for the oracle's rank-1 prior (RESA page, sections "Prior Estimator"
and "Online Aggregator").

The plain O(n) definition (listed rows exact, unlisted rows weighted by
lambda * exp(P_j + c)) and the O(|I|) delta merge are independent codings of
the same quantity; their agreement over every subset of a small cache is one
pin.  The others are the special cases the pages state or imply.
"""
import itertools

import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import synth


def _rand(rng, B, Hq, Hkv, n, d, kshift=0.3):
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    K = (rng.standard_normal((B, Hkv, n, d)) + kshift).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    muQ = (q + 0.5 * rng.standard_normal(q.shape)).astype(np.float32)
    return q, K, V, muQ


def _built(orc, K, V, muQ):
    return orc.prior_build(K, V, muQ)


def test_build_is_dense_attention_with_mean_query(orc):
    """O_Est is softmax(mu_Q K^T) V over the whole cache (the "one extra query
    at the end of prefill"), Z = exp(maxP) * sumP its normaliser, and mu_K the
    key mean; checked against torch SDPA / logsumexp / numpy mean."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, n, d = 2, 8, 2, 333, 128
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    muK, Oest, maxP, sumP = _built(orc, K, V, muQ)
    np.testing.assert_allclose(muK, K.astype(np.float64).mean(axis=2), rtol=1e-12, atol=1e-13)
    G = Hq // Hkv
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=1)
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=1)
    mq = torch.from_numpy(muQ.astype(np.float64))[:, :, None, :]
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = torch.nn.functional.scaled_dot_product_attention(mq, Kt, Vt, scale=scale)[:, :, 0].numpy()
    np.testing.assert_allclose(Oest, ref, rtol=1e-12, atol=1e-12)
    P = (mq @ Kt.transpose(-1, -2))[:, :, 0] * scale
    np.testing.assert_allclose(maxP, P.max(dim=-1).values.numpy(), rtol=1e-14)
    np.testing.assert_allclose(maxP + np.log(sumP), torch.logsumexp(P, dim=-1).numpy(), rtol=1e-13)


def test_empty_index_set_gives_O_est(orc):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, n, d = 1, 4, 1, 120, 64
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    built = _built(orc, K, V, muQ)
    idx = np.zeros((B, Hkv, 1), np.int32)
    lens = np.zeros((B, Hkv), np.int32)
    o, _ = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *built, idx_len=lens)
    np.testing.assert_allclose(o, built[1], rtol=1e-13, atol=1e-14)
    o2, _ = orc.sparse_prior_def(q, K, V, idx, muQ, 1.0, idx_len=lens)
    np.testing.assert_allclose(o2, built[1], rtol=1e-12, atol=1e-13)


def test_full_index_set_gives_dense(orc):
    rng = np.random.default_rng(3)
    B, Hq, Hkv, n, d = 1, 4, 2, 90, 32
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    built = _built(orc, K, V, muQ)
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (B, Hkv, n)).copy()
    o_d, l_d = orc.dense(q, K, V)
    o, lse = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *built)
    np.testing.assert_allclose(o, o_d, rtol=1e-10, atol=1e-11)
    o2, l2 = orc.sparse_prior_def(q, K, V, idx, muQ, 1.0)
    np.testing.assert_allclose(o2, o_d, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, l_d, rtol=1e-13)


def test_query_equal_to_mean_query_gives_dense_for_every_set(orc):
    """q = mu_Q makes the bias shift 0 and the prior logit the exact logit, so
    with lambda = 1 the estimate is exact whatever is read."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, n, d = 1, 2, 1, 70, 16
    q, K, V, _ = _rand(rng, B, Hq, Hkv, n, d)
    muQ = q.copy()
    built = _built(orc, K, V, muQ)
    o_d, l_d = orc.dense(q, K, V)
    for m in (0, 1, 7, 69):
        idx = np.sort(rng.choice(n, max(m, 1), replace=False)).astype(np.int32)[None, None]
        lens = np.array([[m]], np.int32)
        o, lse = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *built, idx_len=lens)
        np.testing.assert_allclose(o, o_d, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, l_d, rtol=1e-12)


def test_equal_keys_give_dense_for_every_set(orc):
    """All keys equal: K = mu_K, the residual delta = (q - mu_Q)(K - mu_K)^T
    vanishes, and the decomposition is exact for any q and mu_Q."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, n, d = 1, 2, 1, 50, 16
    q, _, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    K = np.broadcast_to(rng.standard_normal(d).astype(np.float32), (B, Hkv, n, d)).copy()
    built = _built(orc, K, V, muQ)
    o_d, _ = orc.dense(q, K, V)
    for m in (0, 3, 25):
        idx = np.sort(rng.choice(n, max(m, 1), replace=False)).astype(np.int32)[None, None]
        lens = np.array([[m]], np.int32)
        o, _ = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *built, idx_len=lens)
        np.testing.assert_allclose(o, o_d, rtol=1e-11, atol=1e-12)


def test_lambda_zero_is_plain_sparse(orc):
    rng = np.random.default_rng(6)
    B, Hq, Hkv, n, d, m = 2, 4, 2, 80, 32, 9
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    built = _built(orc, K, V, muQ)
    idx = np.stack([np.stack([np.sort(rng.choice(n, m, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    o_s, l_s = orc.sparse(q, K, V, idx)
    o, lse = orc.sparse_prior(q, K, V, idx, muQ, 0.0, *built)
    np.testing.assert_allclose(o, o_s, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, l_s, rtol=1e-13)
    o2, _ = orc.sparse_prior_def(q, K, V, idx, muQ, 0.0)
    np.testing.assert_allclose(o2, o_s, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("lam", [1.0, 0.37])
def test_delta_form_equals_definition_on_every_subset(orc, lam):
    """Brute force over all 2^10 index subsets of a 10-row cache."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, n, d = 1, 2, 1, 10, 8
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d, kshift=1.0)
    built = _built(orc, K, V, muQ)
    worst = 0.0
    for r in range(n + 1):
        for sub in itertools.combinations(range(n), r):
            idx = np.array(sub if sub else (0,), np.int32)[None, None]
            lens = np.array([[r]], np.int32)
            o1, l1 = orc.sparse_prior(q, K, V, idx, muQ, lam, *built, idx_len=lens)
            o2, l2 = orc.sparse_prior_def(q, K, V, idx, muQ, lam, idx_len=lens)
            worst = max(worst, np.abs(o1 - o2).max() / np.abs(o2).max(), np.abs(l1 - l2).max())
    assert worst < 1e-12


def test_delta_form_equals_definition_on_workload_unit(orc):
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(n=8192, n_top=3933 - 68 - 2000)
    c = synth.unit_case(w, 0, 3)
    built = orc.prior_build(c.K, c.V, c.mu_Q)
    o1, l1 = orc.sparse_prior(c.q, c.K, c.V, c.idx, c.mu_Q, 1.0, *built)
    o2, l2 = orc.sparse_prior_def(c.q, c.K, c.V, c.idx, c.mu_Q, 1.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-10 * np.abs(o2).max())
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_duplicates_rejected(orc):
    rng = np.random.default_rng(8)
    q, K, V, muQ = _rand(rng, 1, 1, 1, 10, 4)
    built = _built(orc, K, V, muQ)
    with pytest.raises(ValueError):
        orc.sparse_prior(q, K, V, np.array([[[1, 1]]], np.int32), muQ, 1.0, *built)


def test_grown_cache_delta_equals_definition(orc):
    """A prior built over the first n0 rows, decoded after the cache grew to
    n rows: the delta form (only listed rows below n0 leave the prior's mass)
    equals the plain definition (unlisted rows past n0 weigh nothing)."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, n0, n, d = 2, 4, 2, 300, 340, 128
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    built = orc.prior_build(np.ascontiguousarray(K[:, :, :n0]), np.ascontiguousarray(V[:, :, :n0]), muQ)
    for trial in range(3):
        idx = np.sort(np.stack([np.stack([rng.choice(n, size=60, replace=False) for _ in range(Hkv)])
                                for _ in range(B)]), axis=-1).astype(np.int32)
        for lam in (1.0, 0.4):
            o1, l1 = orc.sparse_prior(q, K, V, idx, muQ, lam, *built, prior_n=n0)
            o2, l2 = orc.sparse_prior_def(q, K, V, idx, muQ, lam, prior_n=n0)
            np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_grown_cache_splits_by_token_range(orc):
    """Every new row listed: the output is the log-sum-exp merge of (a) the
    prior decode over the first n0 rows with the old list and (b) plain
    softmax attention over the new rows -- the new rows enter exactly once and
    leave the prior's mass alone."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, n0, n, d = 1, 4, 1, 256, 288, 128
    q, K, V, muQ = _rand(rng, B, Hq, Hkv, n, d)
    K0, V0 = np.ascontiguousarray(K[:, :, :n0]), np.ascontiguousarray(V[:, :, :n0])
    built = orc.prior_build(K0, V0, muQ)
    I0 = np.sort(rng.choice(n0, size=40, replace=False)).astype(np.int32)
    idx = np.concatenate([I0, np.arange(n0, n, dtype=np.int32)])[None, None]
    o, l = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *built, prior_n=n0)
    oa, la = orc.sparse_prior(q, K0, V0, I0[None, None], muQ, 1.0, *built)
    Kn, Vn = np.ascontiguousarray(K[:, :, n0:]), np.ascontiguousarray(V[:, :, n0:])
    ob, lb = orc.dense(q, Kn, Vn)
    lm = np.logaddexp(la, lb)
    om = (np.exp(la - lm)[..., None] * oa + np.exp(lb - lm)[..., None] * ob)
    np.testing.assert_allclose(o, om, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l, lm, rtol=1e-12)
    # prior_n = n is the same as covering every row
    full = orc.prior_build(K, V, muQ)
    o3, _ = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *full, prior_n=n)
    o4, _ = orc.sparse_prior(q, K, V, idx, muQ, 1.0, *full)
    np.testing.assert_array_equal(o3, o4)
