"""The seeded input generator: shapes, structure and determinism."""
import numpy as np
import torch

from long_context_sparse_gathered_amd import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -0.0, 3.0e38]   # ties and extremes
    ours = synth.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_index_counts_match_the_workloads():
    assert synth.WORKLOADS["proxy_f32_b1_n4k"].m == 196
    assert synth.WORKLOADS["proxy_bf16_b1_n32k"].m == 328 and synth.WORKLOADS["proxy_bf16_b32_n32k"].m == 328
    assert synth.WORKLOADS["sampled_bf16_b8_n64k"].m == 788
    assert synth.WORKLOADS["prior_bf16_b16_n128k"].m == 3933
    assert abs(synth.WORKLOADS["sampled_bf16_b8_n64k"].z - 1.959963984540054) < 1e-12


def test_unit_structure_f32_single_head():
    w = synth.WORKLOADS["proxy_f32_b1_n4k"]
    u = synth.make_unit(w, 0, 0)
    idx = u.idx
    assert idx.dtype == np.int32 and idx.shape == (w.m,)
    assert np.all(np.diff(idx) > 0)
    assert set(range(w.n_sink)) <= set(idx.tolist())
    assert set(range(w.n - w.n_local, w.n)) <= set(idx.tolist())
    assert set(u.heavy.tolist()) <= set(idx.tolist())
    # planted rows have scaled logit ~ t in [11, 13]
    s = u.K[u.heavy].astype(np.float64) @ u.q[0].astype(np.float64) / np.sqrt(w.d)
    assert np.all((s > 10.9) & (s < 13.1))
    assert np.array_equal(u.cid, np.arange(w.n) // 256)


def test_random_segmentation_and_determinism():
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"]
    a = synth.make_unit(w, 0, 3)
    b = synth.make_unit(w, 0, 3)
    np.testing.assert_array_equal(a.K, b.K)
    np.testing.assert_array_equal(a.idx, b.idx)
    cid = a.cid
    assert cid.min() == 0 and cid.max() == w.C - 1
    assert np.all(np.diff(cid) >= 0) and np.count_nonzero(np.diff(cid)) == w.C - 1
    c = synth.make_unit(w, 0, 4)
    assert not np.array_equal(a.idx, c.idx)


def test_case_assembly_matches_units():
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(n=2048, n_top=60)
    case = synth.make_case(w, threads=4)
    u = synth.make_unit(w, 0, 6)
    np.testing.assert_array_equal(case.K[0, 6], u.K)
    np.testing.assert_array_equal(case.q[0, 24:28], u.q)
    np.testing.assert_array_equal(case.idx[0, 6], u.idx)
    ic = case.idx_cluster
    np.testing.assert_array_equal(ic[0, 6], u.cid[u.idx])


def test_prior_workload_mean_query():
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(n=4096, n_top=100)
    u = synth.make_unit(w, 1, 2)
    assert u.mu_Q.shape == (w.G, w.d) and u.mu_Q.dtype == np.float32
    # the prefill mean sits near a norm-3 vector
    assert np.all(np.abs(np.linalg.norm(u.mu_Q, axis=1) - 3.0) < 0.5)


def test_index_sets_for_another_read_fraction():
    """index_sets(c, n_top) gives the lists make_case gives for that n_top on
    the same keys and queries."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(n=4096, n_top=40)
    c = synth.make_case(w, threads=4)
    w3 = w.replace(n_top=120)
    c3 = synth.make_case(w3, threads=4)
    np.testing.assert_array_equal(c.K, c3.K)
    got = synth.index_sets(c, 120, threads=4)
    np.testing.assert_array_equal(got, c3.idx)
    np.testing.assert_array_equal(synth.index_sets(c, 40, threads=4), c.idx)
