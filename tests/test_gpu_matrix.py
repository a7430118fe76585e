"""GPU parity across the kernel shapes: every query-group size G with each
tail, the tile counts of the one-workgroup-per-unit kernel, the split-K
matrix-core kernel with and without the rank-1 prior, the sampled kernels,
and the full-size workloads in the launch configuration bench.py times
(checked on sampled units against the oracle).

Tolerances as in test_gpu_parity: max over rows of max|o - o*| / max|o*|
<= 2e-3 for bf16 inputs; budgets and drawn positions bit-exact."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, dev, lse_err, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
LSE_TOL = 1e-3


def _sync():
    torch.cuda.synchronize()


def _grouped(w, G, Hkv):
    return w.replace(Hq=G * Hkv, Hkv=Hkv)


# list length -> tiles of 16 entries per wave in the unit kernel (8 waves)
@pytest.mark.parametrize("G,n_top", [(1, 40), (2, 40), (2, 200), (4, 140), (4, 430), (8, 100), (8, 310)])
def test_proxy_unit_kernel_group_sizes(orc, G, n_top):
    """Proxy decode through the one-workgroup-per-unit kernel: G = 1..8 and
    1..4 tiles per wave (m = 108 .. 498; at most 3 tiles for G = 8), so the
    cluster-sum tile both shares a pair with a key tile and stands alone."""
    w = _grouped(synth.WORKLOADS["proxy_bf16_b1_n32k"], G, 2).replace(B=2, n=4096, n_top=n_top, C=37)
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st, idx_cluster=d["idx_cluster"])
    _sync()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
    assert rel_err(out, ref) <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


# list length -> tiles per wave: 200 -> 2, 328 -> 3 (a lone last tile), 100 -> 1
@pytest.mark.parametrize("G,m", [(1, 200), (2, 200), (8, 200), (4, 328), (1, 328), (8, 100), (2, 100)])
def test_none_unit_kernel_group_sizes(orc, G, m):
    """No tail with 128 units (one workgroup per unit): random lists with
    duplicates and log-weights, 1..3 tiles of 16 keys per wave."""
    w = _grouped(synth.WORKLOADS["proxy_bf16_b1_n32k"], G, 2).replace(B=64, n=1024, n_top=40, C=0)
    c = synth.make_case(w)
    rng = np.random.default_rng(G * 1000 + m)
    idx = rng.integers(0, w.n, size=(w.B, w.Hkv, m)).astype(np.int32)
    logw = rng.normal(0, 1, size=idx.shape).astype(np.float32)
    d = case_to_dev(c)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), logw=to_dev(logw))
    _sync()
    ref, ref_lse = orc.sparse(c.q, c.K, c.V, idx, logw=logw)
    assert rel_err(out, ref) <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


@pytest.mark.parametrize("G", [1, 2, 8])
def test_none_stream_kernel_group_sizes(orc, G):
    """No tail with few units and a long list: split-K on the matrix cores
    (several batches per workgroup, several workgroups per unit)."""
    w = _grouped(synth.WORKLOADS["proxy_bf16_b1_n32k"], G, 2).replace(B=1, n=6000, n_top=40, C=0)
    c = synth.make_case(w)
    rng = np.random.default_rng(10 + G)
    idx = np.sort(rng.integers(0, w.n, size=(w.B, w.Hkv, 2500)), axis=-1).astype(np.int32)
    d = case_to_dev(c)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx))
    _sync()
    ref, ref_lse = orc.sparse(c.q, c.K, c.V, idx)
    assert rel_err(out, ref) <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


@pytest.mark.parametrize("G", [1, 2, 8])
def test_prior_group_sizes(orc, G):
    """Rank-1 prior: G = 1, 2 on the matrix-core stream (mean query split in
    high part and remainder rows), G = 8 on the vector stream."""
    w = _grouped(synth.WORKLOADS["prior_bf16_b16_n128k"], G, 2).replace(B=2, n=8192, n_top=1200)
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    _sync()
    muK, Oest, maxP, sumP = orc.prior_build(c.K, c.V, c.mu_Q)
    for lam in (1.0, 0.5):
        out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=ps, lam=lam)
        _sync()
        ref, ref_lse = orc.sparse_prior(c.q, c.K, c.V, c.idx, c.mu_Q, lam, muK, Oest, maxP, sumP)
        assert rel_err(out, ref) <= TOL, lam
        assert lse_err(lse, ref_lse) <= LSE_TOL, lam


@pytest.mark.parametrize("G", [1, 2, 8])
def test_sampled_group_sizes(orc, G):
    """Sampled tail for G = 1, 2, 8: budgets and draws bit-exact."""
    w = _grouped(synth.WORKLOADS["sampled_bf16_b8_n64k"], G, 2).replace(B=2, n=4096, n_top=40)
    c = synth.make_case(w)
    d = case_to_dev(c)
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=4096)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=tail)
    _sync()
    ref = orc.sampled(c.q, c.K, c.V, c.idx, w.eps, w.z, w.b0, w.sampler_seed, 4096)
    r = np.round(ref["bstar"])
    assert not ((np.abs(ref["bstar"] - r) < 1e-9 * np.maximum(ref["bstar"], 1.0)) & (r >= 1)).any()
    np.testing.assert_array_equal(tail.b.cpu().numpy(), ref["b"])
    got = tail.samples.cpu().numpy()
    for s in range(w.B):
        for g in range(w.Hkv):
            k = min(int(ref["b"][s, g]), 4096)
            np.testing.assert_array_equal(got[s, g, :k], ref["samples"][s, g, :k])
    assert rel_err(out, ref["out"]) <= TOL
    assert lse_err(lse, ref["lse"]) <= LSE_TOL


def _sample_units(w, k, seed):
    rng = np.random.default_rng(seed)
    return [divmod(int(u), w.Hkv) for u in rng.choice(w.B * w.Hkv, size=k, replace=False)]


def test_proxy_full_size_b32_n32k(orc):
    """The timed decode step (batch 32, 32K, 1% read, 32 proxies per KV head)
    checked on 8 sampled units against the oracle's definition."""
    w = synth.WORKLOADS["proxy_bf16_b32_n32k"]
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st, idx_cluster=d["idx_cluster"])
    _sync()
    got, got_lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for s, g in _sample_units(w, 8, 1):
        uc = synth.unit_case(w, s, g)
        ref, ref_lse = orc.sparse_proxy_def(uc.q, uc.K, uc.V, uc.idx, uc.cid, w.C)
        rows = slice(g * w.G, (g + 1) * w.G)
        assert rel_err(got[s, rows], ref[0]) <= TOL, (s, g)
        assert np.abs(got_lse[s, rows] - ref_lse[0]).max() <= LSE_TOL, (s, g)


def test_prior_full_size_b16_n128k(orc):
    """The prior decode step (batch 16, 128K, 3% read) checked on 4 sampled
    units against the oracle (its own prior build per unit)."""
    w = synth.WORKLOADS["prior_bf16_b16_n128k"]
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=ps)
    _sync()
    got, got_lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    del d, ps
    torch.cuda.empty_cache()
    for s, g in _sample_units(w, 4, 2):
        uc = synth.unit_case(w, s, g)
        muK, Oest, maxP, sumP = orc.prior_build(uc.K, uc.V, uc.mu_Q)
        ref, ref_lse = orc.sparse_prior(uc.q, uc.K, uc.V, uc.idx, uc.mu_Q, 1.0, muK, Oest, maxP, sumP)
        rows = slice(g * w.G, (g + 1) * w.G)
        assert rel_err(got[s, rows], ref[0]) <= TOL, (s, g)
        assert np.abs(got_lse[s, rows] - ref_lse[0]).max() <= LSE_TOL, (s, g)


@pytest.mark.parametrize("G", [4, 8])
def test_prior_on_grown_cache(orc, G):
    """The prior built over the first n0 rows (the prefill), the decode after
    the cache grew to n rows with the new rows in the local window: rows past
    n0 are exact-only (matrix-core stream at G = 4, vector stream at G = 8)."""
    w = _grouped(synth.WORKLOADS["prior_bf16_b16_n128k"], G, 2).replace(B=2, n=6000, n_top=900)
    n0 = 5800
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"][:, :, :n0], d["V"][:, :, :n0], d["mu_Q"])
    assert ps.n_covered == n0
    _sync()
    K0, V0 = np.ascontiguousarray(c.K[:, :, :n0]), np.ascontiguousarray(c.V[:, :, :n0])
    built = orc.prior_build(K0, V0, c.mu_Q)
    for lam in (1.0, 0.3):
        out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=ps, lam=lam)
        _sync()
        ref, ref_lse = orc.sparse_prior_def(c.q, c.K, c.V, c.idx, c.mu_Q, lam, prior_n=n0)
        ref2, _ = orc.sparse_prior(c.q, c.K, c.V, c.idx, c.mu_Q, lam, *built, prior_n=n0)
        assert rel_err(ref2, ref) <= 1e-10
        assert rel_err(out, ref) <= TOL, lam
        assert lse_err(lse, ref_lse) <= LSE_TOL, lam


@pytest.mark.parametrize("G", [1, 4, 8])
def test_proxy_without_listed_rows(orc, G):
    """m = 0: every unit's output is its cluster proxies alone (the
    matrix-core unit kernel reads no list)."""
    w = _grouped(synth.WORKLOADS["proxy_bf16_b1_n32k"], G, 2).replace(B=2, n=2048, n_top=40, C=13)
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    idx = np.zeros((w.B, w.Hkv, 0), np.int32)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), tail=st, cluster_id=d["cid"])
    _sync()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, idx, c.cid, w.C)
    assert rel_err(out, ref) <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


def test_dense_full_size_b32_n32k(orc):
    """Dense decode in the launch bench.py times (batch 32, 32K: 256 units,
    8 splits of 4096 rows each plus the merge), checked on 4 sampled units
    against the oracle's textbook softmax."""
    w = synth.WORKLOADS["proxy_bf16_b32_n32k"]
    c = synth.make_case(w)
    d = case_to_dev(c)
    out, lse = sda.dense_decode_attn(d["q"], d["K"], d["V"])
    _sync()
    got, got_lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for s, g in _sample_units(w, 4, 7):
        uc = synth.unit_case(w, s, g)
        ref, ref_lse = orc.dense(uc.q, uc.K, uc.V)
        rows = slice(g * w.G, (g + 1) * w.G)
        assert rel_err(got[s, rows], ref[0]) <= TOL, (s, g)
        assert np.abs(got_lse[s, rows] - ref_lse[0]).max() <= LSE_TOL, (s, g)


def _mostly_read_clusters(G, seed):
    """Units where several clusters are listed but for two members each, and
    those unread members hold logits near the unit's largest (held by a listed
    row, so that the proxy weight e^{mu_b - M} is no round number) while the
    listed members sit low; within such a cluster the values are nearly
    equal, so the cluster's value sum and its listed members' share cancel to
    1/64 of their size (OpenAttention, method stage 04: the proxy folds only a
    cluster's unread tokens)."""
    rng = np.random.default_rng(seed)
    B, Hkv, n, d, C, size, m = 2, 8, 4096, 128, 32, 128, 328
    Hq = G * Hkv
    q = synth.round_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    K = (0.5 * rng.standard_normal((B, Hkv, n, d))).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    cid = np.broadcast_to((np.arange(n) // size).astype(np.int32), (B, Hkv, n)).copy()
    idx = np.empty((B, Hkv, m), np.int32)
    for s in range(B):
        for g in range(Hkv):
            qb = qf[s, g * G:(g + 1) * G].mean(axis=0)
            aligned = np.sqrt(d) * qb / (qb @ qb)   # key of scaled logit 1 against the mean query
            listed = set(range(4)) | set(range(n - 64, n))
            K[s, g, n - 1] = (14.5 * aligned).astype(np.float32)   # a listed row holds the unit maximum
            for b in rng.choice(np.arange(1, C - 1), size=2, replace=False):
                members = np.arange(b * size, (b + 1) * size)
                unread = rng.choice(members, size=2, replace=False)
                # two different keys, so the unread mean's weight is no bf16 number
                K[s, g, unread[0]] = (14.0 * aligned).astype(np.float32)
                K[s, g, unread[1]] = (13.6 * aligned + 0.3 * rng.standard_normal(d)).astype(np.float32)
                V[s, g, members] = (3.0 * rng.standard_normal(d) + 0.01 * rng.standard_normal((size, d)))
                listed |= set(members.tolist()) - set(unread.tolist())
            rest = np.setdiff1d(np.arange(n), np.fromiter(listed, int))
            listed |= set(rng.choice(rest, size=m - len(listed), replace=False).tolist())
            idx[s, g] = np.sort(np.fromiter(listed, np.int32))
    return q, synth.round_bf16_bits(K), synth.round_bf16_bits(V), idx, cid, C


@pytest.mark.parametrize("G", [4, 8, 2])
def test_proxy_mostly_read_clusters(orc, G):
    """The cancellation case at the headline kernel's shape (m = 328, three
    tiles of 16 keys per wave): the listed members' correction and the
    cluster's value sum must cancel to the unread members' share within the
    bf16 tolerance; the margin is printed."""
    q, K, V, idx, cid, C = _mostly_read_clusters(G, 11 + G)
    st = sda.build_tail_proxies(to_dev(K), to_dev(V), to_dev(cid), C)
    icl = np.take_along_axis(cid, idx.astype(np.int64), axis=2).astype(np.int32)
    out, lse = sda.sparse_decode_attn(to_dev(q), to_dev(K), to_dev(V), to_dev(idx), tail=st, idx_cluster=to_dev(icl))
    _sync()
    ref, ref_lse = orc.sparse_proxy_def(q, K, V, idx, cid, C)
    err = rel_err(out, ref)
    print(f"mostly-read clusters, G={G}: max rel err {err:.3e} (tolerance {TOL:.0e}, margin {TOL / max(err, 1e-30):.0f}x)")
    assert err <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


@pytest.mark.parametrize("G", [1, 4, 8])
def test_stream_ragged_logw_and_flags(orc, G):
    """The split-K stream kernel with ragged list lengths (chunks ending
    inside a batch, odd batch counts, empty units), log-weights, and list
    errors on two units: an index past the cache (skipped and flagged) and,
    with the prior, two entries out of order (flagged). Every other unit
    matches the oracle."""
    w = _grouped(synth.WORKLOADS["prior_bf16_b16_n128k"], G, 4).replace(B=2, n=8192, n_top=1400)
    c = synth.make_case(w)
    m = c.idx.shape[-1]
    rng = np.random.default_rng(40 + G)
    lens = rng.integers(0, m + 1, size=(w.B, w.Hkv)).astype(np.int32)
    lens[0, 0], lens[1, 3] = 0, m
    lens[0, 1], lens[0, 2] = max(lens[0, 1], 300), max(lens[0, 2], 300)
    logw = rng.normal(0.0, 0.5, size=c.idx.shape).astype(np.float32)
    idx = c.idx.copy()
    idx[0, 1, 200] = w.n + 7                                      # out of range
    idx[0, 2, 100], idx[0, 2, 101] = idx[0, 2, 101], idx[0, 2, 100]  # out of order
    d = case_to_dev(c)
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), idx_len=to_dev(lens), logw=to_dev(logw),
                                      flags=flags)
    _sync()
    f = flags.cpu().numpy()
    assert f[0, 1] & sda.FLAG_IDX_RANGE
    keep = [(s, g) for s in range(w.B) for g in range(w.Hkv) if (s, g) != (0, 1)]
    assert all(f[s, g] == 0 for s, g in keep)  # no order check without the prior
    ref, ref_lse = orc.sparse(c.q, c.K, c.V, c.idx, idx_len=lens, logw=logw)
    for s, g in keep:
        rows = slice(g * w.G, (g + 1) * w.G)
        assert rel_err(out[s, rows], ref[s, rows]) <= TOL, (s, g)
        assert lse_err(lse[s, rows], ref_lse[s, rows]) <= LSE_TOL, (s, g)
    if 3 * G > 16:
        return  # the prior at G = 8 runs on the vector stream kernel
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    flags.zero_()
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), idx_len=to_dev(lens), logw=to_dev(logw),
                                      tail=ps, lam=0.6, flags=flags)
    _sync()
    f = flags.cpu().numpy()
    assert f[0, 1] & sda.FLAG_IDX_RANGE and f[0, 2] & sda.FLAG_IDX_ORDER
    keep = [(s, g) for s in range(w.B) for g in range(w.Hkv) if (s, g) not in ((0, 1), (0, 2))]
    assert all(f[s, g] == 0 for s, g in keep)
    muK, Oest, maxP, sumP = orc.prior_build(c.K, c.V, c.mu_Q)
    ref, ref_lse = orc.sparse_prior(c.q, c.K, c.V, c.idx, c.mu_Q, 0.6, muK, Oest, maxP, sumP, idx_len=lens,
                                    logw=logw)
    for s, g in keep:
        rows = slice(g * w.G, (g + 1) * w.G)
        assert rel_err(out[s, rows], ref[s, rows]) <= TOL, (s, g)
        assert lse_err(lse[s, rows], ref_lse[s, rows]) <= LSE_TOL, (s, g)
