"""GPU parity of the sampled tail (vAttention page, method sections 1-3)
against the fp64 oracle: the budget b and every drawn position bit-exact,
the output within the bf16/fp32 tolerance.

A budget is compared exactly unless the oracle's real-valued budget b* lies
within a relative 1e-9 of an integer (a tie that fp64 summation order can
flip); such ties are counted and reported, and none is expected."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, dev, lse_err, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _ties(bstar):
    """b* within a relative 1e-9 of an integer k >= 1, where the ceiling could
    give k or k + 1 (below 1 every value rounds to the minimum budget, 1)."""
    r = np.round(bstar)
    return (np.abs(bstar - r) < 1e-9 * np.maximum(bstar, 1.0)) & (r >= 1)


def _check(orc, c, w, seed, b_cap, tol, idx=None, idx_len=None, K=None, V=None):
    idx = c.idx if idx is None else idx
    K = c.K if K is None else K
    V = c.V if V is None else V
    d = case_to_dev(c)
    Kd, Vd = to_dev(K), to_dev(V)
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=seed, b_cap=b_cap)
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    out, lse = sda.sparse_decode_attn(d["q"], Kd, Vd, to_dev(idx), idx_len=None if idx_len is None else to_dev(idx_len),
                                      tail=tail, flags=flags)
    torch.cuda.synchronize()
    ref = orc.sampled(c.q, K, V, idx, w.eps, w.z, w.b0, seed, b_cap, idx_len=idx_len)
    b_gpu = tail.b.cpu().numpy()
    ties = _ties(ref["bstar"])
    assert not ties.any(), f"{ties.sum()} budget ties"
    np.testing.assert_array_equal(b_gpu, ref["b"])
    # b* is a sample count: agree to 1e-12 relative, or within 1e-9 where it is rounding noise near 0
    np.testing.assert_allclose(tail.bstar.cpu().numpy(), ref["bstar"], rtol=1e-12, atol=1e-9)
    if b_cap > 0:
        got = tail.samples.cpu().numpy()
        for s in range(w.B):
            for g in range(w.Hkv):
                k = min(int(ref["b"][s, g]), b_cap)
                np.testing.assert_array_equal(got[s, g, :k], ref["samples"][s, g, :k])
    assert rel_err(out, ref["out"]) <= tol
    assert lse_err(lse, ref["lse"]) <= 1e-3
    return tail, flags, ref


def test_sampled_small_bf16(orc):
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=2, n=8192, n_top=82)
    c = synth.make_case(w)
    tail, flags, ref = _check(orc, c, w, w.sampler_seed, b_cap=8192, tol=2e-3)
    assert (flags.cpu().numpy() == 0).all()
    assert (ref["b"] > 1).all()


@pytest.mark.parametrize("seed", [0, 7, 123456789])
def test_sampled_seeds_and_ragged(orc, seed):
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=1, n=4096, n_top=40)
    c = synth.make_case(w)
    lens = np.array([[w.m, w.m // 2, 0, 1, w.m, 5, w.m - 1, 2]], np.int32)
    _check(orc, c, w, seed, b_cap=64, tol=2e-3, idx_len=lens)


def test_sampled_fp32_single_head(orc):
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=2, Hq=2, Hkv=2, n=3000, n_top=30, dtype="f32")
    c = synth.make_case(w)
    _check(orc, c, w, 99, b_cap=4096, tol=1e-5)


def test_sampled_no_tail_and_constant_tail(orc):
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=1, Hq=8, Hkv=2, n=300, n_top=20)
    c = synth.make_case(w)
    full = np.broadcast_to(np.arange(w.n, dtype=np.int32), (1, w.Hkv, w.n)).copy()
    tail, _, ref = _check(orc, c, w, 3, b_cap=4, tol=2e-3, idx=full)
    assert (tail.b.cpu().numpy() == 0).all()
    # all unread rows identical: both variances vanish, b = 1, exact
    K, V = c.K.copy(), c.V.copy()
    for g in range(w.Hkv):
        mask = np.ones(w.n, bool)
        mask[c.idx[0, g]] = False
        first = np.argmax(mask)
        K[0, g, mask] = K[0, g, first]
        V[0, g, mask] = V[0, g, first]
    tail, _, ref = _check(orc, c, w, 3, b_cap=4, tol=2e-3, K=K, V=V)
    assert (tail.b.cpu().numpy() == 1).all()


def test_sampled_full_size_b8_n64k(orc):
    """The full sampling workload (batch 8, 64K context, 788 listed rows per
    KV head): every unit's budget, draws and output against the oracle."""
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"]
    c = synth.make_case(w)
    d = case_to_dev(c)
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=4096)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=tail)
    torch.cuda.synchronize()
    b_gpu = tail.b.cpu().numpy()
    samples = tail.samples.cpu().numpy()
    got = out.cpu().double().numpy()
    # budgets and draws of every unit, from the oracle on the whole workload
    ref = orc.sampled(c.q, c.K, c.V, c.idx, w.eps, w.z, w.b0, w.sampler_seed, 4096)
    assert not _ties(ref["bstar"]).any()
    np.testing.assert_array_equal(b_gpu, ref["b"])
    for s in range(w.B):
        for g in range(w.Hkv):
            k = min(int(ref["b"][s, g]), 4096)
            np.testing.assert_array_equal(samples[s, g, :k], ref["samples"][s, g, :k])
    assert rel_err(got, ref["out"]) <= 2e-3


def test_sampled_budget_reaches_whole_tail_one_unit(orc):
    """One unit at 128K whose budget is the whole unread tail (b* far above
    n_s, so b = n_s = 130,840 draws): 512 work items over the draw grid, one
    record per item, so the merge stages its records in two rounds."""
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=1, Hq=4, Hkv=1, n=131072, n_top=100, eps=0.004)
    c = synth.make_case(w)
    tail, _, ref = _check(orc, c, w, 11, b_cap=1024, tol=2e-3)
    assert int(tail.b.cpu().numpy()[0, 0]) == w.n - w.m


@pytest.mark.parametrize("hq,hkv", [(8, 4), (32, 4)])
def test_sampled_group_sizes(orc, hq, hkv):
    """Two and eight query heads per KV head (the kernels' other register
    shapes and draw-grid occupancies): budgets, draws and output."""
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=2, Hq=hq, Hkv=hkv, n=6000, n_top=60)
    c = synth.make_case(w)
    _check(orc, c, w, 5, b_cap=4096, tol=2e-3)


@pytest.mark.parametrize("eps", [0.2, 0.4])
def test_sampled_verified_budget(orc, eps):
    """The verified budget ("vAttention", verified-SDPA: eps and delta bound
    the output through Lemma 4.2, the budget minimised over the allocation as
    Theorem 4.3 states): budgets, draws and output against the oracle's
    verified estimator, and every budget at least the plain one."""
    from statistics import NormalDist
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=2, n=8192, n_top=82, eps=eps)
    c = synth.make_case(w)
    d = case_to_dev(c)
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=8192, verified=True)
    nd = NormalDist()
    zs = np.array([(nd.inv_cdf(1 - k / 32 * w.delta / 2), nd.inv_cdf(1 - (1 - k / 32) * w.delta / 2))
                   for k in range(1, 32)])
    assert np.array_equal(np.array(tail.z_split), zs)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=tail)
    torch.cuda.synchronize()
    ref = orc.sampled_verified(c.q, c.K, c.V, c.idx, w.eps, zs, w.b0, w.sampler_seed, 8192)
    assert not _ties(ref["bstar"]).any()
    np.testing.assert_array_equal(tail.b.cpu().numpy(), ref["b"])
    np.testing.assert_allclose(tail.bstar.cpu().numpy(), ref["bstar"], rtol=1e-12, atol=1e-9)
    got = tail.samples.cpu().numpy()
    for s in range(w.B):
        for g in range(w.Hkv):
            k = min(int(ref["b"][s, g]), 8192)
            np.testing.assert_array_equal(got[s, g, :k], ref["samples"][s, g, :k])
    assert rel_err(out, ref["out"]) <= 2e-3
    assert lse_err(lse, ref["lse"]) <= 1e-3
    plain = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed)
    sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=plain)
    torch.cuda.synchronize()
    assert (tail.b.cpu().numpy() >= plain.b.cpu().numpy()).all()
