"""Repeatability and split invariance of the paths with a split-K merge and
of the sampled tail: the same call twice gives the same bits (no atomics in
any sum, a fixed merge order), and a unit's result does not depend, beyond
fp32 rounding, on how many workgroups share its rows (the launch shape
follows the number of units).  The log-sum-exp merge is exact arithmetic
over a partition of the rows ("RESA", Online Aggregator: the merge of
partial softmax sums), so only the summation order may differ."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, to_dev

pytestmark = pytest.mark.gpu

SPLIT_TOL = 1e-5   # relative, per row: fp32 summation order only


def _twice(call):
    a = [t.clone() for t in call()]
    torch.cuda.synchronize()
    b = [t.clone() for t in call()]
    torch.cuda.synchronize()
    return a, b


def _bitwise(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.cpu(), y.cpu())


def _none_case(B, seed=5, n=6000, m=2500):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=B, n=n, n_top=40, C=0)
    c = synth.make_case(w)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.integers(0, n, size=(B, w.Hkv, m)), axis=-1).astype(np.int32)
    return w, c, idx


def test_split_k_none_twice():
    w, c, idx = _none_case(1)
    d = case_to_dev(c)
    a, b = _twice(lambda: sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx)))
    _bitwise(a, b)


def test_prior_twice():
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(B=2, n=16384, n_top=600)
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    ps2 = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    torch.cuda.synchronize()
    _bitwise([ps.mu_K, ps.O_est, ps.maxP, ps.sumP], [ps2.mu_K, ps2.O_est, ps2.maxP, ps2.sumP])
    a, b = _twice(lambda: sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=ps, lam=0.7))
    _bitwise(a, b)


def test_dense_twice():
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=20000, n_top=40, C=0)
    c = synth.make_case(w)
    d = case_to_dev(c)
    a, b = _twice(lambda: sda.dense_decode_attn(d["q"], d["K"], d["V"]))
    _bitwise(a, b)


def test_sampled_twice():
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=2, n=16384, n_top=160)
    c = synth.make_case(w)
    d = case_to_dev(c)

    def call():
        t = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=256)
        out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=t)
        return out, lse, t.b, t.bstar, t.samples

    a, b = _twice(call)
    _bitwise(a, b)


def test_proxy_unit_twice():
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=4, n=8192, n_top=260)
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    a, b = _twice(lambda: sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st,
                                                 idx_cluster=d["idx_cluster"]))
    _bitwise(a, b)


def _rows_close(x, y, tol):
    x = x.cpu().double().numpy()
    y = y.cpu().double().numpy()
    den = np.abs(y).max(axis=-1)
    return float((np.abs(x - y).max(axis=-1) / np.where(den > 0, den, 1.0)).max()) <= tol


def _split_counts(K, Hq, m, kind, op=sda.OP_SPARSE):
    """Workspace bytes per unit and split, i.e. a proxy for the split count."""
    return sda.workspace_bytes(sda.make_dims(K, Hq), op, kind, m)


def test_split_count_invariance_none():
    """Units of a batch-1 call (more workgroups per unit) against the same
    units inside a batch-16 call (fewer)."""
    w1, c1, idx1 = _none_case(1)
    w16, c16, idx16 = _none_case(16)
    d1, d16 = case_to_dev(c1), case_to_dev(c16)
    idx16[0] = idx1[0]
    assert _split_counts(d1["K"], w1.Hq, idx1.shape[-1], sda.TAIL_NONE) / (w1.B * w1.Hkv) != \
        _split_counts(d16["K"], w16.Hq, idx16.shape[-1], sda.TAIL_NONE) / (w16.B * w16.Hkv)
    o1, l1 = sda.sparse_decode_attn(d1["q"], d1["K"], d1["V"], to_dev(idx1))
    o16, l16 = sda.sparse_decode_attn(d16["q"], d16["K"], d16["V"], to_dev(idx16))
    torch.cuda.synchronize()
    assert _rows_close(o16[0], o1[0], SPLIT_TOL)
    assert (l16[0] - l1[0]).abs().max().item() <= 1e-5


def test_split_count_invariance_dense_and_prior():
    w1 = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(B=1, n=16384, n_top=1500)
    w8 = w1.replace(B=16)
    c1, c8 = synth.make_case(w1), synth.make_case(w8)   # sequence 0 is the same in both
    d1, d8 = case_to_dev(c1), case_to_dev(c8)
    assert torch.equal(d1["K"][0].cpu(), d8["K"][0].cpu())
    assert sda.workspace_bytes(sda.make_dims(d1["K"], w1.Hq), sda.OP_DENSE) / w1.B != \
        sda.workspace_bytes(sda.make_dims(d8["K"], w8.Hq), sda.OP_DENSE) / w8.B
    o1, _ = sda.dense_decode_attn(d1["q"], d1["K"], d1["V"])
    o8, _ = sda.dense_decode_attn(d8["q"], d8["K"], d8["V"])
    torch.cuda.synchronize()
    assert _rows_close(o8[0], o1[0], SPLIT_TOL)
    p1 = sda.build_prior(d1["K"], d1["V"], d1["mu_Q"])
    p8 = sda.build_prior(d8["K"], d8["V"], d8["mu_Q"])
    torch.cuda.synchronize()
    assert _rows_close(p8.O_est[0], p1.O_est[0], SPLIT_TOL)
    o1, _ = sda.sparse_decode_attn(d1["q"], d1["K"], d1["V"], d1["idx"], tail=p1)
    o8, _ = sda.sparse_decode_attn(d8["q"], d8["K"], d8["V"], d8["idx"], tail=p8)
    torch.cuda.synchronize()
    assert _rows_close(o8[0], o1[0], SPLIT_TOL)
