"""GPU parity: the HIP path against the fp64 CPU oracle on the same inputs.

Tolerances (max over rows of max|o - o*| / max|o*|): 1e-5 for fp32 inputs,
2e-3 for bf16 inputs; integer outputs (cluster counts, flags) bit-exact.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, dev, lse_err, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}
LSE_TOL = {"f32": 1e-5, "bf16": 1e-3}


def _sync():
    torch.cuda.synchronize()


def _proxy_case(orc, w, by_index=True):
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    kw = dict(idx_cluster=d["idx_cluster"]) if by_index else dict(cluster_id=d["cid"])
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st, **kw)
    _sync()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
    return c, d, st, out, lse, ref, ref_lse


def test_proxy_f32_single_head(orc):
    w = synth.WORKLOADS["proxy_f32_b1_n4k"]
    c, d, st, out, lse, ref, ref_lse = _proxy_case(orc, w)
    assert rel_err(out, ref) <= TOL["f32"]
    assert lse_err(lse, ref_lse) <= LSE_TOL["f32"]
    cnt, sK, sV = orc.proxy_build(c.K, c.V, c.cid, w.C)
    np.testing.assert_array_equal(st.count.cpu().numpy(), cnt)
    assert rel_err(st.sumK, sK) <= 1e-6 and rel_err(st.sumV, sV) <= 1e-6


@pytest.mark.parametrize("by_index", [True, False])
def test_proxy_bf16_b1_n32k(orc, by_index):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"]
    c, d, st, out, lse, ref, ref_lse = _proxy_case(orc, w, by_index)
    assert rel_err(out, ref) <= TOL["bf16"]
    assert lse_err(lse, ref_lse) <= LSE_TOL["bf16"]
    cnt, _, _ = orc.proxy_build(c.K, c.V, c.cid, w.C)
    np.testing.assert_array_equal(st.count.cpu().numpy(), cnt)
    # run-to-run bitwise determinism, builder and decode
    st2 = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    kw = dict(idx_cluster=d["idx_cluster"]) if by_index else dict(cluster_id=d["cid"])
    out2, lse2 = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st2, **kw)
    _sync()
    assert torch.equal(st.sumK, st2.sumK) and torch.equal(st.sumV, st2.sumV)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_proxy_general_clusters_and_ragged(orc):
    """Non-contiguous cluster ids (with -1), ragged list lengths including an
    empty unit, log-weights, and C not a multiple of the kernel's slot size."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=3000, n_top=150, C=37)
    c = synth.make_case(w)
    rng = np.random.default_rng(5)
    cid = rng.integers(-1, w.C, size=c.cid.shape).astype(np.int32)
    lens = rng.integers(0, w.m + 1, size=(w.B, w.Hkv)).astype(np.int32)
    lens[0, 0], lens[1, 7] = 0, w.m
    logw = rng.normal(0, 0.5, size=c.idx.shape).astype(np.float32)
    d = case_to_dev(c)
    cid_d = to_dev(cid)
    st = sda.build_tail_proxies(d["K"], d["V"], cid_d, w.C)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], idx_len=to_dev(lens), logw=to_dev(logw),
                                      tail=st, cluster_id=cid_d)
    _sync()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, cid, w.C, idx_len=lens, logw=logw)
    assert rel_err(out, ref) <= TOL["bf16"]
    assert lse_err(lse, ref_lse) <= LSE_TOL["bf16"]


@pytest.mark.parametrize("B", [1, 32])
def test_none_tail_with_duplicates(orc, B):
    """Plain sparse attention: random lists with duplicates and log-weights.
    B = 1 takes the split-K kernel, B = 32 the one-workgroup-per-unit kernel."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=B, n=2048, n_top=100, C=0)
    c = synth.make_case(w)
    rng = np.random.default_rng(9)
    m = 300
    idx = rng.integers(0, w.n, size=(B, w.Hkv, m)).astype(np.int32)
    logw = rng.normal(0, 1, size=(B, w.Hkv, m)).astype(np.float32)
    d = case_to_dev(c)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), logw=to_dev(logw))
    _sync()
    ref, ref_lse = orc.sparse(c.q, c.K, c.V, idx, logw=logw)
    assert rel_err(out, ref) <= TOL["bf16"]
    assert lse_err(lse, ref_lse) <= LSE_TOL["bf16"]


def test_none_tail_long_list_fp32(orc):
    """A list longer than one workgroup's share (split-K + merge), fp32."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, n, d_ = 2, 4, 2, 5000, 128
    q = rng.standard_normal((B, Hq, d_)).astype(np.float32)
    K = (rng.standard_normal((B, Hkv, n, d_)) + 0.2).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d_)).astype(np.float32)
    idx = np.sort(rng.choice(n, size=(B, Hkv, 3001)), axis=-1).astype(np.int32)
    out, lse = sda.sparse_decode_attn(to_dev(q), to_dev(K), to_dev(V), to_dev(idx))
    _sync()
    ref, ref_lse = orc.sparse(q, K, V, idx)
    assert rel_err(out, ref) <= TOL["f32"]
    assert lse_err(lse, ref_lse) <= LSE_TOL["f32"]


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f32", 1), ("bf16", 8), ("f32", 2)])
def test_dense(orc, dtype, G):
    rng = np.random.default_rng(G)
    B, Hkv, n = 2, 2, 3001
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    K = (rng.standard_normal((B, Hkv, n, 128)) + 0.3).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, 128)).astype(np.float32)
    if dtype == "bf16":
        q, K, V = (synth.round_bf16_bits(a) for a in (q, K, V))
    out, lse = sda.dense_decode_attn(to_dev(q), to_dev(K), to_dev(V))
    _sync()
    ref, ref_lse = orc.dense(q, K, V)
    assert rel_err(out, ref) <= TOL[dtype]
    assert lse_err(lse, ref_lse) <= LSE_TOL[dtype]


def test_prior_build_and_decode(orc):
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(B=2, n=8192, n_top=300)
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    _sync()
    muK, Oest, maxP, sumP = orc.prior_build(c.K, c.V, c.mu_Q)
    assert rel_err(ps.mu_K, muK) <= 1e-5
    assert rel_err(ps.O_est, Oest) <= TOL["bf16"]
    z_gpu = ps.maxP.double().cpu().numpy() + np.log(ps.sumP.double().cpu().numpy())
    assert np.abs(z_gpu - (maxP + np.log(sumP))).max() <= 1e-3
    for lam in (1.0, 0.37, 0.0):
        out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=ps, lam=lam)
        _sync()
        ref, ref_lse = orc.sparse_prior(c.q, c.K, c.V, c.idx, c.mu_Q, lam, muK, Oest, maxP, sumP)
        assert rel_err(out, ref) <= TOL["bf16"], lam
        assert lse_err(lse, ref_lse) <= LSE_TOL["bf16"], lam
    # empty read set: the prior alone (O_est)
    lens = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    out, _ = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], idx_len=lens, tail=ps)
    _sync()
    assert rel_err(out, Oest) <= TOL["bf16"]


def test_device_flags(orc):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, n=2048, n_top=60, C=8)
    c = synth.make_case(w)
    idx = c.idx.copy()
    idx[0, 1, 5] = w.n + 3          # out of range -> skipped, flagged
    idx[0, 2, 10], idx[0, 2, 11] = idx[0, 2, 11], idx[0, 2, 10]   # order broken
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    out, _ = sda.sparse_decode_attn(d["q"], d["K"], d["V"], to_dev(idx), tail=st, cluster_id=d["cid"], flags=flags)
    _sync()
    f = flags.cpu().numpy()
    assert f[0, 1] & sda.FLAG_IDX_RANGE
    assert f[0, 2] & sda.FLAG_IDX_ORDER
    assert f[0, 0] == 0 and (f[0, 3:] == 0).all()
    # untouched units still match the oracle
    ref, _ = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
    keep = [0] + list(range(3, w.Hkv))
    G = w.G
    rows = [h for g in keep for h in range(g * G, (g + 1) * G)]
    assert rel_err(out[:, rows], ref[:, rows]) <= TOL["bf16"]


def test_interleaved_kv_layout(orc):
    """K and V as views into one [B, Hkv, n, 2, d] buffer (strided rows)."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=2048, n_top=60, C=8)
    c = synth.make_case(w)
    d = case_to_dev(c)
    kv = torch.stack([d["K"], d["V"]], dim=3).contiguous()     # [B,Hkv,n,2,d]
    Kv, Vv = kv[:, :, :, 0, :], kv[:, :, :, 1, :]
    st = sda.build_tail_proxies(Kv, Vv, d["cid"], w.C)
    out, lse = sda.sparse_decode_attn(d["q"], Kv, Vv, d["idx"], tail=st, idx_cluster=d["idx_cluster"])
    _sync()
    ref, _ = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
    assert rel_err(out, ref) <= TOL["bf16"]
    dense, _ = sda.dense_decode_attn(d["q"], Kv, Vv)
    _sync()
    ref_d, _ = orc.dense(c.q, c.K, c.V)
    assert rel_err(dense, ref_d) <= TOL["bf16"]
