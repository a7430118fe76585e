"""GPU parity of the proxy tail with lists longer than the one-pass kernel
holds ("OpenAttention: One Percent Is Enough with Tail Proxies", method stage
04: each cluster's unread tokens fold into one virtual token; key points: 3%
read, 96K context).  Up to 1024 entries the library runs one workgroup per
unit that streams the value rows behind the key rows; beyond that split-K on
the matrix cores, each split keeping per-cluster listed counts, logit sums
and value sums that a merge adds before it forms the proxies (the log-weight
and ragged case with 1268 entries).  Against the oracle's O(n) definition,
max rel err <= 2e-3 (bf16 inputs)."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, dev, lse_err, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
LSE_TOL = 1e-3


def _pct(n, frac):
    return int(np.ceil(n * frac - 1e-9))


def _check(orc, w, c, d, idx_cluster=True, logw=None, idx_len=None):
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    kw = dict(idx_cluster=d["idx_cluster"]) if idx_cluster else dict(cluster_id=d["cid"])
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st, flags=flags,
                                      logw=None if logw is None else to_dev(logw),
                                      idx_len=None if idx_len is None else to_dev(idx_len), **kw)
    torch.cuda.synchronize()
    assert (flags.cpu().numpy() == 0).all()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C, idx_len=idx_len, logw=logw)
    err = rel_err(out, ref)
    assert err <= TOL, err
    assert lse_err(lse, ref_lse) <= LSE_TOL
    return err


def _long_list(w, m):
    """The list is longer than the one-pass kernel takes (512 entries, 384
    at eight query heads per KV head)."""
    return m > (384 if w.G == 8 else 512)


def _split_k(d, w, m):
    """Beyond 1024 entries: split-K, whose per-cluster records need a
    workspace."""
    return sda.workspace_bytes(sda.make_dims(d["K"], w.Hq), sda.OP_SPARSE, sda.TAIL_PROXY, m, w.C) > 0


def test_proxy_32k_three_percent(orc):
    """Batch 2, 32K rows, 3% read (984 listed rows per KV head), 32 random
    contiguous clusters."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n_top=_pct(32768, 0.03) - 68)
    c = synth.make_case(w)
    d = case_to_dev(c)
    assert c.idx.shape[-1] == 984 and _long_list(w, 984) and not _split_k(d, w, 984)
    _check(orc, w, c, d)


def test_proxy_96k_one_percent(orc):
    """One sequence of 98,304 rows, 1% read (984 listed rows per KV head)."""
    n = 98304
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, n=n, n_top=_pct(n, 0.01) - 68)
    c = synth.make_case(w)
    d = case_to_dev(c)
    assert _long_list(w, c.idx.shape[-1])
    _check(orc, w, c, d)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_proxy_long_group_sizes(orc, G):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, Hq=2 * G, Hkv=2, n=8192, n_top=700, C=37)
    c = synth.make_case(w)
    d = case_to_dev(c)
    assert _long_list(w, c.idx.shape[-1])
    _check(orc, w, c, d, idx_cluster=(G != 2))


def test_proxy_long_logw_and_ragged(orc):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=16384, n_top=1200, C=20)
    c = synth.make_case(w)
    d = case_to_dev(c)
    rng = np.random.default_rng(3)
    logw = rng.normal(0.0, 0.5, size=c.idx.shape).astype(np.float32)
    lens = rng.integers(0, c.idx.shape[-1] + 1, size=(w.B, w.Hkv)).astype(np.int32)
    lens[0, 0], lens[0, 1] = 0, c.idx.shape[-1]
    assert _split_k(d, w, c.idx.shape[-1])
    _check(orc, w, c, d, logw=logw, idx_len=lens)


def test_proxy_long_list_logw_and_ragged(orc):
    """The same on the one-workgroup long-list path (1000 entries)."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=16384, n_top=932, C=20)
    c = synth.make_case(w)
    d = case_to_dev(c)
    rng = np.random.default_rng(6)
    logw = rng.normal(0.0, 0.5, size=c.idx.shape).astype(np.float32)
    lens = rng.integers(0, c.idx.shape[-1] + 1, size=(w.B, w.Hkv)).astype(np.int32)
    lens[0, 0], lens[0, 1], lens[1, 2] = 0, c.idx.shape[-1], 513
    assert _long_list(w, c.idx.shape[-1]) and not _split_k(d, w, c.idx.shape[-1])
    _check(orc, w, c, d, logw=logw, idx_len=lens)


def test_proxy_long_general_clusters_c64(orc):
    """Non-contiguous cluster ids (every row's cluster drawn at random, some
    rows in no cluster), 64 clusters: every split touches every cluster."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, n=12000, n_top=900, C=64)
    c = synth.make_case(w)
    rng = np.random.default_rng(4)
    cid = rng.integers(-1, 64, size=c.cid.shape).astype(np.int32)
    c.cid = cid
    d = case_to_dev(c)
    _check(orc, w, c, d)
    _check(orc, w, c, d, idx_cluster=False)


def test_proxy_long_mostly_read_clusters(orc):
    """The cancellation case on the long-list path: clusters of 256 rows
    with 254 listed (low logits) and 2 unread near the unit's largest logit."""
    rng = np.random.default_rng(5)
    B, Hkv, G, n, d_, C, size, m = 1, 4, 4, 8192, 128, 32, 256, 900
    q = synth.round_bf16_bits(rng.standard_normal((B, G * Hkv, d_)).astype(np.float32))
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    K = (0.5 * rng.standard_normal((B, Hkv, n, d_))).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d_)).astype(np.float32)
    cid = np.broadcast_to((np.arange(n) // size).astype(np.int32), (B, Hkv, n)).copy()
    idx = np.empty((B, Hkv, m), np.int32)
    for g in range(Hkv):
        qb = qf[0, g * G:(g + 1) * G].mean(axis=0)
        aligned = np.sqrt(d_) * qb / (qb @ qb)
        listed = set(range(4)) | set(range(n - 64, n))
        K[0, g, n - 1] = 14.5 * aligned
        for b in rng.choice(np.arange(1, C - 1), size=3, replace=False):
            members = np.arange(b * size, (b + 1) * size)
            unread = rng.choice(members, size=2, replace=False)
            K[0, g, unread[0]] = 14.0 * aligned
            K[0, g, unread[1]] = 13.6 * aligned + 0.3 * rng.standard_normal(d_)
            V[0, g, members] = 3.0 * rng.standard_normal(d_) + 0.01 * rng.standard_normal((size, d_))
            listed |= set(members.tolist()) - set(unread.tolist())
        rest = np.setdiff1d(np.arange(n), np.fromiter(listed, int))
        listed |= set(rng.choice(rest, size=m - len(listed), replace=False).tolist())
        idx[0, g] = np.sort(np.fromiter(listed, np.int32))
    K, V = synth.round_bf16_bits(K), synth.round_bf16_bits(V)
    st = sda.build_tail_proxies(to_dev(K), to_dev(V), to_dev(cid), C)
    out, lse = sda.sparse_decode_attn(to_dev(q), to_dev(K), to_dev(V), to_dev(idx), tail=st, cluster_id=to_dev(cid))
    torch.cuda.synchronize()
    ref, ref_lse = orc.sparse_proxy_def(q, K, V, idx, cid, C)
    err = rel_err(out, ref)
    print(f"mostly-read clusters, long list: max rel err {err:.3e} (tolerance {TOL:.0e})")
    assert err <= TOL
    assert lse_err(lse, ref_lse) <= LSE_TOL


def test_proxy_long_twice_and_flags():
    """The same call twice gives the same bits; a listed row counted beyond
    its cluster's count is flagged."""
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=8192, n_top=800, C=16)
    c = synth.make_case(w)
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    a = [t.clone() for t in sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st,
                                                   idx_cluster=d["idx_cluster"])]
    b = [t.clone() for t in sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st,
                                                   idx_cluster=d["idx_cluster"])]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.cpu(), y.cpu())
    bad = sda.ProxyState(C=st.C, count=st.count.clone(), sumK=st.sumK, sumV=st.sumV)
    bad.count[0, 1, :] = 0
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=bad, idx_cluster=d["idx_cluster"], flags=flags)
    torch.cuda.synchronize()
    f = flags.cpu().numpy()
    assert f[0, 1] & sda.FLAG_CLUSTER and f[1, 0] == 0


def test_long_list_edges(orc):
    """The one-workgroup long-list path at its limits: 1024 entries at eight
    query heads per KV head; an interleaved K|V cache with the cluster looked
    up per row and a single cluster; every cluster entirely listed (no proxy
    at all: plain sparse attention over the list); empty and one-entry units."""
    # 1024 entries, G = 8
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, Hq=16, Hkv=2, n=8192, n_top=956, C=24)
    c = synth.make_case(w)
    d = case_to_dev(c)
    assert c.idx.shape[-1] == 1024 and _long_list(w, 1024) and not _split_k(d, w, 1024)
    _check(orc, w, c, d)
    # interleaved K|V, cluster lookup, C = 1
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, n=6000, n_top=700, C=1, seg="equal")
    c = synth.make_case(w)
    kv = np.stack([c.K, c.V], axis=3)              # [B, Hkv, n, 2, d]
    KV = to_dev(kv)
    K, V = KV[:, :, :, 0, :], KV[:, :, :, 1, :]
    cid = to_dev(c.cid)
    st = sda.build_tail_proxies(K, V, cid, w.C)
    out, lse = sda.sparse_decode_attn(to_dev(c.q), K, V, to_dev(c.idx), tail=st, cluster_id=cid)
    torch.cuda.synchronize()
    ref, ref_lse = orc.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
    assert rel_err(out, ref) <= TOL and lse_err(lse, ref_lse) <= LSE_TOL
    # every cluster entirely listed: the clusters are the listed rows' own, so
    # n_b = 0 for all and the result is plain sparse attention
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=1, n=4096, n_top=632, C=8)
    c = synth.make_case(w)
    cid = np.full(c.cid.shape, -1, np.int32)
    for g in range(w.Hkv):
        cid[0, g, c.idx[0, g]] = np.arange(c.idx.shape[-1]) * 8 // c.idx.shape[-1]
    c.cid = cid
    d = case_to_dev(c)
    st = sda.build_tail_proxies(d["K"], d["V"], d["cid"], w.C)
    out, lse = sda.sparse_decode_attn(d["q"], d["K"], d["V"], d["idx"], tail=st, idx_cluster=d["idx_cluster"])
    torch.cuda.synchronize()
    ref, ref_lse = orc.sparse(c.q, c.K, c.V, c.idx)
    assert rel_err(out, ref) <= TOL and lse_err(lse, ref_lse) <= LSE_TOL
    # empty and one-entry units
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=8192, n_top=700, C=16)
    c = synth.make_case(w)
    d = case_to_dev(c)
    lens = np.full((w.B, w.Hkv), c.idx.shape[-1], np.int32)
    lens[0, :4] = 0
    lens[1, 3] = 1
    _check(orc, w, c, d, idx_len=lens)
