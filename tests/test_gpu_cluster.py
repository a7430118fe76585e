"""GPU parity of the query-geometry clustering ("OpenAttention" stage 01 and
the settings list; readings G1-G4 in oracle/qgc.py): the cluster id of every
row is bit-exact against the oracle (fp64 coordinates, distances added in
coordinate order with no fused multiply-add, centroid sums exact on a 2^-32
grid: the same arithmetic on both sides), and the same as the plain k-means
with exactly rounded means on the sampled full-size units.  Then the ids
drive the proxy builder, the selector and the proxy decode end to end."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from oracle import qgc, qgs
from tests.gpu_util import dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _w(**kw):
    return synth.WORKLOADS["qgs_bf16_b32_n32k"].replace(**kw)


def _v16(c):
    return np.ascontiguousarray(c.U[..., :16])


@pytest.mark.parametrize("C,T,n", [(16, 10, 3001), (64, 10, 5000), (1, 3, 700), (8, 1, 2048)])
def test_clusters_bit_exact(C, T, n):
    w = _w(B=2, Hkv=2, Hq=8, n=n, n_top=20, C=max(C, 2))
    c = synth.make_case(w)
    V = _v16(c)
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    cid = sda.build_qgc_clusters(to_dev(c.K), to_dev(V), C, T=T, flags=flags)
    _sync()
    got = cid.cpu().numpy()
    assert (flags.cpu().numpy() == 0).all()
    for s in range(w.B):
        for g in range(w.Hkv):
            ref = qgc.cluster_unit(c.K[s, g], V[s, g], C, T=T)
            np.testing.assert_array_equal(got[s, g], ref)


def test_clusters_fp32_keys_and_fixed_point():
    """fp32 keys; long run (T = 30) that reaches the fixed point."""
    w = _w(B=1, Hkv=2, Hq=2, n=1500, n_top=20, C=12, dtype="f32")
    c = synth.make_case(w)
    V = _v16(c)
    cid = sda.build_qgc_clusters(to_dev(c.K), to_dev(V), 12, T=30)
    _sync()
    for g in range(w.Hkv):
        z = qgc.project(c.K[0, g], V[0, g])
        a, _, it = qgc.kmeans(z, 12, T=30)
        np.testing.assert_array_equal(cid[0, g].cpu().numpy(), a)


def test_clamped_coordinates_flagged():
    """Keys whose projection exceeds 2048 are clamped there (as in the
    oracle) and flagged."""
    w = _w(B=1, Hkv=1, Hq=4, n=600, n_top=20, C=4, dtype="f32")
    c = synth.make_case(w)
    K = c.K.copy()
    K[0, 0, 17] = 5000.0 * c.U[0, 0][:, 0]          # projection 5000 on the first axis
    V = _v16(c)
    flags = torch.zeros((1, 1), dtype=torch.int32, device=dev())
    cid = sda.build_qgc_clusters(to_dev(K), to_dev(V), 4, T=5, flags=flags)
    _sync()
    assert flags.cpu().numpy()[0, 0] & sda.FLAG_CLUSTER
    np.testing.assert_array_equal(cid[0, 0].cpu().numpy(), qgc.cluster_unit(K[0, 0], V[0, 0], 4, T=5))


def test_clusters_full_size_b32_n32k():
    """The timed shape (batch 32, 32K rows, C = 64, 10 passes): 4 sampled
    units bit-exact against the oracle, and the same as the plain k-means
    (exactly rounded means) on 2 of them; every id in range."""
    w = _w(C=64)
    c = synth.make_case(w)
    V = _v16(c)
    cid = sda.build_qgc_clusters(to_dev(c.K), to_dev(V), 64, T=10)
    _sync()
    got = cid.cpu().numpy()
    assert got.min() >= 0 and got.max() < 64
    rng = np.random.default_rng(7)
    for i, u in enumerate(rng.choice(w.B * w.Hkv, size=4, replace=False)):
        s, g = divmod(int(u), w.Hkv)
        np.testing.assert_array_equal(got[s, g], qgc.cluster_unit(c.K[s, g], V[s, g], 64, T=10))
        if i < 2:
            np.testing.assert_array_equal(got[s, g], qgc.cluster_unit_plain(c.K[s, g], V[s, g], 64, T=10))


def test_clusters_feed_selector_and_decode(orc):
    """Ids from the GPU clustering -> proxy builder -> selector -> proxy
    decode, against the oracle chain on the oracle's own ids."""
    w = _w(B=1, Hkv=2, Hq=8, n=4096, n_top=100, C=64)
    c = synth.make_case(w)
    V = _v16(c)
    K, Vv, q, U = to_dev(c.K), to_dev(c.V), to_dev(c.q), to_dev(c.U)
    cid = sda.build_qgc_clusters(K, to_dev(V), 64, T=10)
    st = sda.build_tail_proxies(K, Vv, cid, 64, with_sumK2=True)
    qc = sda.build_qgs_codes(K, U)
    idx, idx_len, icl = sda.select_qgs(q, K, cid, st, qc, w.n_sink, w.n_local, w.n_top)
    out, lse = sda.sparse_decode_attn(q, K, Vv, idx, idx_len=idx_len, tail=st, idx_cluster=icl)
    _sync()
    checked = 0
    for g in range(w.Hkv):
        ocid = qgc.cluster_unit(c.K[0, g], V[0, g], 64, T=10)
        np.testing.assert_array_equal(cid[0, g].cpu().numpy(), ocid)
        o = qgs.select_unit(c.q[0, g * 4:(g + 1) * 4], c.K[0, g], ocid, 64, c.U[0, g], w.n_sink, w.n_local,
                            w.n_top, np.float32(1.0 / np.sqrt(w.d)))
        if o["margin"] < 1e-3:
            continue
        checked += 1
        np.testing.assert_array_equal(idx[0, g, :int(idx_len[0, g])].cpu().numpy(), o["idx"])
        ref, ref_lse = orc.sparse_proxy_def(c.q[:, g * 4:(g + 1) * 4], c.K[:, g:g + 1], c.V[:, g:g + 1],
                                            o["idx"][None, None], ocid[None, None], 64)
        assert rel_err(out[0, g * 4:(g + 1) * 4], ref[0]) <= 2e-3
        assert np.abs(lse[0, g * 4:(g + 1) * 4].cpu().double().numpy() - ref_lse[0]).max() <= 1e-3
    assert checked >= 1
