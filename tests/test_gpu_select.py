"""GPU parity of the selector (QGS codes and scores, ErrorGate budgets,
per-cluster top-q; "OpenAttention", method stages 01-03) against the oracle
in oracle/qgs.py.

Bit-exact: the int8 codes, the fp64 coordinate maxima, the budgets and every
listed row, with the oracle's ErrorGate fed the GPU builder's own cluster
count and fp32 sums (so both sides start from the same numbers); only a unit
whose budget decision lies within a few fp64 roundings of a tie (margin below
EXACT_MARGIN) is checked for validity instead.  Separately, against the
oracle's fp64 cluster sums: units whose decision is clear by MARGIN match bit
for bit, the others must be valid -- the budget spent in full, no cluster
above its eligible rows, at most two rows moved between clusters, and every
cluster listing exactly its top-q_b rows by the oracle's exact scores.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from oracle import qgs
from tests.gpu_util import dev, rel_err, to_dev

pytestmark = pytest.mark.gpu

MARGIN = 1e-3         # against the oracle's fp64 cluster sums
EXACT_MARGIN = 1e-9   # against the GPU builder's sums: a few fp64 roundings


def _sync():
    torch.cuda.synchronize()


def _workload(**kw):
    return synth.WORKLOADS["qgs_bf16_b32_n32k"].replace(**kw)


def _gpu_select(c, w, E=None, n_sink=None, n_local=None, cid=None):
    E = w.n_top if E is None else E
    n_sink = w.n_sink if n_sink is None else n_sink
    n_local = w.n_local if n_local is None else n_local
    K, V, q, U = to_dev(c.K), to_dev(c.V), to_dev(c.q), to_dev(c.U)
    cid_d = to_dev(c.cid if cid is None else cid)
    st = sda.build_tail_proxies(K, V, cid_d, w.C, with_sumK2=True)
    qc = sda.build_qgs_codes(K, U)
    budget = torch.zeros((w.B, w.Hkv, w.C), dtype=torch.int32, device=dev())
    flags = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev())
    idx, idx_len, icl = sda.select_qgs(q, K, cid_d, st, qc, n_sink, n_local, E, budget=budget, flags=flags)
    _sync()
    return dict(K=K, V=V, q=q, st=st, qc=qc, idx=idx, idx_len=idx_len, icl=icl, budget=budget, flags=flags,
                cid=cid_d)


def _check_unit(r, s, g, q, K, cid, U, w, E, n_sink, n_local):
    """Compares unit (s, g) with the oracle; returns True if its budget
    decision was fragile against the oracle's own fp64 sums (then only
    validity is checked there)."""
    sc = np.float32(1.0 / np.sqrt(w.d))
    gb = r["budget"][s, g].cpu().numpy()
    L = int(r["idx_len"][s, g])
    gidx = r["idx"][s, g, :L].cpu().numpy()
    gicl = r["icl"][s, g, :L].cpu().numpy()
    m = r["idx"].shape[-1]
    assert (r["idx"][s, g, L:].cpu().numpy() == 0).all() and (r["icl"][s, g, L:].cpu().numpy() == -1).all()
    # the listed rows' cluster ids are the rows' own
    own = np.where((cid[gidx] >= 0) & (cid[gidx] < w.C), cid[gidx], -1)
    np.testing.assert_array_equal(gicl, own)
    assert L <= m and (np.diff(gidx) > 0).all()
    # 1. the same inputs on both sides: the GPU builder's count and sums
    st = r["st"]
    stats = (st.count[s, g].cpu().numpy().astype(np.int64), st.sumK[s, g].cpu().double().numpy(),
             st.sumK2[s, g].cpu().double().numpy())
    og = qgs.select_unit(q, K, cid, w.C, U, n_sink, n_local, E, sc, stats=stats)
    if og["margin"] >= EXACT_MARGIN:
        np.testing.assert_array_equal(gb, og["budget"])
        np.testing.assert_array_equal(gidx, og["idx"])
    # 2. the oracle's own fp64 sums
    o = qgs.select_unit(q, K, cid, w.C, U, n_sink, n_local, E, sc)
    if o["margin"] >= MARGIN:
        np.testing.assert_array_equal(gb, o["budget"])
        np.testing.assert_array_equal(gidx, o["idx"])
        return False
    # fragile: valid allocation and per-cluster top-q by the oracle's scores
    assert gb.sum() == min(E, o["avail"].sum()) and (gb <= o["avail"]).all()
    assert np.abs(gb - o["budget"]).sum() <= 2
    expect = qgs.select(o["scores"], cid, gb, n_sink, n_local)
    np.testing.assert_array_equal(gidx, expect)
    return True


def test_codes_and_maxima_bit_exact():
    """Codes and kmax of every unit, bf16 keys, ragged n (several 256-row
    chunks and a partial one)."""
    w = _workload(B=2, Hkv=2, Hq=8, n=3001, n_top=40, C=8)
    c = synth.make_case(w)
    qc = sda.build_qgs_codes(to_dev(c.K), to_dev(c.U))
    _sync()
    codes, kmax = qc.codes.cpu().numpy(), qc.kmax.cpu().numpy()
    for s in range(w.B):
        for g in range(w.Hkv):
            oc, ok = qgs.codes(c.K[s, g], c.U[s, g])
            np.testing.assert_array_equal(kmax[s, g], ok)
            np.testing.assert_array_equal(codes[s, g], oc)


def test_codes_without_room_for_the_projections():
    """A workspace that holds only the chunk maxima: the quantizing pass
    recomputes the projections and the codes and kmax are the same bits as
    with the projections kept (and as the oracle's)."""
    import ctypes
    w = _workload(B=2, Hkv=2, Hq=8, n=3001, n_top=40, C=8)
    c = synth.make_case(w)
    K, U = to_dev(c.K), to_dev(c.U)
    full = sda.build_qgs_codes(K, U)
    dims = sda.make_dims(K, 1)
    dims.Hq = dims.Hkv
    need = sda.workspace_bytes(dims, sda.OP_BUILD_QGS)
    small = need - w.B * w.Hkv * w.n * sda.QGS_RANK * 8
    assert 0 < small < need
    ws = torch.empty(small, dtype=torch.uint8, device=dev())
    codes = torch.empty_like(full.codes)
    kmax = torch.empty_like(full.kmax)
    L = sda.lib()
    assert L.sda_build_qgs_codes(ctypes.byref(dims), K.data_ptr(), U.data_ptr(), codes.data_ptr(), kmax.data_ptr(),
                                 ws.data_ptr(), small - 1, None) == sda.SDA_EWORKSPACE
    rc = L.sda_build_qgs_codes(ctypes.byref(dims), K.data_ptr(), U.data_ptr(), codes.data_ptr(), kmax.data_ptr(),
                               ws.data_ptr(), small, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    _sync()
    assert torch.equal(codes, full.codes) and torch.equal(kmax, full.kmax)
    oc, ok = qgs.codes(c.K[1, 1], c.U[1, 1])
    np.testing.assert_array_equal(codes[1, 1].cpu().numpy(), oc)


def test_codes_fp32_keys():
    w = _workload(B=1, Hkv=2, Hq=2, n=700, n_top=20, C=4, dtype="f32")
    c = synth.make_case(w)
    qc = sda.build_qgs_codes(to_dev(c.K), to_dev(c.U))
    _sync()
    for g in range(w.Hkv):
        oc, ok = qgs.codes(c.K[0, g], c.U[0, g])
        np.testing.assert_array_equal(qc.kmax[0, g].cpu().numpy(), ok)
        np.testing.assert_array_equal(qc.codes[0, g].cpu().numpy(), oc)


def test_squared_key_sums():
    """The cluster cache's sum of squared keys (and the other sums) against
    the oracle's fp64 sums; counts bit-exact."""
    w = _workload(B=2, Hkv=2, Hq=8, n=5000, n_top=40, C=16)
    c = synth.make_case(w)
    st = sda.build_tail_proxies(to_dev(c.K), to_dev(c.V), to_dev(c.cid), w.C, with_sumK2=True)
    _sync()
    for s in range(w.B):
        for g in range(w.Hkv):
            N, S1, S2 = qgs.cluster_stats(c.K[s, g], c.cid[s, g], w.C)
            np.testing.assert_array_equal(st.count[s, g].cpu().numpy(), N)
            assert rel_err(st.sumK[s, g], S1) <= 1e-6
            assert rel_err(st.sumK2[s, g], S2) <= 1e-6


@pytest.mark.parametrize("G,C,E,n", [(4, 16, 100, 4500), (1, 8, 60, 4500), (2, 32, 200, 4500),
                                     (8, 64, 300, 4500), (4, 48, 150, 4500), (4, 8, 120, 40000),
                                     (2, 64, 200, 40000)])
def test_select_small(G, C, E, n):
    """Whole selector on small workloads: G = 1..8, C up to 64 (7-bit radix
    digits up to 32 clusters, 6-bit beyond), n with a ragged last score
    chunk.  n = 40000 takes the three-launch path (workspace keys), the
    others the one-launch path (LDS records)."""
    w = _workload(B=2, Hkv=2, Hq=2 * G, n=n, n_top=E, C=C)
    c = synth.make_case(w)
    r = _gpu_select(c, w)
    assert (r["flags"].cpu().numpy() == 0).all()
    fragile = 0
    for s in range(w.B):
        for g in range(w.Hkv):
            fragile += _check_unit(r, s, g, c.q[s, g * G:(g + 1) * G], c.K[s, g], c.cid[s, g], c.U[s, g], w, E,
                                   w.n_sink, w.n_local)
    assert fragile <= 1


def test_select_general_clusters_and_edges():
    """Non-contiguous cluster ids with -1 rows; then budget 0, a budget above
    the eligible rows, and sink + local covering the whole cache."""
    w = _workload(B=1, Hkv=2, Hq=8, n=2000, n_top=50, C=12)
    c = synth.make_case(w)
    rng = np.random.default_rng(11)
    cid = rng.integers(-1, w.C, size=c.cid.shape).astype(np.int32)
    for E, ns, nl in ((50, 4, 64), (0, 4, 64), (5000, 4, 64), (50, 1000, 1500)):
        r = _gpu_select(c, w, E=E, n_sink=ns, n_local=nl, cid=cid)
        for g in range(w.Hkv):
            _check_unit(r, 0, g, c.q[0, g * 4:(g + 1) * 4], c.K[0, g], cid[0, g], c.U[0, g], w, E, ns, nl)
        if E == 5000:     # every eligible row is listed
            el = (cid[0] >= 0) & (np.arange(w.n) >= 4) & (np.arange(w.n) < w.n - 64)
            assert (r["idx_len"].cpu().numpy()[0] == 68 + el.sum(axis=-1)).all()
        if ns + nl >= w.n:
            assert (r["idx_len"].cpu().numpy() == w.n).all()


def test_select_feeds_proxy_decode(orc):
    """Selector output straight into the proxy decode: the attention output
    equals the oracle's definition on the oracle's own index set."""
    w = _workload(B=2, Hkv=2, Hq=8, n=4096, n_top=100, C=16)
    c = synth.make_case(w)
    r = _gpu_select(c, w)
    out, lse = sda.sparse_decode_attn(r["q"], r["K"], r["V"], r["idx"], idx_len=r["idx_len"], tail=r["st"],
                                      idx_cluster=r["icl"])
    _sync()
    checked = 0
    for s in range(w.B):
        for g in range(w.Hkv):
            o = qgs.select_unit(c.q[s, g * 4:(g + 1) * 4], c.K[s, g], c.cid[s, g], w.C, c.U[s, g], w.n_sink,
                                w.n_local, w.n_top, np.float32(1.0 / np.sqrt(w.d)))
            if o["margin"] < MARGIN:
                continue
            checked += 1
            np.testing.assert_array_equal(r["idx"][s, g].cpu().numpy(), o["idx"])
            uc = synth.unit_case(w, s, g)
            ref, ref_lse = orc.sparse_proxy_def(uc.q, uc.K, uc.V, o["idx"][None, None], uc.cid, w.C)
            rows = slice(g * 4, (g + 1) * 4)
            assert rel_err(out[s, rows], ref[0]) <= 2e-3
            assert np.abs(lse[s, rows].cpu().double().numpy() - ref_lse[0]).max() <= 1e-3
    assert checked >= 3


def test_select_full_size_b32_n32k():
    """The selector at the timed shape (batch 32, 32K, 32 clusters, 260 rows
    to pick): every unit's list is valid; 8 sampled units against the
    oracle."""
    w = synth.WORKLOADS["qgs_bf16_b32_n32k"]
    c = synth.make_case(w)
    r = _gpu_select(c, w)
    assert (r["flags"].cpu().numpy() == 0).all()
    lens = r["idx_len"].cpu().numpy()
    assert (lens == w.n_sink + w.n_local + w.n_top).all()
    assert (r["budget"].cpu().numpy().sum(axis=-1) == w.n_top).all()
    idx = r["idx"].cpu().numpy()
    assert (np.diff(idx, axis=-1) > 0).all()
    rng = np.random.default_rng(6)
    fragile = 0
    for u in rng.choice(w.B * w.Hkv, size=8, replace=False):
        s, g = divmod(int(u), w.Hkv)
        fragile += _check_unit(r, s, g, c.q[s, g * w.G:(g + 1) * w.G], c.K[s, g], c.cid[s, g], c.U[s, g], w,
                               w.n_top, w.n_sink, w.n_local)
    assert fragile <= 2
