"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects malformed arguments on the host before any
launch (these calls return before touching HIP, so fake pointers are safe)."""
import ctypes
import os
import re

import pytest

from long_context_sparse_gathered_amd import sda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)      # never dereferenced on these paths
FAKE2 = ctypes.c_void_p(0x200000)
MISALIGNED = ctypes.c_void_p(0x100004)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sda.LIB_PATH):
        pytest.skip("libsda.so not built")
    return sda.lib()


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:sda_status|size_t|const char\*)\s+(sda_\w+)\s*\(", text, re.M))
    return names


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"sda_build_tail_proxies", "sda_build_prior", "sda_sparse_decode_attn",
            "sda_dense_decode_attn", "sda_workspace_bytes"} <= names
    for name in names:
        assert hasattr(L, name), name
    assert set(sda.EXPORTED) == names


def test_status_strings_and_version(L):
    assert sda.status_str(0) == "ok"
    assert "workspace" in sda.status_str(-4)
    assert re.match(r"\d+\.\d+\.\d+", sda.version())


def _dims(**kw):
    d = dict(B=2, Hq=8, Hkv=2, n=1024, d=128, dtype=sda.SDA_BF16, kv_stride_b=0, kv_stride_h=0,
             kv_stride_n=0, scale=0.0)
    d.update(kw)
    return sda.Dims(**d)


def _sparse(L, dims, tail=None, m=16, q=FAKE, K=FAKE, V=FAKE, idx=FAKE2, ws=None, ws_bytes=0, out=FAKE):
    t = tail if tail is not None else sda.Tail()
    return L.sda_sparse_decode_attn(ctypes.byref(dims) if dims is not None else None, q, K, V, idx, None, None,
                                    m, ctypes.byref(t), out, None, None, ws, ws_bytes, None)


def test_dims_validation(L):
    assert _sparse(L, None) == sda.SDA_EINVAL
    assert _sparse(L, _dims(dtype=7)) == sda.SDA_EDTYPE
    assert _sparse(L, _dims(d=64)) == sda.SDA_EUNSUPPORTED
    assert _sparse(L, _dims(Hq=6, Hkv=4)) == sda.SDA_ESHAPE
    assert _sparse(L, _dims(Hq=6, Hkv=2)) == sda.SDA_EUNSUPPORTED     # group of 3
    assert _sparse(L, _dims(n=0)) == sda.SDA_ESHAPE
    assert _sparse(L, _dims(B=0)) == sda.SDA_ESHAPE
    # explicit strides: row stride below d, or misaligned for 16-byte loads
    assert _sparse(L, _dims(kv_stride_b=2 * 1024 * 128, kv_stride_h=1024 * 128, kv_stride_n=64)) == sda.SDA_ESHAPE
    assert _sparse(L, _dims(kv_stride_b=2 * 1024 * 136, kv_stride_h=1024 * 136, kv_stride_n=132)) == sda.SDA_ESHAPE
    # a unit too large for 32-bit row offsets
    assert _sparse(L, _dims(n=1 << 24, dtype=sda.SDA_F32)) == sda.SDA_EUNSUPPORTED
    assert _sparse(L, _dims(scale=-1.0)) == sda.SDA_EINVAL


def test_argument_validation(L):
    dims = _dims()
    assert _sparse(L, dims, q=None) == sda.SDA_EINVAL
    assert _sparse(L, dims, out=None) == sda.SDA_EINVAL
    assert _sparse(L, dims, K=MISALIGNED) == sda.SDA_EINVAL
    assert _sparse(L, dims, m=-1) == sda.SDA_ESHAPE
    assert _sparse(L, dims, m=0) == sda.SDA_EINVAL                    # nothing to attend to
    assert _sparse(L, dims, idx=None) == sda.SDA_EINVAL
    bad = sda.Tail()
    bad.kind = 9
    assert _sparse(L, dims, tail=bad) == sda.SDA_EINVAL


def test_proxy_tail_validation(L):
    dims = _dims()
    t = sda.Tail()
    t.kind = sda.TAIL_PROXY
    t.C = 0
    assert _sparse(L, dims, tail=t) == sda.SDA_EUNSUPPORTED
    t.C = 65
    assert _sparse(L, dims, tail=t) == sda.SDA_EUNSUPPORTED
    t.C = 32
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL                 # no state
    t.count, t.sumK, t.sumV = FAKE, FAKE, FAKE
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL                 # no cluster lookup
    t.cluster_id = FAKE2
    # up to 1024 entries (bf16) one workgroup per unit, no workspace; longer
    # lists split across workgroups with per-cluster records, which need a
    # workspace; fp32 rows take only the one-pass kernel (m <= 512)
    assert L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SPARSE, sda.TAIL_PROXY, 600, 32) == 0
    assert L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SPARSE, sda.TAIL_PROXY, 1024, 32) == 0
    need = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SPARSE, sda.TAIL_PROXY, 1025, 32)
    assert need > 0
    assert _sparse(L, dims, tail=t, m=1025) == sda.SDA_EWORKSPACE
    assert _sparse(L, dims, tail=t, m=1025, ws=FAKE2, ws_bytes=need - 1) == sda.SDA_EWORKSPACE
    d32 = _dims()
    d32.dtype = sda.SDA_F32
    assert _sparse(L, d32, tail=t, m=600) == sda.SDA_EUNSUPPORTED


def test_prior_tail_validation(L):
    dims = _dims()
    t = sda.Tail()
    t.kind = sda.TAIL_PRIOR
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL
    t.mu_Q, t.mu_K, t.O_est, t.maxP, t.sumP = FAKE, FAKE, FAKE, FAKE, FAKE
    t.lam = -0.5
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL
    t.lam = float("nan")
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL
    t.lam = 1.0
    t.prior_n = dims.n + 1                      # more rows than the cache holds
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL
    t.prior_n = -1
    assert _sparse(L, dims, tail=t) == sda.SDA_EINVAL
    t.prior_n = 0
    # B*Hkv = 4 units: the split-K path needs a workspace
    need = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SPARSE, sda.TAIL_PRIOR, 2000, 0)
    assert need > 0
    assert _sparse(L, dims, tail=t, m=2000) == sda.SDA_EWORKSPACE
    assert _sparse(L, dims, tail=t, m=2000, ws=FAKE2, ws_bytes=need - 1) == sda.SDA_EWORKSPACE


def test_builder_and_dense_validation(L):
    dims = _dims()
    assert L.sda_build_tail_proxies(ctypes.byref(dims), FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, None, None, FAKE,
                                    1 << 30, None) == sda.SDA_EUNSUPPORTED
    assert L.sda_build_tail_proxies(ctypes.byref(dims), FAKE, FAKE, None, 8, FAKE, FAKE, FAKE, None, None, FAKE,
                                    1 << 30, None) == sda.SDA_EINVAL
    assert L.sda_build_tail_proxies(ctypes.byref(dims), FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16,
                                    None) == sda.SDA_EWORKSPACE
    assert L.sda_build_prior(ctypes.byref(dims), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 0,
                             None) == sda.SDA_EINVAL
    assert L.sda_dense_decode_attn(ctypes.byref(dims), FAKE, FAKE, FAKE, None, None, None, 0, None) == sda.SDA_EINVAL
    assert L.sda_dense_decode_attn(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, None, None, 0,
                                   None) == sda.SDA_EWORKSPACE


def test_workspace_sizes(L):
    b32 = _dims(B=32, Hq=32, Hkv=8, n=32768)
    assert L.sda_workspace_bytes(ctypes.byref(b32), sda.OP_SPARSE, sda.TAIL_PROXY, 328, 32) == 0
    dense = L.sda_workspace_bytes(ctypes.byref(b32), sda.OP_DENSE, 0, 0, 0)
    assert dense > 0 and dense % (4 * 264 * 4) == 0
    assert L.sda_workspace_bytes(ctypes.byref(b32), sda.OP_BUILD_PRIOR, 0, 0, 0) > dense
    assert L.sda_workspace_bytes(ctypes.byref(b32), sda.OP_BUILD_PROXIES, 0, 0, 32) > 0
    assert L.sda_workspace_bytes(ctypes.byref(b32), sda.OP_BUILD_PROXIES, 0, 0, 99) == 0
    assert L.sda_workspace_bytes(None, sda.OP_DENSE, 0, 0, 0) == 0


def test_selector_validation(L):
    """Host-side checks of the selector entry points (nothing launches)."""
    dims = _dims()
    assert L.sda_build_qgs_codes(ctypes.byref(dims), FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == sda.SDA_EINVAL
    assert L.sda_build_qgs_codes(ctypes.byref(dims), MISALIGNED, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                 None) == sda.SDA_EINVAL
    need = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_BUILD_QGS, 0, 0, 0)
    # fp64 chunk maxima per (unit, chunk, coordinate), rounded up to 256
    # bytes, then the fp64 projections per (unit, row, coordinate)
    least = (2 * 2 * (1024 // 256) * 32 * 8 + 255) // 256 * 256
    assert need == least + 2 * 2 * 1024 * 32 * 8
    assert L.sda_build_qgs_codes(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, least - 1,
                                 None) == sda.SDA_EWORKSPACE

    def sel(**kw):
        f = dict(n_sink=4, n_local=16, E=40, C=8, cluster_id=FAKE, count=FAKE, sumK=FAKE, sumK2=FAKE, U=FAKE,
                 codes=FAKE, kmax=FAKE)
        f.update(kw)
        return sda.Selector(**f)

    def call(s, m=60, ws_bytes=1 << 30, d=dims):
        return L.sda_select_qgs(ctypes.byref(d), FAKE, ctypes.byref(s), m, FAKE, FAKE, FAKE, None, None, FAKE,
                                ws_bytes, None)

    assert call(sel(C=0)) == sda.SDA_EUNSUPPORTED
    assert call(sel(C=65)) == sda.SDA_EUNSUPPORTED
    assert call(sel(sumK2=None)) == sda.SDA_EINVAL
    assert call(sel(E=-1)) == sda.SDA_EINVAL
    assert call(sel(), m=59) == sda.SDA_EINVAL                  # capacity below 4 + 16 + 40
    assert call(sel(codes=MISALIGNED)) == sda.SDA_EINVAL
    big = _dims(n=(1 << 20) + 1, B=1, Hq=4, Hkv=1)
    assert call(sel(), d=big) == sda.SDA_EUNSUPPORTED
    wsel = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SELECT_QGS, 0, 0, 8)
    assert wsel >= 4 * 1024 * 8                                 # one 8-byte key per row
    assert call(sel(), ws_bytes=wsel - 1) == sda.SDA_EWORKSPACE
    assert L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SELECT_QGS, 0, 0, 0) == 0


def test_clustering_validation(L):
    """Host-side checks of the clustering entry point (nothing launches)."""
    dims = _dims()
    need = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_BUILD_QGC, 0, 0, 64)
    assert need >= 4 * 1024 * 16 * 4                           # 16 fixed-point coordinates per row
    assert L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_BUILD_QGC, 0, 0, 65) == 0

    def call(C=64, T=10, K=FAKE, V=FAKE, cid=FAKE, ws_bytes=1 << 30):
        return L.sda_build_qgc_clusters(ctypes.byref(dims), K, V, C, T, cid, None, FAKE, ws_bytes, None)

    assert call(C=0) == sda.SDA_EUNSUPPORTED
    assert call(C=65) == sda.SDA_EUNSUPPORTED
    assert call(T=0) == sda.SDA_EINVAL
    assert call(T=1001) == sda.SDA_EINVAL
    assert call(V=None) == sda.SDA_EINVAL
    assert call(cid=None) == sda.SDA_EINVAL
    assert call(K=MISALIGNED) == sda.SDA_EINVAL
    assert call(ws_bytes=need - 1) == sda.SDA_EWORKSPACE


def test_noalloc_entry_rejects_calls_beyond_its_scratch(L):
    """The allocation-free decode refuses, before touching the device, a call
    whose scratch would exceed the static array (sampled tail at batch 64,
    128K rows needs far more than 64 MiB of draw records)."""
    dims = sda.Dims(64, 256, 32, 131072, 128, sda.SDA_BF16, 0, 0, 0, 0.0)
    need = L.sda_workspace_bytes(ctypes.byref(dims), sda.OP_SPARSE, sda.TAIL_SAMPLED, 1000, 0)
    assert need > sda.NOALLOC_SCRATCH_BYTES
    t = sda.Tail()
    t.kind, t.eps, t.z, t.b0 = sda.TAIL_SAMPLED, 0.05, 1.96, 64
    rc = L.sda_sparse_decode_attn_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE2, None, None, 1000,
                                          ctypes.byref(t), FAKE, None, None, None)
    assert rc == sda.SDA_EWORKSPACE


def test_gather_rows_validation(L):
    """The gather measurement aid: bf16 rows only, supported shapes, aligned
    state whose size is a multiple of 16, rows per group within registers."""
    def call(dims, m=100, state=None, sbytes=0, waves=8, parts=1):
        return L.sda_gather_rows(ctypes.byref(dims), FAKE, FAKE2, FAKE, m, state, sbytes, waves, parts, FAKE2, None)
    assert call(_dims(dtype=sda.SDA_F32)) == sda.SDA_EUNSUPPORTED
    assert call(_dims(), waves=2) == sda.SDA_EUNSUPPORTED
    assert call(_dims(), parts=17) == sda.SDA_EUNSUPPORTED
    assert call(_dims(), m=8 * 4 * 25) == sda.SDA_EUNSUPPORTED        # 25 rows per row group at 8 waves
    assert call(_dims(), state=FAKE, sbytes=24) == sda.SDA_EINVAL      # not a multiple of 16
    assert call(_dims(), state=MISALIGNED, sbytes=32) == sda.SDA_EINVAL
    assert call(_dims(), m=-1) == sda.SDA_ESHAPE


def test_verified_budget_validation(L):
    """The verified sampled budget's host checks (nothing launches): a split
    count outside 0..SDA_MAX_Z_SPLITS, a missing table, eps >= 1 (the
    output's relative error), a table entry that is not a positive z."""
    dims = _dims()
    zs = (ctypes.c_double * 4)(2.2, 2.0, 2.0, 2.2)

    def call(nz, table, eps=0.05, z=0.0):
        t = sda.Tail()
        t.kind, t.eps, t.z, t.b0 = sda.TAIL_SAMPLED, eps, z, 64
        t.nz, t.z_split = nz, (ctypes.cast(table, ctypes.c_void_p) if table is not None else None)
        return _sparse(L, dims, tail=t, m=16)
    assert call(-1, zs) == sda.SDA_EINVAL
    assert call(65, zs) == sda.SDA_EINVAL
    assert call(2, None) == sda.SDA_EINVAL
    assert call(2, zs, eps=1.0) == sda.SDA_EINVAL
    bad = (ctypes.c_double * 4)(2.2, 0.0, 2.0, 2.2)
    assert call(2, bad) == sda.SDA_EINVAL
    nan = (ctypes.c_double * 4)(2.2, float("nan"), 2.0, 2.2)
    assert call(2, nan) == sda.SDA_EINVAL
    assert call(0, None, z=0.0) == sda.SDA_EINVAL  # the plain budget still needs z
