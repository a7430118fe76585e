"""Thin ctypes binding of libsda (``include/sda.h``).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch provides device memory and the current stream.  If the
library is not built, the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from statistics import NormalDist
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsda.so")

# status codes / enums (mirror sda.h)
SDA_OK, SDA_EINVAL, SDA_ESHAPE, SDA_EDTYPE, SDA_EWORKSPACE, SDA_EUNSUPPORTED, SDA_EHIP = 0, -1, -2, -3, -4, -5, -6
SDA_BF16, SDA_F32 = 0, 1
TAIL_NONE, TAIL_PROXY, TAIL_PRIOR, TAIL_SAMPLED = 0, 1, 2, 3
OP_SPARSE, OP_DENSE, OP_BUILD_PROXIES, OP_BUILD_PRIOR, OP_BUILD_QGS, OP_SELECT_QGS, OP_BUILD_QGC = 0, 1, 2, 3, 4, 5, 6
QGS_RANK = 32
QGC_RANK = 16
FLAG_IDX_RANGE, FLAG_IDX_ORDER, FLAG_SAMPLE_CAP, FLAG_CLUSTER, FLAG_LEN = 1, 2, 4, 8, 16

EXPORTED = ["sda_workspace_bytes", "sda_build_tail_proxies", "sda_build_prior", "sda_sparse_decode_attn",
            "sda_dense_decode_attn", "sda_build_qgs_codes", "sda_select_qgs", "sda_build_qgc_clusters",
            "sda_status_str", "sda_version"]


class SdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("n", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
                ("kv_stride_n", ctypes.c_int64), ("scale", ctypes.c_float)]


_vp = ctypes.c_void_p


class Tail(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32),
                ("C", ctypes.c_int32), ("idx_cluster", _vp), ("cluster_id", _vp), ("count", _vp),
                ("sumK", _vp), ("sumV", _vp),
                ("mu_Q", _vp), ("mu_K", _vp), ("O_est", _vp), ("maxP", _vp), ("sumP", _vp),
                ("lam", ctypes.c_float), ("prior_n", ctypes.c_int32),
                ("eps", ctypes.c_double), ("z", ctypes.c_double), ("b0", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("b_cap", ctypes.c_int32), ("b_out", _vp), ("bstar_out", _vp),
                ("samples_out", _vp)]


class Selector(ctypes.Structure):
    _fields_ = [("n_sink", ctypes.c_int32), ("n_local", ctypes.c_int32), ("E", ctypes.c_int32),
                ("C", ctypes.c_int32), ("cluster_id", _vp), ("count", _vp), ("sumK", _vp), ("sumK2", _vp),
                ("U", _vp), ("codes", _vp), ("kmax", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libsda.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                           "python -m long_context_sparse_gathered_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    D, T = ctypes.POINTER(Dims), ctypes.POINTER(Tail)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    L.sda_workspace_bytes.restype = sz
    L.sda_workspace_bytes.argtypes = [D, i32, i32, i32, i32]
    L.sda_build_tail_proxies.restype = i32
    L.sda_build_tail_proxies.argtypes = [D, _vp, _vp, _vp, i32, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_build_qgs_codes.restype = i32
    L.sda_build_qgs_codes.argtypes = [D, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_build_qgc_clusters.restype = i32
    L.sda_build_qgc_clusters.argtypes = [D, _vp, _vp, i32, i32, _vp, _vp, _vp, sz, _vp]
    L.sda_select_qgs.restype = i32
    L.sda_select_qgs.argtypes = [D, _vp, ctypes.POINTER(Selector), i32, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_build_prior.restype = i32
    L.sda_build_prior.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_sparse_decode_attn.restype = i32
    L.sda_sparse_decode_attn.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, i32, T, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_dense_decode_attn.restype = i32
    L.sda_dense_decode_attn.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_status_str.restype = ctypes.c_char_p
    L.sda_status_str.argtypes = [i32]
    L.sda_version.restype = ctypes.c_char_p
    L.sda_version.argtypes = []
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().sda_status_str(int(status)).decode()


def version() -> str:
    return lib().sda_version().decode()


# ---------------------------------------------------------------------------
# marshalling helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SDA_BF16
    if t.dtype == torch.float32:
        return SDA_F32
    raise TypeError(f"unsupported element type {t.dtype}")


def make_dims(K: torch.Tensor, Hq: int, scale: Optional[float] = None) -> Dims:
    """Dims from a [B, Hkv, n, d] K view (any strides with stride(-1) == 1)."""
    if K.dim() != 4 or K.stride(-1) != 1:
        raise ValueError("K must be a [B, Hkv, n, d] view with unit stride along d")
    B, Hkv, n, d = K.shape
    sb, sh, sn, _ = K.stride()
    return Dims(B, Hq, Hkv, n, d, _dtype_code(K), sb, sh, sn, 0.0 if scale is None else float(scale))


def _check(rc: int, where: str):
    if rc != SDA_OK:
        raise SdaError(rc, where)


def workspace_bytes(dims: Dims, op: int, tail_kind: int = TAIL_NONE, m: int = 0, C: int = 0) -> int:
    return int(lib().sda_workspace_bytes(ctypes.byref(dims), op, tail_kind, m, C))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws, 0
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _i32(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError("index-like tensors must be contiguous int32")
    return t


def _f32c(t: Optional[torch.Tensor], name: str) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    return t


# ---------------------------------------------------------------------------
# tails

@dataclass
class ProxyState:
    """Per-cluster state from build_tail_proxies."""
    C: int
    count: torch.Tensor     # [B,Hkv,C] int32
    sumK: torch.Tensor      # [B,Hkv,C,d] fp32
    sumV: torch.Tensor      # [B,Hkv,C,d] fp32
    sumK2: Optional[torch.Tensor] = None   # [B,Hkv,C,d] fp32 sums of squared keys (selector)


@dataclass
class PriorState:
    """Rank-1 prior state from build_prior (plus the mean query it came from).
    n_covered: the cache rows it was built over; a decode over a cache that
    has grown since treats the later rows as exact-only."""
    mu_Q: torch.Tensor      # [B,Hq,d] fp32
    mu_K: torch.Tensor      # [B,Hkv,d]
    O_est: torch.Tensor     # [B,Hq,d]
    maxP: torch.Tensor      # [B,Hq]
    sumP: torch.Tensor      # [B,Hq]
    n_covered: int = 0


@dataclass
class SampledTail:
    """Parameters of the sampled tail; outputs are filled by the call."""
    eps: float = 0.05
    delta: float = 0.05
    b0: int = 64
    seed: int = 0
    b_cap: int = 0
    b: Optional[torch.Tensor] = None         # [B,Hkv] int32 (output)
    bstar: Optional[torch.Tensor] = None     # [B,Hkv] float64 (output)
    samples: Optional[torch.Tensor] = None   # [B,Hkv,b_cap] int32 (output)

    @property
    def z(self) -> float:
        return NormalDist().inv_cdf(1.0 - self.delta / 2.0)


def _tail_struct(tail, idx_cluster, cluster_id, lam, keep) -> Tail:
    t = Tail()
    if tail is None:
        t.kind = TAIL_NONE
    elif isinstance(tail, ProxyState):
        t.kind = TAIL_PROXY
        t.C = tail.C
        t.idx_cluster = _ptr(_i32(idx_cluster))
        t.cluster_id = _ptr(_i32(cluster_id))
        t.count = _ptr(_i32(tail.count))
        t.sumK = _ptr(_f32c(tail.sumK, "sumK"))
        t.sumV = _ptr(_f32c(tail.sumV, "sumV"))
    elif isinstance(tail, PriorState):
        t.kind = TAIL_PRIOR
        for name in ("mu_Q", "mu_K", "O_est", "maxP", "sumP"):
            setattr(t, name, _ptr(_f32c(getattr(tail, name), name)))
        t.lam = float(lam)
        t.prior_n = int(tail.n_covered)
    elif isinstance(tail, SampledTail):
        t.kind = TAIL_SAMPLED
        t.eps, t.z, t.b0, t.seed, t.b_cap = tail.eps, tail.z, tail.b0, tail.seed & (2**64 - 1), tail.b_cap
        t.b_out, t.bstar_out, t.samples_out = _ptr(tail.b), _ptr(tail.bstar), _ptr(tail.samples)
    else:
        raise TypeError("tail must be None, ProxyState, PriorState or SampledTail")
    keep.append(t)
    return t


# ---------------------------------------------------------------------------
# entry points

def build_tail_proxies(K: torch.Tensor, V: torch.Tensor, cluster_id: torch.Tensor, C: int,
                       flags: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None, with_sumK2: bool = False) -> ProxyState:
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
    B, Hkv, n, d = K.shape
    dev = K.device
    count = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev)
    sumK = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev)
    sumV = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev)
    sumK2 = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev) if with_sumK2 else None
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_PROXIES, C=C), dev, ws)
    rc = lib().sda_build_tail_proxies(ctypes.byref(dims), _ptr(K), _ptr(V), _ptr(_i32(cluster_id)), int(C),
                                      _ptr(count), _ptr(sumK), _ptr(sumV), _ptr(sumK2), _ptr(flags), _ptr(ws),
                                      wsb, _stream(stream))
    _check(rc, "sda_build_tail_proxies")
    return ProxyState(C=C, count=count, sumK=sumK, sumV=sumV, sumK2=sumK2)


def build_prior(K: torch.Tensor, V: torch.Tensor, mu_Q: torch.Tensor, scale: Optional[float] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> PriorState:
    Hq = mu_Q.shape[1]
    dims = make_dims(K, Hq, scale)
    B, Hkv, n, d = K.shape
    dev = K.device
    mu_Q = _f32c(mu_Q, "mu_Q")
    mu_K = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
    O_est = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    maxP = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    sumP = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_PRIOR), dev, ws)
    rc = lib().sda_build_prior(ctypes.byref(dims), _ptr(K), _ptr(V), _ptr(mu_Q), _ptr(mu_K), _ptr(O_est),
                               _ptr(maxP), _ptr(sumP), _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_build_prior")
    return PriorState(mu_Q=mu_Q, mu_K=mu_K, O_est=O_est, maxP=maxP, sumP=sumP, n_covered=n)


def dense_decode_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    B, Hq, d = q.shape
    dims = make_dims(K, Hq, scale)
    dev = q.device
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws, wsb = _workspace(workspace_bytes(dims, OP_DENSE), dev, ws)
    rc = lib().sda_dense_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse),
                                     _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_dense_decode_attn")
    return out, lse


def sparse_decode_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: Optional[torch.Tensor],
                       idx_len: Optional[torch.Tensor] = None, logw: Optional[torch.Tensor] = None,
                       tail=None, idx_cluster: Optional[torch.Tensor] = None,
                       cluster_id: Optional[torch.Tensor] = None, lam: float = 1.0,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, flags: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, m: Optional[int] = None, stream=None):
    """One decode step; returns (out [B,Hq,d] fp32, lse [B,Hq] fp32)."""
    B, Hq, d = q.shape
    dims = make_dims(K, Hq, scale)
    dev = q.device
    if m is None:
        m = 0 if idx is None else idx.shape[-1]
    if isinstance(tail, SampledTail):
        Hkv = K.shape[1]
        if tail.b is None:
            tail.b = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        if tail.bstar is None:
            tail.bstar = torch.empty((B, Hkv), dtype=torch.float64, device=dev)
        if tail.samples is None and tail.b_cap > 0:
            tail.samples = torch.full((B, Hkv, tail.b_cap), -1, dtype=torch.int32, device=dev)
    keep = []
    t = _tail_struct(tail, idx_cluster, cluster_id, lam, keep)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws, wsb = _workspace(workspace_bytes(dims, OP_SPARSE, t.kind, m, getattr(tail, "C", 0)), dev, ws)
    rc = lib().sda_sparse_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(_i32(idx)),
                                      _ptr(_i32(idx_len)), _ptr(_f32c(logw, "logw")), int(m), ctypes.byref(t),
                                      _ptr(out), _ptr(lse), _ptr(flags), _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_sparse_decode_attn")
    return out, lse


@dataclass
class QgsCodes:
    """Selector key codes from build_qgs_codes."""
    U: torch.Tensor         # [B,Hkv,d,32] fp32 basis the codes were built with
    codes: torch.Tensor     # [B,Hkv,n,32] int8
    kmax: torch.Tensor      # [B,Hkv,32] fp64


def build_qgs_codes(K: torch.Tensor, U: torch.Tensor, ws: Optional[torch.Tensor] = None,
                    stream=None) -> QgsCodes:
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
    B, Hkv, n, d = K.shape
    dev = K.device
    U = _f32c(U, "U")
    if tuple(U.shape) != (B, Hkv, d, QGS_RANK):
        raise ValueError(f"U must be [B, Hkv, d, {QGS_RANK}]")
    codes = torch.empty((B, Hkv, n, QGS_RANK), dtype=torch.int8, device=dev)
    kmax = torch.empty((B, Hkv, QGS_RANK), dtype=torch.float64, device=dev)
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_QGS), dev, ws)
    rc = lib().sda_build_qgs_codes(ctypes.byref(dims), _ptr(K), _ptr(U), _ptr(codes), _ptr(kmax), _ptr(ws), wsb,
                                   _stream(stream))
    _check(rc, "sda_build_qgs_codes")
    return QgsCodes(U=U, codes=codes, kmax=kmax)


def select_qgs(q: torch.Tensor, K: torch.Tensor, cluster_id: torch.Tensor, proxies: ProxyState, qc: QgsCodes,
               n_sink: int, n_local: int, E: int, m: Optional[int] = None, scale: Optional[float] = None,
               out: Optional[tuple] = None, budget: Optional[torch.Tensor] = None,
               flags: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """The selector: returns (idx [B,Hkv,m], idx_len [B,Hkv], idx_cluster [B,Hkv,m]); fills budget
    [B,Hkv,C] when given.  K only supplies the cache's shape and strides."""
    B, Hq, d = q.shape
    dims = make_dims(K, Hq, scale)
    n, Hkv = K.shape[2], K.shape[1]
    dev = q.device
    if proxies.sumK2 is None:
        raise ValueError("the selector needs the proxies built with with_sumK2=True")
    if m is None:
        m = min(n, n_sink + n_local + E)
    if out is None:
        out = (torch.empty((B, Hkv, m), dtype=torch.int32, device=dev),
               torch.empty((B, Hkv), dtype=torch.int32, device=dev),
               torch.empty((B, Hkv, m), dtype=torch.int32, device=dev))
    idx, idx_len, idx_cluster = out
    sel = Selector(int(n_sink), int(n_local), int(E), int(proxies.C), _ptr(_i32(cluster_id)),
                   _ptr(_i32(proxies.count)), _ptr(_f32c(proxies.sumK, "sumK")),
                   _ptr(_f32c(proxies.sumK2, "sumK2")), _ptr(_f32c(qc.U, "U")), _ptr(qc.codes), _ptr(qc.kmax))
    ws, wsb = _workspace(workspace_bytes(dims, OP_SELECT_QGS, C=proxies.C), dev, ws)
    rc = lib().sda_select_qgs(ctypes.byref(dims), _ptr(q), ctypes.byref(sel), int(m), _ptr(idx), _ptr(idx_len),
                              _ptr(idx_cluster), _ptr(budget), _ptr(flags), _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_select_qgs")
    return idx, idx_len, idx_cluster


def build_qgc_clusters(K: torch.Tensor, V: torch.Tensor, C: int, T: int = 10,
                       flags: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Query-geometry clustering of the keys: cluster ids [B, Hkv, n] int32
    from the basis V [B, Hkv, d, 16] (k-means with T passes)."""
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
    B, Hkv, n, d = K.shape
    V = _f32c(V, "V")
    if tuple(V.shape) != (B, Hkv, d, QGC_RANK):
        raise ValueError(f"V must be [B, Hkv, d, {QGC_RANK}]")
    cid = torch.empty((B, Hkv, n), dtype=torch.int32, device=K.device)
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_QGC, C=C), K.device, ws)
    rc = lib().sda_build_qgc_clusters(ctypes.byref(dims), _ptr(K), _ptr(V), int(C), int(T), _ptr(cid), _ptr(flags),
                                      _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_build_qgc_clusters")
    return cid


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
