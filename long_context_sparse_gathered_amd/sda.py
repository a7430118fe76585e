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
            "sda_sparse_decode_attn_noalloc", "sda_gather_rows", "sda_status_str", "sda_version"]


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
                ("samples_out", _vp), ("nz", ctypes.c_int32), ("z_split", _vp)]


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
    L.sda_sparse_decode_attn_noalloc.restype = i32
    L.sda_sparse_decode_attn_noalloc.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, i32, T, _vp, _vp, _vp, _vp]
    L.sda_dense_decode_attn.restype = i32
    L.sda_dense_decode_attn.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    L.sda_gather_rows.restype = i32
    L.sda_gather_rows.argtypes = [D, _vp, _vp, _vp, i32, _vp, ctypes.c_int64, i32, i32, _vp, _vp]
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


# ---------------------------------------------------------------------------
# argument checks: everything the kernels assume about a tensor (element type,
# shape, strides, device) is checked here, before the library is called, so a
# mismatch raises instead of reading or writing past a caller's buffer

def _need(t, name: str, dtype=None, shape=None, contiguous: bool = True, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _opt(t, name: str, **kw):
    return None if t is None else _need(t, name, **kw)


def _check_kv(K: torch.Tensor, V: torch.Tensor):
    """K and V: [B, Hkv, n, d] views with the same shape, strides, element
    type and device; unit stride along d."""
    _need(K, "K", contiguous=False)
    _need(V, "V", contiguous=False)
    if K.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"K must be bfloat16 or float32, got {K.dtype}")
    if K.dim() != 4 or K.stride(-1) != 1:
        raise ValueError("K must be a [B, Hkv, n, d] view with unit stride along d")
    if V.dtype != K.dtype:
        raise TypeError(f"V must have K's element type {K.dtype}, got {V.dtype}")
    if tuple(V.shape) != tuple(K.shape):
        raise ValueError(f"V must have K's shape {tuple(K.shape)}, got {tuple(V.shape)}")
    if tuple(V.stride()) != tuple(K.stride()):
        raise ValueError(f"V must have K's strides {tuple(K.stride())}, got {tuple(V.stride())}")
    if V.device != K.device:
        raise ValueError(f"V is on {V.device}, K on {K.device}")


def _check_q(q: torch.Tensor, K: torch.Tensor, dtype=None) -> int:
    """q: contiguous [B, Hq, d] in K's element type (or `dtype`), Hq a
    multiple of Hkv; returns Hq."""
    B, Hkv, _, d = K.shape
    _need(q, "q", dtype=K.dtype if dtype is None else dtype, device=K.device)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != d or q.shape[1] % Hkv != 0:
        raise ValueError(f"q must be [B={B}, Hq (a multiple of {Hkv}), d={d}], got {tuple(q.shape)}")
    return q.shape[1]


def _on_gpu(t: torch.Tensor, name: str):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")


def _check_ws(ws, device):
    if ws is not None:
        _need(ws, "ws", dtype=torch.uint8, device=device)


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

    verified: bool = False                   # eps, delta bound the output (verified budget)
    splits: int = 32                         # delta split into d_N = k delta / splits, k = 1 .. splits-1

    @property
    def z(self) -> float:
        return NormalDist().inv_cdf(1.0 - self.delta / 2.0)

    @property
    def z_split(self):
        """(Phi^-1(1 - d_N/2), Phi^-1(1 - d_D/2)) per split of delta."""
        nd = NormalDist()
        fr = [k / self.splits for k in range(1, self.splits)]
        return [(nd.inv_cdf(1.0 - f * self.delta / 2.0), nd.inv_cdf(1.0 - (1.0 - f) * self.delta / 2.0)) for f in fr]


def _tail_struct(tail, idx_cluster, cluster_id, lam, keep, B, Hq, Hkv, n, d, m, device) -> Tail:
    """The tail block, after checking every tensor it points at against the
    step's shapes."""
    t = Tail()
    if tail is None:
        t.kind = TAIL_NONE
    elif isinstance(tail, ProxyState):
        C = int(tail.C)
        t.kind = TAIL_PROXY
        t.C = C
        t.idx_cluster = _ptr(_opt(idx_cluster, "idx_cluster", dtype=torch.int32, shape=(B, Hkv, m), device=device))
        t.cluster_id = _ptr(_opt(cluster_id, "cluster_id", dtype=torch.int32, shape=(B, Hkv, n), device=device))
        t.count = _ptr(_need(tail.count, "count", dtype=torch.int32, shape=(B, Hkv, C), device=device))
        t.sumK = _ptr(_need(tail.sumK, "sumK", dtype=torch.float32, shape=(B, Hkv, C, d), device=device))
        t.sumV = _ptr(_need(tail.sumV, "sumV", dtype=torch.float32, shape=(B, Hkv, C, d), device=device))
    elif isinstance(tail, PriorState):
        t.kind = TAIL_PRIOR
        shapes = {"mu_Q": (B, Hq, d), "mu_K": (B, Hkv, d), "O_est": (B, Hq, d), "maxP": (B, Hq), "sumP": (B, Hq)}
        for name, shp in shapes.items():
            setattr(t, name, _ptr(_need(getattr(tail, name), name, dtype=torch.float32, shape=shp, device=device)))
        t.lam = float(lam)
        t.prior_n = int(tail.n_covered)
    elif isinstance(tail, SampledTail):
        t.kind = TAIL_SAMPLED
        _need(tail.b, "b", dtype=torch.int32, shape=(B, Hkv), device=device)
        _need(tail.bstar, "bstar", dtype=torch.float64, shape=(B, Hkv), device=device)
        if tail.b_cap < 0:
            raise ValueError("b_cap must be >= 0")
        _opt(tail.samples, "samples", dtype=torch.int32, shape=(B, Hkv, tail.b_cap), device=device)
        t.eps, t.z, t.b0, t.seed, t.b_cap = tail.eps, tail.z, tail.b0, tail.seed & (2**64 - 1), tail.b_cap
        t.b_out, t.bstar_out, t.samples_out = _ptr(tail.b), _ptr(tail.bstar), _ptr(tail.samples)
        if tail.verified:
            zs = [v for pair in tail.z_split for v in pair]
            buf = (ctypes.c_double * len(zs))(*zs)
            keep.append(buf)  # host table, read during the call
            t.nz, t.z_split = len(zs) // 2, ctypes.cast(buf, _vp)
    else:
        raise TypeError("tail must be None, ProxyState, PriorState or SampledTail")
    keep.append(t)
    return t


def _outputs(out, lse, B, Hq, d, device):
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=device) if out is None else \
        _need(out, "out", dtype=torch.float32, shape=(B, Hq, d), device=device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=device) if lse is None else \
        _need(lse, "lse", dtype=torch.float32, shape=(B, Hq), device=device)
    return out, lse


# ---------------------------------------------------------------------------
# entry points

def build_tail_proxies(K: torch.Tensor, V: torch.Tensor, cluster_id: torch.Tensor, C: int,
                       flags: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None, with_sumK2: bool = False) -> ProxyState:
    _check_kv(K, V)
    B, Hkv, n, d = K.shape
    dev = K.device
    _need(cluster_id, "cluster_id", dtype=torch.int32, shape=(B, Hkv, n), device=dev)
    _opt(flags, "flags", dtype=torch.int32, shape=(B, Hkv), device=dev)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
    count = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev)
    sumK = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev)
    sumV = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev)
    sumK2 = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=dev) if with_sumK2 else None
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_PROXIES, C=C), dev, ws)
    rc = lib().sda_build_tail_proxies(ctypes.byref(dims), _ptr(K), _ptr(V), _ptr(cluster_id), int(C),
                                      _ptr(count), _ptr(sumK), _ptr(sumV), _ptr(sumK2), _ptr(flags), _ptr(ws),
                                      wsb, _stream(stream))
    _check(rc, "sda_build_tail_proxies")
    return ProxyState(C=C, count=count, sumK=sumK, sumV=sumV, sumK2=sumK2)


def build_prior(K: torch.Tensor, V: torch.Tensor, mu_Q: torch.Tensor, scale: Optional[float] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> PriorState:
    _check_kv(K, V)
    B, Hkv, n, d = K.shape
    dev = K.device
    Hq = _check_q(mu_Q, K, dtype=torch.float32)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, Hq, scale)
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
    _check_kv(K, V)
    Hq = _check_q(q, K)
    B, _, _, d = K.shape
    dev = K.device
    out, lse = _outputs(out, lse, B, Hq, d, dev)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, Hq, scale)
    ws, wsb = _workspace(workspace_bytes(dims, OP_DENSE), dev, ws)
    rc = lib().sda_dense_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse),
                                     _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_dense_decode_attn")
    return out, lse


def _decode_args(q, K, V, idx, idx_len, logw, tail, idx_cluster, cluster_id, lam, out, lse, flags, m):
    """Checks shared by the decode entry points; returns (m, tail block, keep-alive list, out, lse)."""
    _check_kv(K, V)
    Hq = _check_q(q, K)
    B, Hkv, n, d = K.shape
    dev = K.device
    if idx is None:
        if m not in (None, 0):
            raise ValueError("m must be 0 when idx is None")
        m = 0
    else:
        _need(idx, "idx", dtype=torch.int32, device=dev)
        if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Hkv):
            raise ValueError(f"idx must be [B={B}, Hkv={Hkv}, m], got {tuple(idx.shape)}")
        if m is not None and m != idx.shape[-1]:
            raise ValueError(f"m = {m} does not match idx's last dimension {idx.shape[-1]}")
        m = idx.shape[-1]
    _opt(idx_len, "idx_len", dtype=torch.int32, shape=(B, Hkv), device=dev)
    _opt(logw, "logw", dtype=torch.float32, shape=(B, Hkv, m), device=dev)
    _opt(flags, "flags", dtype=torch.int32, shape=(B, Hkv), device=dev)
    keep = []
    t = _tail_struct(tail, idx_cluster, cluster_id, lam, keep, B, Hq, Hkv, n, d, m, dev)
    out, lse = _outputs(out, lse, B, Hq, d, dev)
    return m, t, keep, out, lse


def sparse_decode_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: Optional[torch.Tensor],
                       idx_len: Optional[torch.Tensor] = None, logw: Optional[torch.Tensor] = None,
                       tail=None, idx_cluster: Optional[torch.Tensor] = None,
                       cluster_id: Optional[torch.Tensor] = None, lam: float = 1.0,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, flags: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, m: Optional[int] = None, stream=None):
    """One decode step; returns (out [B,Hq,d] fp32, lse [B,Hq] fp32).
    idx is [B, Hkv, m] (m = idx.shape[-1]; `m`, if given, must agree), or None
    for an empty list."""
    if isinstance(tail, SampledTail):
        B, Hkv = K.shape[0], K.shape[1]
        if tail.b is None:
            tail.b = torch.empty((B, Hkv), dtype=torch.int32, device=K.device)
        if tail.bstar is None:
            tail.bstar = torch.empty((B, Hkv), dtype=torch.float64, device=K.device)
        if tail.samples is None and tail.b_cap > 0:
            tail.samples = torch.full((B, Hkv, tail.b_cap), -1, dtype=torch.int32, device=K.device)
    m, t, keep, out, lse = _decode_args(q, K, V, idx, idx_len, logw, tail, idx_cluster, cluster_id, lam, out, lse,
                                        flags, m)
    _check_ws(ws, K.device)
    _on_gpu(K, "K")
    dims = make_dims(K, q.shape[1], scale)
    ws, wsb = _workspace(workspace_bytes(dims, OP_SPARSE, t.kind, m, getattr(tail, "C", 0)), K.device, ws)
    rc = lib().sda_sparse_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(idx),
                                      _ptr(idx_len), _ptr(logw), int(m), ctypes.byref(t),
                                      _ptr(out), _ptr(lse), _ptr(flags), _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_sparse_decode_attn")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def sparse_decode_attn_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: Optional[torch.Tensor],
                               out: torch.Tensor, lse: torch.Tensor, idx_len: Optional[torch.Tensor] = None,
                               logw: Optional[torch.Tensor] = None, tail=None,
                               idx_cluster: Optional[torch.Tensor] = None, cluster_id: Optional[torch.Tensor] = None,
                               lam: float = 1.0, scale: Optional[float] = None, flags: Optional[torch.Tensor] = None,
                               m: Optional[int] = None, stream=None):
    """The decode step through the entry point that allocates nothing (its
    scratch is the library's per-GPU static array).  Every output, including
    a sampled tail's b and bstar, must be given; nothing is allocated here."""
    if out is None or lse is None:
        raise ValueError("out and lse must be given (this entry point allocates nothing)")
    if isinstance(tail, SampledTail) and (tail.b is None or tail.bstar is None):
        raise ValueError("a sampled tail's b and bstar must be given (this entry point allocates nothing)")
    m, t, keep, out, lse = _decode_args(q, K, V, idx, idx_len, logw, tail, idx_cluster, cluster_id, lam, out, lse,
                                        flags, m)
    _on_gpu(K, "K")
    dims = make_dims(K, q.shape[1], scale)
    rc = lib().sda_sparse_decode_attn_noalloc(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(idx),
                                              _ptr(idx_len), _ptr(logw), int(m), ctypes.byref(t), _ptr(out),
                                              _ptr(lse), _ptr(flags), _stream(stream))
    _check(rc, "sda_sparse_decode_attn_noalloc")
    return out, lse


@dataclass
class QgsCodes:
    """Selector key codes from build_qgs_codes."""
    U: torch.Tensor         # [B,Hkv,d,32] fp32 basis the codes were built with
    codes: torch.Tensor     # [B,Hkv,n,32] int8
    kmax: torch.Tensor      # [B,Hkv,32] fp64


def build_qgs_codes(K: torch.Tensor, U: torch.Tensor, ws: Optional[torch.Tensor] = None,
                    stream=None) -> QgsCodes:
    _need(K, "K", contiguous=False)
    if K.dim() != 4:
        raise ValueError("K must be a [B, Hkv, n, d] view")
    B, Hkv, n, d = K.shape
    dev = K.device
    _need(U, "U", dtype=torch.float32, shape=(B, Hkv, d, QGS_RANK), device=dev)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
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
    _need(K, "K", contiguous=False)
    if K.dim() != 4:
        raise ValueError("K must be a [B, Hkv, n, d] view")
    Hq = _check_q(q, K)
    B, Hkv, n, d = K.shape
    dev = K.device
    C = int(proxies.C)
    if proxies.sumK2 is None:
        raise ValueError("the selector needs the proxies built with with_sumK2=True")
    _need(cluster_id, "cluster_id", dtype=torch.int32, shape=(B, Hkv, n), device=dev)
    _need(proxies.count, "count", dtype=torch.int32, shape=(B, Hkv, C), device=dev)
    for name in ("sumK", "sumK2"):
        _need(getattr(proxies, name), name, dtype=torch.float32, shape=(B, Hkv, C, d), device=dev)
    _need(qc.U, "U", dtype=torch.float32, shape=(B, Hkv, d, QGS_RANK), device=dev)
    _need(qc.codes, "codes", dtype=torch.int8, shape=(B, Hkv, n, QGS_RANK), device=dev)
    _need(qc.kmax, "kmax", dtype=torch.float64, shape=(B, Hkv, QGS_RANK), device=dev)
    if m is None:
        m = min(n, n_sink + n_local + E)
    if out is None:
        out = (torch.empty((B, Hkv, m), dtype=torch.int32, device=dev),
               torch.empty((B, Hkv), dtype=torch.int32, device=dev),
               torch.empty((B, Hkv, m), dtype=torch.int32, device=dev))
    idx, idx_len, idx_cluster = out
    _need(idx, "idx", dtype=torch.int32, shape=(B, Hkv, m), device=dev)
    _need(idx_len, "idx_len", dtype=torch.int32, shape=(B, Hkv), device=dev)
    _need(idx_cluster, "idx_cluster", dtype=torch.int32, shape=(B, Hkv, m), device=dev)
    _opt(budget, "budget", dtype=torch.int32, shape=(B, Hkv, C), device=dev)
    _opt(flags, "flags", dtype=torch.int32, shape=(B, Hkv), device=dev)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, Hq, scale)
    sel = Selector(int(n_sink), int(n_local), int(E), C, _ptr(cluster_id), _ptr(proxies.count), _ptr(proxies.sumK),
                   _ptr(proxies.sumK2), _ptr(qc.U), _ptr(qc.codes), _ptr(qc.kmax))
    ws, wsb = _workspace(workspace_bytes(dims, OP_SELECT_QGS, C=C), dev, ws)
    rc = lib().sda_select_qgs(ctypes.byref(dims), _ptr(q), ctypes.byref(sel), int(m), _ptr(idx), _ptr(idx_len),
                              _ptr(idx_cluster), _ptr(budget), _ptr(flags), _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_select_qgs")
    return idx, idx_len, idx_cluster


def build_qgc_clusters(K: torch.Tensor, V: torch.Tensor, C: int, T: int = 10,
                       flags: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Query-geometry clustering of the keys: cluster ids [B, Hkv, n] int32
    from the basis V [B, Hkv, d, 16] (k-means with T passes)."""
    _need(K, "K", contiguous=False)
    if K.dim() != 4:
        raise ValueError("K must be a [B, Hkv, n, d] view")
    B, Hkv, n, d = K.shape
    dev = K.device
    _need(V, "V", dtype=torch.float32, shape=(B, Hkv, d, QGC_RANK), device=dev)
    _opt(flags, "flags", dtype=torch.int32, shape=(B, Hkv), device=dev)
    _check_ws(ws, dev)
    _on_gpu(K, "K")
    dims = make_dims(K, 1)
    dims.Hq = dims.Hkv
    cid = torch.empty((B, Hkv, n), dtype=torch.int32, device=dev)
    ws, wsb = _workspace(workspace_bytes(dims, OP_BUILD_QGC, C=C), dev, ws)
    rc = lib().sda_build_qgc_clusters(ctypes.byref(dims), _ptr(K), _ptr(V), int(C), int(T), _ptr(cid), _ptr(flags),
                                      _ptr(ws), wsb, _stream(stream))
    _check(rc, "sda_build_qgc_clusters")
    return cid


def gather_rows(K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, waves: int = 8, parts: int = 1,
                state: Optional[torch.Tensor] = None, checksum: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Measurement aid: read the listed K/V rows (and each unit's slice of
    `state`, a [B*Hkv, ...] tensor) in the given launch shape; returns the
    per-wave XOR checksums [B*Hkv*parts*waves] (uint32 bits in an int32
    tensor)."""
    _check_kv(K, V)
    B, Hkv, n, d = K.shape
    dev = K.device
    _need(idx, "idx", dtype=torch.int32, device=dev)
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Hkv):
        raise ValueError(f"idx must be [B={B}, Hkv={Hkv}, m], got {tuple(idx.shape)}")
    state_bytes = 0
    if state is not None:
        _need(state, "state", device=dev)
        if state.shape[0] != B * Hkv:
            raise ValueError("state must be [B*Hkv, ...]")
        state_bytes = state[0].numel() * state.element_size()
    words = B * Hkv * int(parts) * int(waves)
    if checksum is None:
        checksum = torch.zeros(words, dtype=torch.int32, device=dev)
    else:
        _need(checksum, "checksum", dtype=torch.int32, shape=(words,), device=dev)
    _on_gpu(K, "K")
    dims = make_dims(K, Hkv)
    rc = lib().sda_gather_rows(ctypes.byref(dims), _ptr(K), _ptr(V), _ptr(idx), int(idx.shape[-1]), _ptr(state),
                               int(state_bytes), int(waves), int(parts), _ptr(checksum), _stream(stream))
    _check(rc, "sda_gather_rows")
    return checksum


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
