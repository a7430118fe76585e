"""Python access to the fp64 CPU oracle (``oracle_sda.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does.  It
imports nothing from the product package.

Arrays are numpy.  bf16 tensors are passed as ``uint16`` bit patterns, fp32
tensors as ``float32``; ``q`` must have the same element type as ``K``/``V``.
Every routine returns float64 results.  Shapes follow ``oracle_sda.h``:
q [B,Hq,d], K/V [B,Hkv,n,d], idx/logw [B,Hkv,m], out [B,Hq,d], lse [B,Hq].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_sda.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_sda.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, strict IEEE doubles)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("n", ctypes.c_int), ("d", ctypes.c_int), ("dtype", ctypes.c_int),
                ("scale", ctypes.c_float)]


_P = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    D = ctypes.POINTER(_Dims)
    i32, i64, u64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    sig = {
        "orc_dense": (i32, [D, _P, _P, _P, _P, _P]),
        "orc_sparse": (i32, [D, _P, _P, _P, _P, _P, _P, i32, _P, _P]),
        "orc_proxy_build": (i32, [D, _P, _P, _P, i32, _P, _P, _P]),
        "orc_sparse_proxy_def": (i32, [D, _P, _P, _P, _P, _P, _P, i32, _P, i32, _P, _P]),
        "orc_sparse_proxy": (i32, [D, _P, _P, _P, _P, _P, _P, i32, _P, i32, _P, _P, _P, _P, _P]),
        "orc_prior_build": (i32, [D, _P, _P, _P, _P, _P, _P, _P]),
        "orc_sparse_prior_def": (i32, [D, _P, _P, _P, _P, _P, _P, i32, _P, f64, i32, _P, _P]),
        "orc_sparse_prior": (i32, [D, _P, _P, _P, _P, _P, _P, i32, _P, f64, i32, _P, _P, _P, _P, _P, _P]),
        "orc_splitmix64_next": (u64, [ctypes.POINTER(ctypes.c_uint64)]),
        "orc_unit_key": (u64, [u64, i64]),
        "orc_draw_rank": (i64, [u64, i64, i64]),
        "orc_tail_pos": (i64, [_P, i32, i64]),
        "orc_budget_from_terms": (f64, [i32, i32, _P, _P, f64, _P, i64, f64, f64]),
        "orc_budget_verified_from_terms": (f64, [i32, i32, _P, _P, f64, _P, i64, f64, i32, _P]),
        "orc_sampled": (i32, [D, _P, _P, _P, _P, _P, i32, f64, f64, i32, u64, _P, _P, _P, i32, _P, _P]),
        "orc_sampled_verified": (i32, [D, _P, _P, _P, _P, _P, i32, f64, i32, _P, i32, u64, _P, _P, _P, i32, _P, _P]),
        "orc_sampled_fixed_b": (i32, [D, _P, _P, _P, _P, _P, i32, i32, i32, u64, _P, _P]),
        "orc_set_threads": (None, [i32]),
        "orc_get_threads": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ---------------------------------------------------------------------------

def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _dims(q, K, scale):
    if K.dtype == np.uint16:
        dt = 0
    elif K.dtype == np.float32:
        dt = 1
    else:
        raise TypeError("K must be uint16 (bf16 bits) or float32")
    if q.dtype != K.dtype:
        raise TypeError("q must have the same element type as K")
    B, Hkv, n, d = K.shape
    Hq = q.shape[1]
    if q.shape != (B, Hq, d):
        raise ValueError("q shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return _Dims(B, Hq, Hkv, n, d, dt, np.float32(scale))


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def _out(D):
    return (np.zeros((D.B, D.Hq, D.d), np.float64), np.zeros((D.B, D.Hq), np.float64))


def dense(q, K, V, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    _check(_load().orc_dense(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse)), "dense")
    return out, lse


def sparse(q, K, V, idx, idx_len=None, logw=None, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len, logw = _c(idx, np.int32), _c(idx_len, np.int32), _c(logw, np.float32)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    m = idx.shape[-1]
    _check(_load().orc_sparse(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                              _ptr(logw), m, _ptr(out), _ptr(lse)), "sparse")
    return out, lse


def proxy_build(K, V, cid, C, scale=None):
    K, V, cid = _c(K), _c(V), _c(cid, np.int32)
    B, Hkv, n, d = K.shape
    D = _dims(np.zeros((B, Hkv, d), K.dtype), K, scale)
    count = np.zeros((B, Hkv, C), np.int32)
    sumK = np.zeros((B, Hkv, C, d), np.float64)
    sumV = np.zeros((B, Hkv, C, d), np.float64)
    _check(_load().orc_proxy_build(ctypes.byref(D), _ptr(K), _ptr(V), _ptr(cid), C,
                                   _ptr(count), _ptr(sumK), _ptr(sumV)), "proxy_build")
    return count, sumK, sumV


def sparse_proxy_def(q, K, V, idx, cid, C, idx_len=None, logw=None, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len, logw, cid = _c(idx, np.int32), _c(idx_len, np.int32), _c(logw, np.float32), _c(cid, np.int32)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    _check(_load().orc_sparse_proxy_def(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                        _ptr(logw), idx.shape[-1], _ptr(cid), C, _ptr(out), _ptr(lse)),
           "sparse_proxy_def")
    return out, lse


def sparse_proxy(q, K, V, idx, cid, C, count, sumK, sumV, idx_len=None, logw=None, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len, logw, cid = _c(idx, np.int32), _c(idx_len, np.int32), _c(logw, np.float32), _c(cid, np.int32)
    count, sumK, sumV = _c(count, np.int32), _c(sumK, np.float64), _c(sumV, np.float64)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    _check(_load().orc_sparse_proxy(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                    _ptr(logw), idx.shape[-1], _ptr(cid), C, _ptr(count), _ptr(sumK),
                                    _ptr(sumV), _ptr(out), _ptr(lse)), "sparse_proxy")
    return out, lse


def prior_build(K, V, mu_Q, scale=None):
    K, V, mu_Q = _c(K), _c(V), _c(mu_Q, np.float32)
    B, Hkv, n, d = K.shape
    Hq = mu_Q.shape[1]
    D = _dims(np.zeros((B, Hq, d), K.dtype), K, scale)
    muK = np.zeros((B, Hkv, d), np.float64)
    Oest = np.zeros((B, Hq, d), np.float64)
    maxP = np.zeros((B, Hq), np.float64)
    sumP = np.zeros((B, Hq), np.float64)
    _check(_load().orc_prior_build(ctypes.byref(D), _ptr(K), _ptr(V), _ptr(mu_Q), _ptr(muK), _ptr(Oest),
                                   _ptr(maxP), _ptr(sumP)), "prior_build")
    return muK, Oest, maxP, sumP


def sparse_prior_def(q, K, V, idx, mu_Q, lam=1.0, idx_len=None, logw=None, scale=None, prior_n=0):
    """prior_n: rows [0, prior_n) covered by the prior (0 = all)."""
    q, K, V, mu_Q = _c(q), _c(K), _c(V), _c(mu_Q, np.float32)
    idx, idx_len, logw = _c(idx, np.int32), _c(idx_len, np.int32), _c(logw, np.float32)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    _check(_load().orc_sparse_prior_def(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                        _ptr(logw), idx.shape[-1], _ptr(mu_Q), float(lam), int(prior_n), _ptr(out),
                                        _ptr(lse)),
           "sparse_prior_def")
    return out, lse


def sparse_prior(q, K, V, idx, mu_Q, lam, muK, Oest, maxP, sumP, idx_len=None, logw=None, scale=None, prior_n=0):
    """prior_n: rows [0, prior_n) the state was built over (0 = all)."""
    q, K, V, mu_Q = _c(q), _c(K), _c(V), _c(mu_Q, np.float32)
    idx, idx_len, logw = _c(idx, np.int32), _c(idx_len, np.int32), _c(logw, np.float32)
    muK, Oest, maxP, sumP = (_c(a, np.float64) for a in (muK, Oest, maxP, sumP))
    D = _dims(q, K, scale)
    out, lse = _out(D)
    _check(_load().orc_sparse_prior(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                    _ptr(logw), idx.shape[-1], _ptr(mu_Q), float(lam), int(prior_n), _ptr(muK),
                                    _ptr(Oest), _ptr(maxP), _ptr(sumP), _ptr(out), _ptr(lse)), "sparse_prior")
    return out, lse


# ---- sampled tail ----------------------------------------------------------

def splitmix64_stream(seed: int, count: int):
    st = ctypes.c_uint64(seed)
    f = _load().orc_splitmix64_next
    return [int(f(ctypes.byref(st))) for _ in range(count)]


def unit_key(seed: int, unit: int) -> int:
    return int(_load().orc_unit_key(seed, unit))


def draw_rank(key: int, k: int, n_s: int) -> int:
    return int(_load().orc_draw_rank(key, k, n_s))


def tail_pos(If, u: int) -> int:
    If = _c(If, np.int32)
    return int(_load().orc_tail_pos(_ptr(If), len(If), u))


def budget_from_terms(rD, rN, Df, Nf, n_s, eps, z):
    rD, rN, Nf = _c(rD, np.float64), _c(rN, np.float64), _c(Nf, np.float64)
    b0 = rD.shape[0]
    d = Nf.shape[0]
    assert rN.shape == (b0, d)
    return float(_load().orc_budget_from_terms(d, b0, _ptr(rD), _ptr(rN), float(Df), _ptr(Nf),
                                               int(n_s), float(eps), float(z)))


def budget_verified_from_terms(rD, rN, Df, Nf, n_s, eps, z_split):
    """The verified budget of one head: z_split is an (nz, 2) array of
    (Phi^-1(1 - d_N/2), Phi^-1(1 - d_D/2)) for splits d_N + d_D = delta."""
    rD, rN, Nf = _c(rD), _c(rN), _c(Nf)
    zs = _c(np.asarray(z_split, np.float64).reshape(-1, 2))
    b0, d = rN.shape
    return float(_load().orc_budget_verified_from_terms(d, b0, _ptr(rD), _ptr(rN), float(Df), _ptr(Nf),
                                                        int(n_s), float(eps), zs.shape[0], _ptr(zs)))


def sampled_verified(q, K, V, idx, eps, z_split, b0, seed, b_cap, idx_len=None, scale=None):
    """The sampled estimator with the verified budget (see
    budget_verified_from_terms); returns what sampled() returns."""
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len = _c(idx, np.int32), _c(idx_len, np.int32)
    zs = _c(np.asarray(z_split, np.float64).reshape(-1, 2))
    D = _dims(q, K, scale)
    out, lse = _out(D)
    b = np.zeros((D.B, D.Hkv), np.int32)
    bstar = np.zeros((D.B, D.Hkv), np.float64)
    samples = np.full((D.B, D.Hkv, max(b_cap, 1)), -1, np.int32)
    _check(_load().orc_sampled_verified(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                        idx.shape[-1], float(eps), zs.shape[0], _ptr(zs), int(b0), int(seed),
                                        _ptr(b), _ptr(bstar), _ptr(samples), int(b_cap), _ptr(out), _ptr(lse)),
           "sampled_verified")
    return {"b": b, "bstar": bstar, "samples": samples[..., :b_cap], "out": out, "lse": lse}


def sampled(q, K, V, idx, eps, z, b0, seed, b_cap, idx_len=None, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len = _c(idx, np.int32), _c(idx_len, np.int32)
    D = _dims(q, K, scale)
    out, lse = _out(D)
    U = D.B * D.Hkv
    b = np.zeros((D.B, D.Hkv), np.int32)
    bstar = np.zeros((D.B, D.Hkv), np.float64)
    samples = np.full((D.B, D.Hkv, max(b_cap, 1)), -1, np.int32)
    _check(_load().orc_sampled(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                               idx.shape[-1], float(eps), float(z), int(b0), int(seed), _ptr(b), _ptr(bstar),
                               _ptr(samples), int(b_cap), _ptr(out), _ptr(lse)), "sampled")
    del U
    return {"b": b, "bstar": bstar, "samples": samples[..., :b_cap], "out": out, "lse": lse}


def sampled_fixed_b(q, K, V, idx, b0, b, seed, idx_len=None, scale=None):
    q, K, V = _c(q), _c(K), _c(V)
    idx, idx_len = _c(idx, np.int32), _c(idx_len, np.int32)
    D = _dims(q, K, scale)
    Nhat, Dhat = _out(D)
    _check(_load().orc_sampled_fixed_b(ctypes.byref(D), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(idx_len),
                                       idx.shape[-1], int(b0), int(b), int(seed), _ptr(Dhat), _ptr(Nhat)),
           "sampled_fixed_b")
    return Dhat, Nhat
