"""Selector oracle: QGS key codes and scores, ErrorGate budgets, per-cluster
top-q selection.  Plain numpy: fp64 where the method has real arithmetic,
exact integers where it scores codes.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does.  It
imports nothing from the product package and shares no code with it.

Source: "OpenAttention: One Percent Is Enough with Tail Proxies"
(ai-frontier-tracker summary), the four-stage method list -- stage 01 (the
cluster cache: a count, a mean token and a diagonal-variance token per
cluster), stage 02 (ErrorGate: the token budget E is split over the clusters
in proportion to each cluster's estimated weight error), stage 03 (QGS: keys
coded in int8 are scored in an r = 32 subspace and each cluster reads its q_b
best-scoring tokens) -- and the settings list (QGS rank r = 32; int8 per head
and coordinate; C = 64 clusters).

The page gives the stages, not their formulas.  Readings (the design notes
list them with the reasons):
  Q1  The subspace basis U [d, r] is an input with orthonormal columns (the
      page takes it from the query geometry: the leading eigenvectors of the
      queries' second moment).
  Q2  Projection y_j = U^T k_j, accumulated over the d key dimensions in
      order, in fp64.  Every product of a bf16 or fp32 key element and an
      fp32 basis entry is exact in fp64, so the only roundings are the
      in-order additions.
  Q3  Codes, one scale per (KV head, coordinate): kmax_i = max_j |y_ji| and
      code_ji = rint(127 * y_ji / kmax_i), rounding half to even (0 where
      kmax_i = 0).  Codes lie in [-127, 127].
  Q4  Query side: qt_h = U^T q_h (in order, fp64), w_hi = qt_hi * kmax_i (the
      code scale moved onto the query), one scale per KV group
      wmax = max_{h,i} |w_hi| and wq_hi = rint(127 * w_hi / wmax).  Score of
      row j: S_j = max over the group's heads of sum_i wq_hi * code_ji, an
      exact integer (|S_j| <= 32 * 127 * 127).  The page codes the keys in
      int8 and says nothing of the query; the plain reading keeps the query
      in fp64: S_j = max_h sum_i qt_hi * (kmax_i / 127) * code_ji
      (scores_plain, select_unit_plain).  Rounding the query too makes the
      scores exact integers, so the GPU's ranking is bit-exact; on the
      selector workload it moves 1-2.5% of the listed rows against the plain
      reading (the tests measure it).
  Q5  ErrorGate weight error.  Per head h and cluster b: mean logit
      zbar = scale <q_h, mu_b>, diagonal logit variance
      s2 = scale^2 sum_d q_hd^2 nu_bd, with mu_b = sumK_b / N_b and
      nu_bd = max(0, sumK2_bd / N_b - mu_bd^2).  With Gaussian member logits
      the members' total weight is N_b e^{zbar + s2/2} while the count-aware
      mean proxy gives N_b e^{zbar}, so the proxy's weight error is
      e_hb = N_b e^{zbar} (e^{s2/2} - 1).  Normalised by the head's estimated
      total weight Z_h = sum_b N_b e^{zbar + s2/2} and summed over the
      group's heads: eps_b = sum_h e_hb / Z_h.  Clusters with N_b = 0 have
      eps_b = 0.
  Q6  Budget: q_b proportional to eps_b by the largest-remainder rule (ties
      of the remainders go to the lower b), capped at the cluster's eligible
      rows A_b (members in [n_sink, n - n_local)); capped clusters are fixed
      and the rest is allocated again among the others.  Where every
      remaining eps is 0 the remaining capacity A_b is the weight.  In all,
      sum_b q_b = min(E, sum_b A_b).
  Q7  Selection: each cluster's q_b eligible members with the largest S
      (ties to the lower position).  The index set is the sink [0, n_sink),
      the local window [n - n_local, n) and the selected rows, ascending.
      Rows with cluster id -1 are never selected.
"""
from __future__ import annotations

import numpy as np

R_QGS = 32          # subspace rank (settings list)
CODE_MAX = 127      # int8 codes


def _f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32 values, widened exactly to fp64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def project(X, U) -> np.ndarray:
    """Q2: rows of X [N, d] projected on the columns of U [d, r]; the sum over
    d runs in index order (each product exact in fp64)."""
    X, U = _f64(X), np.asarray(U, dtype=np.float32).astype(np.float64)
    y = np.zeros((X.shape[0], U.shape[1]), np.float64)
    for dd in range(X.shape[1]):
        y += X[:, dd:dd + 1] * U[dd][None, :]
    return y


def _quantize(y, ymax) -> np.ndarray:
    """rint(127 * y / ymax) per column (0 where ymax == 0), half to even."""
    out = np.zeros(y.shape, np.int32)
    nz = ymax > 0
    out[..., nz] = np.rint((y[..., nz] * float(CODE_MAX)) / ymax[nz]).astype(np.int32)
    return out


def codes(K, U):
    """Q3: int8 codes [n, r] and the per-coordinate maxima kmax [r] of one
    unit's keys K [n, d]."""
    y = project(K, U)
    kmax = np.abs(y).max(axis=0) if y.shape[0] else np.zeros(y.shape[1])
    return _quantize(y, kmax).astype(np.int8), kmax


def query_weights(q, U, kmax) -> np.ndarray:
    """Q4: integer query weights wq [G, r] of one KV group (q [G, d])."""
    qt = project(q, U)
    w = qt * np.asarray(kmax, np.float64)[None, :]
    wmax = np.abs(w).max()
    if wmax == 0:
        return np.zeros(w.shape, np.int32)
    return np.rint((w * float(CODE_MAX)) / wmax).astype(np.int32)


def scores(code, wq) -> np.ndarray:
    """Q4: S_j = max_h sum_i wq_hi code_ji as exact int64."""
    dots = np.asarray(code, np.int64) @ np.asarray(wq, np.int64).T     # [n, G]
    return dots.max(axis=1)


def scores_plain(code, q, U, kmax) -> np.ndarray:
    """Q4, plain reading: S_j = max_h <U^T q_h, code_j * kmax / 127> in fp64
    (the key's coded projection against the unrounded query projection)."""
    qt = project(q, U)                                                  # [G, r]
    yhat = np.asarray(code, np.float64) * (np.asarray(kmax, np.float64) / float(CODE_MAX))[None, :]
    return (yhat @ qt.T).max(axis=1)


def cluster_stats(K, cid, C):
    """The cluster cache of one unit: N_b, sum of keys and sum of squared keys
    per cluster (fp64, exact inputs)."""
    Kf = _f64(K)
    cid = np.asarray(cid)
    N = np.zeros(C, np.int64)
    S1 = np.zeros((C, Kf.shape[1]))
    S2 = np.zeros((C, Kf.shape[1]))
    for b in range(C):
        m = cid == b
        N[b] = int(m.sum())
        S1[b] = Kf[m].sum(axis=0)
        S2[b] = (Kf[m] * Kf[m]).sum(axis=0)
    return N, S1, S2


def logit_moments(q, N, sumK, sumK2, scale):
    """Q5: mean logit zbar [C, G] and diagonal logit variance s2 [C, G] of each
    cluster's members (rows with N_b = 0 are nan)."""
    qf = _f64(q)
    N = np.asarray(N, np.int64)
    sumK, sumK2 = np.asarray(sumK, np.float64), np.asarray(sumK2, np.float64)
    sc = float(np.float32(scale))
    with np.errstate(invalid="ignore", divide="ignore"):
        Nf = N.astype(np.float64)[:, None]
        mu = sumK / Nf
        nu = np.maximum(sumK2 / Nf - mu * mu, 0.0)
    return sc * (mu @ qf.T), (sc * sc) * (nu @ (qf * qf).T)


def weight_errors(q, N, sumK, sumK2, scale) -> np.ndarray:
    """Q5: eps_b for one KV group; q [G, d] (bf16 bits or fp32), N [C],
    sumK / sumK2 [C, d]."""
    N = np.asarray(N, np.int64)
    sumK, sumK2 = np.asarray(sumK, np.float64), np.asarray(sumK2, np.float64)
    C = N.shape[0]
    eps = np.zeros(C)
    live = N > 0
    if not live.any():
        return eps
    zbar, s2 = logit_moments(q, N[live], sumK[live], sumK2[live], scale)   # [Cl, G]
    lnN = np.log(N[live].astype(np.float64))[:, None]
    top = lnN + zbar + 0.5 * s2                      # log of each cluster's estimated weight
    M = top.max(axis=0, keepdims=True)
    Z = np.exp(top - M).sum(axis=0, keepdims=True)
    e = np.exp(lnN + zbar - M) * np.expm1(0.5 * s2)
    eps[live] = (e / Z).sum(axis=1)
    return eps


def allocate(eps, avail, E):
    """Q6: integer budgets q [C] and the decision margin: the smallest
    distance, over every allocation round, of a quota from an integer or of
    the two remainders on either side of the cut (a margin near 0 means a
    last-bit change in eps could move one row between clusters)."""
    eps = np.asarray(eps, np.float64)
    avail = np.asarray(avail, np.int64)
    C = eps.shape[0]
    q = np.zeros(C, np.int64)
    fixed = avail <= 0
    R = int(min(int(E), int(avail.sum())))
    margin = np.inf
    while R > 0 and not fixed.all():
        act = np.flatnonzero(~fixed)
        w = eps[act]
        if not (w > 0).any():
            w = avail[act].astype(np.float64)
        tot = 0.0
        for v in w:
            tot += v
        quota = (float(R) * w) / tot
        base = np.floor(quota)
        frac = quota - base
        rem = R - int(base.sum())
        order = np.lexsort((act, -frac))            # largest remainder first, lower b on ties
        tent = base.astype(np.int64)
        tent[order[:rem]] += 1
        pos = frac[w > 0]
        if pos.size:
            margin = min(margin, float(np.minimum(pos, 1.0 - pos).min()))
        if 0 < rem < act.size:
            margin = min(margin, float(frac[order[rem - 1]] - frac[order[rem]]))
        over = tent > avail[act]
        if not over.any():
            q[act] = tent
            break
        cap = act[over]
        q[cap] = avail[cap]
        fixed[cap] = True
        R -= int(avail[cap].sum())
    return q, margin


def eligible(cid, n_sink, n_local):
    """Mask of rows the selector may pick: cluster id >= 0 and position in
    [n_sink, n - n_local)."""
    cid = np.asarray(cid)
    n = cid.shape[0]
    pos = np.arange(n)
    return (cid >= 0) & (pos >= n_sink) & (pos < n - n_local)


def select(S, cid, qb, n_sink, n_local):
    """Q7: the index set (ascending int32) of one unit."""
    cid = np.asarray(cid)
    n = cid.shape[0]
    el = eligible(cid, n_sink, n_local)
    pos = np.arange(n)
    picked = []
    for b in range(len(qb)):
        k = int(qb[b])
        if k <= 0:
            continue
        mem = pos[el & (cid == b)]
        order = np.lexsort((mem, -np.asarray(S)[mem]))   # score descending, then position
        picked.append(mem[order[:k]])
    base = np.concatenate([np.arange(0, min(n_sink, n)), np.arange(max(0, n - n_local), n)])
    out = np.unique(np.concatenate([base] + picked)) if picked else np.unique(base)
    return out.astype(np.int32)


def select_unit(q, K, cid, C, U, n_sink, n_local, E, scale, stats=None):
    """The whole selector for one unit: codes, scores, ErrorGate, budgets,
    selection.  Returns a dict with idx, budget, eps, margin, scores, codes,
    kmax and wq."""
    code, kmax = codes(K, U)
    wq = query_weights(q, U, kmax)
    S = scores(code, wq)
    N, S1, S2 = cluster_stats(K, cid, C) if stats is None else stats
    eps = weight_errors(q, N, S1, S2, scale)
    el = eligible(cid, n_sink, n_local)
    avail = np.array([int((el & (np.asarray(cid) == b)).sum()) for b in range(C)], np.int64)
    qb, margin = allocate(eps, avail, E)
    idx = select(S, cid, qb, n_sink, n_local)
    return dict(idx=idx, budget=qb, eps=eps, margin=margin, scores=S, codes=code, kmax=kmax, wq=wq, avail=avail)


def select_unit_plain(q, K, cid, C, U, n_sink, n_local, E, scale, stats=None):
    """The selector for one unit with the plain scores (query unrounded);
    budgets as in select_unit."""
    code, kmax = codes(K, U)
    S = scores_plain(code, q, U, kmax)
    N, S1, S2 = cluster_stats(K, cid, C) if stats is None else stats
    eps = weight_errors(q, N, S1, S2, scale)
    el = eligible(cid, n_sink, n_local)
    avail = np.array([int((el & (np.asarray(cid) == b)).sum()) for b in range(C)], np.int64)
    qb, margin = allocate(eps, avail, E)
    idx = select(S, cid, qb, n_sink, n_local)
    return dict(idx=idx, budget=qb, eps=eps, margin=margin, scores=S)
