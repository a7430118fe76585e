// sda_api.cpp -- C ABI entry points of libsda: argument validation,
// workspace sizing, launch-shape selection and dispatch.  Nothing here
// allocates device memory or synchronises the host.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include <hip/hip_runtime.h>

#include "sda.h"
#include "sda_kernels.hpp"
#include "sda_proxy_long.hpp"
#include "sda_select.hpp"
#include "sda_cluster.hpp"

#define SDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace sda;

struct Resolved {
  int32_t B, Hq, Hkv, n, d, G, dtype;
  int64_t sb, sh, sn;
  size_t esize;
  float scale;
};

sda_status resolve(const sda_dims* dims, Resolved* r) {
  if (!dims) return SDA_EINVAL;
  if (dims->dtype != SDA_BF16 && dims->dtype != SDA_F32) return SDA_EDTYPE;
  if (dims->B < 1 || dims->Hq < 1 || dims->Hkv < 1 || dims->n < 1 || dims->d < 1) return SDA_ESHAPE;
  if (dims->Hq % dims->Hkv != 0) return SDA_ESHAPE;
  if (dims->d != kD) return SDA_EUNSUPPORTED;
  const int G = dims->Hq / dims->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SDA_EUNSUPPORTED;
  r->B = dims->B;
  r->Hq = dims->Hq;
  r->Hkv = dims->Hkv;
  r->n = dims->n;
  r->d = dims->d;
  r->G = G;
  r->dtype = dims->dtype;
  r->esize = dims->dtype == SDA_BF16 ? 2 : 4;
  const bool contiguous = dims->kv_stride_b == 0 && dims->kv_stride_h == 0 && dims->kv_stride_n == 0;
  if (contiguous) {
    r->sn = kD;
    r->sh = (int64_t)dims->n * kD;
    r->sb = r->sh * dims->Hkv;
  } else {
    r->sb = dims->kv_stride_b;
    r->sh = dims->kv_stride_h;
    r->sn = dims->kv_stride_n;
    if (r->sn < kD || r->sh < 0 || r->sb < 0) return SDA_ESHAPE;
    if (dims->Hkv > 1 && r->sh == 0) return SDA_ESHAPE;
    if (dims->B > 1 && r->sb == 0) return SDA_ESHAPE;
  }
  // rows are read as 16-byte vectors
  const int64_t align = 16 / (int64_t)r->esize;
  if (r->sn % align || r->sh % align || r->sb % align) return SDA_ESHAPE;
  // a unit's rows are addressed with 32-bit byte offsets
  const int64_t unit_bytes = ((int64_t)(dims->n - 1) * r->sn + kD) * (int64_t)r->esize;
  if (unit_bytes > kMaxUnitBytes) return SDA_EUNSUPPORTED;
  float scale = dims->scale;
  if (scale == 0.f) scale = 1.0f / sqrtf((float)kD);
  if (!(scale > 0.f) || !isfinite(scale)) return SDA_EINVAL;
  r->scale = scale;
  return SDA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Split-K shape for the streaming kernels: enough workgroups to fill the chip
// several times over, chunks a multiple of one batch of rows of either kernel
// and at most max_chunk entries.
void stream_shape(int units, int len, int min_chunk, int target_wgs, int* splits, int* chunk,
                  int max_chunk = 1 << 30) {
  int sp = ceil_div(target_wgs, units);
  const int max_sp = len > 0 ? ceil_div(len, min_chunk) : 1;
  if (sp > max_sp) sp = max_sp;
  if (len > 0 && sp < ceil_div(len, max_chunk)) sp = ceil_div(len, max_chunk);
  if (sp < 1) sp = 1;
  int ch = ceil_div(len > 0 ? len : 1, sp);
  ch = ceil_div(ch, kStreamMfmaStep) * kStreamMfmaStep;
  sp = len > 0 ? ceil_div(len, ch) : 1;
  *splits = sp;
  *chunk = ch;
}

struct SparsePlan {
  bool unit;      // one workgroup per unit
  bool two;       // proxy tail over a long list (keys, then values), one workgroup per unit
  int ns;         // slots per wave (unit kernel)
  int splits, chunk;
  size_t ws;
};

sda_status plan_sparse(const Resolved& r, int kind, int m, int C, SparsePlan* pl) {
  const int units = r.B * r.Hkv;
  pl->unit = false;
  pl->two = false;
  pl->ns = 0;
  pl->splits = 1;
  pl->chunk = m;
  pl->ws = 0;
  // One workgroup per unit: each of its waves owns a contiguous run of
  // `chunk` list entries.  bf16 takes the matrix-core kernel, whose waves
  // work in tiles of 16 keys (chunk a multiple of 16, slots = 4 per tile);
  // fp32 takes the vector kernel (chunk a multiple of 4).
  int ns = 0, unit_chunk = 0;
  if (r.dtype == SDA_BF16) {
    const int tiles = ceil_div(ceil_div(m, kUnitWaves), 16);
    if (m > 0 && tiles <= unit_max_tiles(r.G)) {
      ns = 4 * (tiles > 0 ? tiles : 1);
      unit_chunk = 16 * tiles;
    } else if (m == 0) {
      ns = 4;
      unit_chunk = 0;
    }
  } else {
    ns = unit_slots_for(m);
    unit_chunk = 4 * ceil_div(ceil_div(m, kUnitWaves), 4);
  }
  if (kind == SDA_TAIL_PROXY) {
    if (ns != 0) {
      pl->unit = true;
      pl->ns = ns;
      pl->chunk = unit_chunk;
      return SDA_OK;
    }
    if (r.dtype != SDA_BF16 || C < 1 || C > kCmax) return SDA_EUNSUPPORTED;
    // up to 1024 entries: one workgroup per unit, value rows requested as
    // the key tiles are consumed, no workspace
    if (m <= kLongMaxList) {
      pl->two = true;
      pl->chunk = long_chunk(m);
      return SDA_OK;
    }
    // longer: split-K on the matrix cores, each split keeping per-cluster
    // listed counts, logit sums and value sums for the merge that forms the
    // proxies
    stream_shape(units, m, 256, 512, &pl->splits, &pl->chunk);
    pl->ws = (size_t)units * pl->splits * ((size_t)r.G * kPartStride + (size_t)C * kClusterRec) * sizeof(float);
    return SDA_OK;
  }
  if (kind == SDA_TAIL_NONE) {
    if (ns != 0 && units >= 128) {
      pl->unit = true;
      pl->ns = ns;
      pl->chunk = unit_chunk;
      return SDA_OK;
    }
  }
  if (kind == SDA_TAIL_SAMPLED) {
    // scratch per unit: the fp64 exact part (M, D_f, N_f) and its split
    // records, the base draws' moments, the draw partials, the budget and
    // the work-item numbering
    if (m > kSampMaxList || units > kSampMaxUnits) return SDA_EUNSUPPORTED;
    pl->splits = sampled_exact_splits(units);
    pl->ws = (size_t)units * ((size_t)(1 + pl->splits) * r.G * (2 + kD) * sizeof(double) +
                              (size_t)r.G * (4 + kD) * sizeof(double) +
                              (size_t)sampled_max_items(r.n) * r.G * kDrawRec * sizeof(float) +
                              2 * sizeof(int32_t)) +
             sizeof(int32_t);
    return SDA_OK;
  }
  if (kind == SDA_TAIL_NONE || kind == SDA_TAIL_PRIOR) {
    // the matrix-core kernel runs two workgroups per CU: one round of long
    // workgroups beats several rounds of short ones
    const bool mfma = r.dtype == SDA_BF16 && (kind == SDA_TAIL_NONE || 3 * r.G <= 16);
    stream_shape(units, m, 256, mfma ? 512 : 2048, &pl->splits, &pl->chunk, mfma ? kStreamDmaMaxChunk : 1 << 30);
    if (pl->splits > 1) pl->ws = (size_t)units * pl->splits * r.G * kPartStride * sizeof(float);
    return SDA_OK;
  }
  return SDA_EUNSUPPORTED;
}

// bf16 streams run on the matrix-core kernel (the prior when 3G <= 16).
hipError_t launch_stream_any(const AttnParams& p, const Resolved& r, int mode, hipStream_t hs) {
  if (r.dtype == SDA_BF16 && (mode == kModeSparse || mode == kModeDense || (mode == kModePrior && 3 * r.G <= 16)))
    return launch_stream_mfma(p, r.G, mode, hs);
  return launch_stream(p, r.dtype, r.G, mode, hs);
}

void dense_shape(const Resolved& r, int* splits, int* chunk) {
  stream_shape(r.B * r.Hkv, r.n, 512, 2048, splits, chunk);
}

size_t dense_ws(const Resolved& r, bool build) {
  int splits, chunk;
  dense_shape(r, &splits, &chunk);
  if (splits <= 1) return 0;
  size_t ws = (size_t)r.B * r.Hkv * splits * r.G * kPartStride * sizeof(float);
  if (build) ws += (size_t)r.B * r.Hkv * splits * kD * sizeof(float);
  return ws;
}

size_t proxy_ws(const Resolved& r, int C) {
  int chunks, rows;
  proxy_build_shape(r.B * r.Hkv, r.n, C, &chunks, &rows);
  const size_t units = (size_t)r.B * r.Hkv;
  // column sums of K, V and K^2 per (unit, chunk, cluster), then the counts
  return units * chunks * C * (3 * kD * sizeof(float) + sizeof(int32_t));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The chunk maxima (required), then room for the fp64 projections, which
// spares the second pass their recomputation when the workspace holds them.
size_t qgs_build_ws_min(const Resolved& r) {
  return align256((size_t)r.B * r.Hkv * qgs_chunks(r.n) * kQgsRank * sizeof(double));
}
size_t qgs_build_ws(const Resolved& r) {
  return qgs_build_ws_min(r) + (size_t)r.B * r.Hkv * r.n * kQgsRank * sizeof(double);
}

struct QgsSelectWs {
  size_t keys, wq, budget, avail, total;
};

QgsSelectWs qgs_select_ws(const Resolved& r, int C) {
  const size_t units = (size_t)r.B * r.Hkv;
  QgsSelectWs w;
  w.keys = 0;
  w.wq = w.keys + align256(units * r.n * sizeof(uint64_t));
  w.budget = w.wq + align256(units * r.G * (kQgsRank / 4) * sizeof(uint32_t));
  w.avail = w.budget + align256(units * C * sizeof(int32_t));
  w.total = w.avail + align256(units * C * sizeof(int32_t));
  return w;
}

struct QgcWs {
  size_t z, cent, sums, cnt, total;
};

QgcWs qgc_ws(const Resolved& r, int C) {
  const size_t units = (size_t)r.B * r.Hkv;
  QgcWs w;
  w.z = 0;
  w.cent = align256(units * r.n * kQgcRank * sizeof(double));
  w.sums = w.cent + align256(units * C * kQgcRank * sizeof(double));
  w.cnt = w.sums + align256(units * C * kQgcRank * sizeof(uint64_t));
  w.total = w.cnt + align256(units * C * sizeof(int32_t));
  return w;
}

void fill_common(const Resolved& r, AttnParams* p) {
  memset(p, 0, sizeof(*p));
  p->sb = r.sb;
  p->sh = r.sh;
  p->sn = r.sn;
  p->B = r.B;
  p->Hq = r.Hq;
  p->Hkv = r.Hkv;
  p->n = r.n;
  p->qscale = r.scale * 1.4426950408889634f;
  p->q_f32 = r.dtype == SDA_F32;
  p->splits = 1;
}

sda_status hip_status(hipError_t e) { return e == hipSuccess ? SDA_OK : SDA_EHIP; }

}  // namespace

SDA_EXPORT const char* sda_version(void) { return "0.1.0"; }

SDA_EXPORT const char* sda_status_str(int32_t status) {
  switch (status) {
    case SDA_OK: return "ok";
    case SDA_EINVAL: return "invalid argument";
    case SDA_ESHAPE: return "inconsistent shape or stride";
    case SDA_EDTYPE: return "unknown element type";
    case SDA_EWORKSPACE: return "workspace missing or too small";
    case SDA_EUNSUPPORTED: return "unsupported configuration";
    case SDA_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

SDA_EXPORT size_t sda_workspace_bytes(const sda_dims* dims, int32_t op, int32_t tail_kind, int32_t m,
                                      int32_t C) {
  Resolved r;
  if (resolve(dims, &r) != SDA_OK) return 0;
  switch (op) {
    case SDA_OP_SPARSE: {
      if (m < 0) return 0;
      SparsePlan pl;
      if (plan_sparse(r, tail_kind, m, C, &pl) != SDA_OK) return 0;
      return pl.ws;
    }
    case SDA_OP_DENSE: return dense_ws(r, false);
    case SDA_OP_BUILD_PRIOR: return dense_ws(r, true);
    case SDA_OP_BUILD_PROXIES: return (C >= 1 && C <= kCmax) ? proxy_ws(r, C) : 0;
    case SDA_OP_BUILD_QGS: return qgs_build_ws(r);
    case SDA_OP_SELECT_QGS: return (C >= 1 && C <= kCmax) ? qgs_select_ws(r, C).total : 0;
    case SDA_OP_BUILD_QGC: return (C >= 1 && C <= kCmax) ? qgc_ws(r, C).total : 0;
  }
  return 0;
}

SDA_EXPORT sda_status sda_build_tail_proxies(const sda_dims* dims, const void* K, const void* V,
                                             const int32_t* cluster_id, int32_t C, int32_t* count,
                                             float* sumK, float* sumV, float* sumK2, int32_t* dev_flags,
                                             void* ws, size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!K || !V || !cluster_id || !count || !sumK || !sumV) return SDA_EINVAL;
  if (!aligned16(K) || !aligned16(V)) return SDA_EINVAL;
  if (C < 1 || C > kCmax) return SDA_EUNSUPPORTED;
  const size_t need = proxy_ws(r, C);
  if (!ws || ws_bytes < need) return SDA_EWORKSPACE;
  ProxyBuildParams p;
  memset(&p, 0, sizeof(p));
  p.K = K;
  p.V = V;
  p.cid = cluster_id;
  p.sb = r.sb;
  p.sh = r.sh;
  p.sn = r.sn;
  p.Hkv = r.Hkv;
  p.n = r.n;
  p.C = C;
  const int units = r.B * r.Hkv;
  proxy_build_shape(units, r.n, C, &p.chunks, &p.rows_per_chunk);
  p.part = reinterpret_cast<float*>(ws);
  p.pcount = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                        (size_t)units * p.chunks * C * 3 * kD * sizeof(float));
  p.count = count;
  p.sumK = sumK;
  p.sumK2 = sumK2;
  p.sumV = sumV;
  p.flags = dev_flags;
  return hip_status(launch_proxy_build(p, r.dtype, units, reinterpret_cast<hipStream_t>(stream)));
}

SDA_EXPORT sda_status sda_build_prior(const sda_dims* dims, const void* K, const void* V, const float* mu_Q,
                                      float* mu_K, float* O_est, float* maxP, float* sumP, void* ws,
                                      size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!K || !V || !mu_Q || !mu_K || !O_est || !maxP || !sumP) return SDA_EINVAL;
  if (!aligned16(K) || !aligned16(V) || !aligned16(mu_Q)) return SDA_EINVAL;
  const size_t need = dense_ws(r, true);
  if (need && (!ws || ws_bytes < need)) return SDA_EWORKSPACE;
  AttnParams p;
  fill_common(r, &p);
  p.q = mu_Q;
  p.q_f32 = 1;
  p.K = K;
  p.V = V;
  dense_shape(r, &p.splits, &p.chunk);
  const size_t part_bytes = (size_t)r.B * r.Hkv * p.splits * r.G * kPartStride * sizeof(float);
  p.part = reinterpret_cast<float*>(ws);
  p.ksum = p.splits > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + part_bytes) : nullptr;
  p.out = O_est;
  p.lse = maxP;
  p.aux = sumP;
  p.aux2 = mu_K;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_stream(p, r.dtype, r.G, kModeBuildPrior, hs);
  if (e == hipSuccess && p.splits > 1) e = launch_merge(p, r.G, kModeBuildPrior, hs);
  return hip_status(e);
}

SDA_EXPORT sda_status sda_dense_decode_attn(const sda_dims* dims, const void* q, const void* K, const void* V,
                                            float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!q || !K || !V || !out) return SDA_EINVAL;
  if (!aligned16(q) || !aligned16(K) || !aligned16(V)) return SDA_EINVAL;
  const size_t need = dense_ws(r, false);
  if (need && (!ws || ws_bytes < need)) return SDA_EWORKSPACE;
  AttnParams p;
  fill_common(r, &p);
  p.q = q;
  p.K = K;
  p.V = V;
  dense_shape(r, &p.splits, &p.chunk);
  p.part = reinterpret_cast<float*>(ws);
  p.out = out;
  p.lse = lse;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_stream_any(p, r, kModeDense, hs);
  if (e == hipSuccess && p.splits > 1) e = launch_merge(p, r.G, kModeDense, hs);
  return hip_status(e);
}

namespace {

// The decode step behind both decode entry points: ws/ws_bytes is the
// caller's workspace or the library's static scratch.
sda_status sparse_decode(const sda_dims* dims, const void* q, const void* K, const void* V, const int32_t* idx,
                         const int32_t* idx_len, const float* logw, int32_t m, const sda_tail* tail, float* out,
                         float* lse, int32_t* dev_flags, void* ws, size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!q || !K || !V || !out) return SDA_EINVAL;
  if (!aligned16(q) || !aligned16(K) || !aligned16(V)) return SDA_EINVAL;
  const int kind = tail ? tail->kind : SDA_TAIL_NONE;
  if (kind < SDA_TAIL_NONE || kind > SDA_TAIL_SAMPLED) return SDA_EINVAL;
  if (m < 0) return SDA_ESHAPE;
  if (m > 0 && !idx) return SDA_EINVAL;
  if (m == 0 && kind == SDA_TAIL_NONE) return SDA_EINVAL;

  AttnParams p;
  fill_common(r, &p);
  p.q = q;
  p.K = K;
  p.V = V;
  p.idx = idx;
  p.idx_len = idx_len;
  p.logw = logw;
  p.m = m;
  p.out = out;
  p.lse = lse;
  p.flags = dev_flags;

  if (kind == SDA_TAIL_PROXY) {
    if (tail->C < 1 || tail->C > kCmax) return SDA_EUNSUPPORTED;
    if (!tail->count || !tail->sumK || !tail->sumV) return SDA_EINVAL;
    if (!aligned16(tail->sumK) || !aligned16(tail->sumV)) return SDA_EINVAL;
    if (m > 0 && !tail->idx_cluster && !tail->cluster_id) return SDA_EINVAL;
    p.C = tail->C;
    p.idx_cluster = tail->idx_cluster;
    p.cluster_id = tail->cluster_id;
    p.count = tail->count;
    p.sumK = tail->sumK;
    p.sumV = tail->sumV;
  } else if (kind == SDA_TAIL_PRIOR) {
    if (!tail->mu_Q || !tail->mu_K || !tail->O_est || !tail->maxP || !tail->sumP) return SDA_EINVAL;
    if (!aligned16(tail->mu_Q) || !aligned16(tail->mu_K)) return SDA_EINVAL;
    if (!(tail->lambda >= 0.f) || !isfinite(tail->lambda)) return SDA_EINVAL;
    if (tail->prior_n < 0 || tail->prior_n > r.n) return SDA_EINVAL;
    p.mu_Q = tail->mu_Q;
    p.mu_K = tail->mu_K;
    p.O_est = tail->O_est;
    p.maxP = tail->maxP;
    p.sumP = tail->sumP;
    p.lambda = tail->lambda;
    p.prior_n = tail->prior_n > 0 ? tail->prior_n : r.n;
  } else if (kind == SDA_TAIL_SAMPLED) {
    if (!(tail->eps > 0.0) || !isfinite(tail->eps)) return SDA_EINVAL;
    if (tail->nz < 0 || tail->nz > SDA_MAX_Z_SPLITS) return SDA_EINVAL;
    if (tail->nz == 0) {
      if (!(tail->z > 0.0) || !isfinite(tail->z)) return SDA_EINVAL;
    } else {
      // the verified budget: eps bounds the output's relative error (< 1)
      if (!tail->z_split || !(tail->eps < 1.0)) return SDA_EINVAL;
      for (int k = 0; k < 2 * tail->nz; ++k) {
        const double zk = tail->z_split[k];
        if (!(zk > 0.0) || !isfinite(zk)) return SDA_EINVAL;
        p.zs[k] = zk;
      }
      p.nz = tail->nz;
    }
    if (tail->b0 < 2 || tail->b0 > kSampMaxB0) return SDA_EUNSUPPORTED;
    if (tail->b_cap < 0 || (tail->samples_out && tail->b_cap == 0)) return SDA_EINVAL;
    p.scale = r.scale;
    p.eps = tail->eps;
    p.z = tail->z;
    p.b0 = tail->b0;
    p.seed = tail->seed;
    p.b_cap = tail->b_cap;
    p.b_out = tail->b_out;
    p.bstar_out = tail->bstar_out;
    p.samples_out = tail->samples_out;
  }

  SparsePlan pl;
  st = plan_sparse(r, kind, m, kind == SDA_TAIL_PROXY ? tail->C : 0, &pl);
  if (st != SDA_OK) return st;
  if (pl.ws && (!ws || ws_bytes < pl.ws)) return SDA_EWORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (kind == SDA_TAIL_SAMPLED) {
    const size_t units = (size_t)r.B * r.Hkv;
    char* w = reinterpret_cast<char*>(ws);
    p.wstat = reinterpret_cast<double*>(w);
    w += units * (size_t)r.G * (2 + kD) * sizeof(double);
    p.splits = pl.splits;
    p.wexact = reinterpret_cast<double*>(w);
    w += units * (size_t)pl.splits * r.G * (2 + kD) * sizeof(double);
    p.wbase = reinterpret_cast<double*>(w);
    w += units * (size_t)r.G * (4 + kD) * sizeof(double);
    p.part = reinterpret_cast<float*>(w);
    w += units * (size_t)sampled_max_items(r.n) * r.G * kDrawRec * sizeof(float);
    p.wb = reinterpret_cast<int32_t*>(w);
    w += units * sizeof(int32_t);
    p.wsched = reinterpret_cast<int32_t*>(w);
    return hip_status(launch_sampled(p, r.dtype, r.G, hs));
  }
  if (pl.unit) {
    p.chunk = pl.chunk;
    return hip_status(launch_sparse_unit(p, r.dtype, r.G, kind == SDA_TAIL_PROXY, pl.ns, hs));
  }
  if (pl.two) {
    p.chunk = pl.chunk;
    return hip_status(launch_proxy_long(p, r.G, hs));
  }
  if (kind == SDA_TAIL_PROXY) {
    p.splits = pl.splits;
    p.chunk = pl.chunk;
    p.part = reinterpret_cast<float*>(ws);
    p.cpart = p.part + (size_t)r.B * r.Hkv * pl.splits * r.G * kPartStride;
    hipError_t e = launch_stream_mfma(p, r.G, kModeProxy, hs);
    if (e == hipSuccess) e = launch_merge(p, r.G, kModeProxy, hs);
    return hip_status(e);
  }
  p.splits = pl.splits;
  p.chunk = pl.chunk;
  p.part = reinterpret_cast<float*>(ws);
  const int mode = kind == SDA_TAIL_PRIOR ? kModePrior : kModeSparse;
  hipError_t e = launch_stream_any(p, r, mode, hs);
  if (e == hipSuccess && p.splits > 1) e = launch_merge(p, r.G, mode, hs);
  return hip_status(e);
}

// Scratch for the entry point that allocates nothing: one array per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address); it uses the address hipGetSymbolAddress returns for the current
// device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[SDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

sda_status scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SDA_EHIP;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SDA_EHIP;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // the same value from any racing thread
  }
  *out = ptr;
  return SDA_OK;
}

}  // namespace

SDA_EXPORT sda_status sda_sparse_decode_attn(const sda_dims* dims, const void* q, const void* K, const void* V,
                                             const int32_t* idx, const int32_t* idx_len, const float* logw,
                                             int32_t m, const sda_tail* tail, float* out, float* lse,
                                             int32_t* dev_flags, void* ws, size_t ws_bytes, void* stream) {
  return sparse_decode(dims, q, K, V, idx, idx_len, logw, m, tail, out, lse, dev_flags, ws, ws_bytes, stream);
}

SDA_EXPORT sda_status sda_sparse_decode_attn_noalloc(const sda_dims* dims, const void* q, const void* K,
                                                     const void* V, const int32_t* idx, const int32_t* idx_len,
                                                     const float* logw, int32_t m, const sda_tail* tail, float* out,
                                                     float* lse, int32_t* dev_flags, void* stream) {
  // the size check first, so that a call too large for the scratch fails
  // before anything touches the device
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  const int kind = tail ? tail->kind : SDA_TAIL_NONE;
  if (kind < SDA_TAIL_NONE || kind > SDA_TAIL_SAMPLED || m < 0) return SDA_EINVAL;
  SparsePlan pl;
  st = plan_sparse(r, kind, m, (kind == SDA_TAIL_PROXY && tail) ? tail->C : 0, &pl);
  if (st != SDA_OK) return st;
  if (pl.ws > (size_t)SDA_NOALLOC_SCRATCH_BYTES) return SDA_EWORKSPACE;
  void* ws = nullptr;
  if (pl.ws > 0) {
    st = scratch_for_current_device(&ws);
    if (st != SDA_OK) return st;
  }
  return sparse_decode(dims, q, K, V, idx, idx_len, logw, m, tail, out, lse, dev_flags, ws,
                       pl.ws > 0 ? (size_t)SDA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

SDA_EXPORT sda_status sda_build_qgs_codes(const sda_dims* dims, const void* K, const float* U, int8_t* codes,
                                          double* kmax, void* ws, size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!K || !U || !codes || !kmax) return SDA_EINVAL;
  if (!aligned16(K) || !aligned16(codes)) return SDA_EINVAL;
  const size_t need = qgs_build_ws_min(r);
  if (!ws || ws_bytes < need) return SDA_EWORKSPACE;
  QgsBuildParams p;
  memset(&p, 0, sizeof(p));
  p.K = K;
  p.U = U;
  p.sb = r.sb;
  p.sh = r.sh;
  p.sn = r.sn;
  p.Hkv = r.Hkv;
  p.n = r.n;
  p.chunks = qgs_chunks(r.n);
  p.part = reinterpret_cast<double*>(ws);
  p.y = ws_bytes >= qgs_build_ws(r) ? reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + need) : nullptr;
  p.codes = codes;
  p.kmax = kmax;
  return hip_status(launch_qgs_build(p, r.dtype, r.B * r.Hkv, reinterpret_cast<hipStream_t>(stream)));
}

SDA_EXPORT sda_status sda_select_qgs(const sda_dims* dims, const void* q, const sda_selector* sel, int32_t m,
                                     int32_t* idx, int32_t* idx_len, int32_t* idx_cluster, int32_t* budget,
                                     int32_t* dev_flags, void* ws, size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!q || !sel || !idx || !idx_len || !idx_cluster) return SDA_EINVAL;
  if (!sel->cluster_id || !sel->count || !sel->sumK || !sel->sumK2 || !sel->U || !sel->codes || !sel->kmax)
    return SDA_EINVAL;
  if (!aligned16(sel->codes) || !aligned16(sel->U) || !aligned16(sel->sumK) || !aligned16(sel->sumK2))
    return SDA_EINVAL;
  if (sel->C < 1 || sel->C > kCmax) return SDA_EUNSUPPORTED;
  if (r.n > kQgsMaxN) return SDA_EUNSUPPORTED;
  if (sel->n_sink < 0 || sel->n_local < 0 || sel->E < 0) return SDA_EINVAL;
  const int64_t most = std::min<int64_t>((int64_t)r.n, (int64_t)sel->n_sink + sel->n_local + sel->E);
  if (m < most) return SDA_EINVAL;
  const QgsSelectWs w = qgs_select_ws(r, sel->C);
  if (!ws || ws_bytes < w.total) return SDA_EWORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  QgsSelectParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.cid = sel->cluster_id;
  p.count = sel->count;
  p.sumK = sel->sumK;
  p.sumK2 = sel->sumK2;
  p.U = sel->U;
  p.codes = sel->codes;
  p.kmax = sel->kmax;
  p.B = r.B;
  p.Hq = r.Hq;
  p.Hkv = r.Hkv;
  p.n = r.n;
  p.G = r.G;
  p.C = sel->C;
  p.n_sink = sel->n_sink;
  p.n_local = sel->n_local;
  p.E = sel->E;
  p.m = m;
  p.scale = r.scale;
  p.keys = reinterpret_cast<uint64_t*>(base + w.keys);
  p.wq = reinterpret_cast<uint32_t*>(base + w.wq);
  p.wbudget = reinterpret_cast<int32_t*>(base + w.budget);
  p.wavail = reinterpret_cast<int32_t*>(base + w.avail);
  p.idx = idx;
  p.idx_len = idx_len;
  p.idx_cluster = idx_cluster;
  p.budget = budget;
  p.flags = dev_flags;
  return hip_status(launch_qgs_select(p, r.dtype, reinterpret_cast<hipStream_t>(stream)));
}

SDA_EXPORT sda_status sda_build_qgc_clusters(const sda_dims* dims, const void* K, const float* V, int32_t C,
                                             int32_t T, int32_t* cluster_id, int32_t* dev_flags, void* ws,
                                             size_t ws_bytes, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!K || !V || !cluster_id) return SDA_EINVAL;
  if (!aligned16(K) || !aligned16(V)) return SDA_EINVAL;
  if (C < 1 || C > kCmax) return SDA_EUNSUPPORTED;
  if (T < 1 || T > 1000) return SDA_EINVAL;
  if (r.n > kQgcMaxN) return SDA_EUNSUPPORTED;
  const QgcWs w = qgc_ws(r, C);
  if (!ws || ws_bytes < w.total) return SDA_EWORKSPACE;
  char* base = reinterpret_cast<char*>(ws);
  QgcParams p;
  memset(&p, 0, sizeof(p));
  p.K = K;
  p.V = V;
  p.sb = r.sb;
  p.sh = r.sh;
  p.sn = r.sn;
  p.Hkv = r.Hkv;
  p.n = r.n;
  p.C = C;
  p.z = reinterpret_cast<double*>(base + w.z);
  p.cent = reinterpret_cast<double*>(base + w.cent);
  p.sums = reinterpret_cast<unsigned long long*>(base + w.sums);
  p.cnt = reinterpret_cast<int32_t*>(base + w.cnt);
  p.cluster_id = cluster_id;
  p.flags = dev_flags;
  return hip_status(launch_qgc(p, r.dtype, r.B * r.Hkv, T, reinterpret_cast<hipStream_t>(stream)));
}

SDA_EXPORT sda_status sda_gather_rows(const sda_dims* dims, const void* K, const void* V, const int32_t* idx,
                                      int32_t m, const void* state, int64_t state_bytes, int32_t waves,
                                      int32_t parts, uint32_t* checksum, void* stream) {
  Resolved r;
  sda_status st = resolve(dims, &r);
  if (st != SDA_OK) return st;
  if (!K || !V || !checksum || (m > 0 && !idx)) return SDA_EINVAL;
  if (r.dtype != SDA_BF16) return SDA_EUNSUPPORTED;  // a lane quarter covers one 256-byte bf16 row
  if (!aligned16(K) || !aligned16(V)) return SDA_EINVAL;
  if (m < 0 || state_bytes < 0) return SDA_ESHAPE;
  if (state_bytes > 0 && (!state || !aligned16(state) || state_bytes % 16)) return SDA_EINVAL;
  if (waves != 4 && waves != 8 && waves != 16) return SDA_EUNSUPPORTED;
  if (parts < 1 || parts > 16) return SDA_EUNSUPPORTED;
  const int rows = gather_rows_per_group(m, waves, parts);
  if (rows > (waves == 16 ? 12 : 24)) return SDA_EUNSUPPORTED;
  GatherParams p;
  memset(&p, 0, sizeof(p));
  p.K = K;
  p.V = V;
  // with an empty list the kernel still reads one (discarded) word
  p.idx = idx ? idx : reinterpret_cast<const int32_t*>(checksum);
  p.state = state;
  p.state_bytes = state_bytes;
  p.sb = r.sb;
  p.sh = r.sh;
  p.sn = r.sn;
  p.esize = (int)r.esize;
  p.row_bytes = (int)(r.sn * (int64_t)r.esize);
  p.Hkv = r.Hkv;
  p.n = r.n;
  p.m = m;
  p.parts = parts;
  p.checksum = checksum;
  return hip_status(launch_gather_rows(p, waves, r.B * r.Hkv, reinterpret_cast<hipStream_t>(stream)));
}
