// sda_proxy_long.hip -- the decode step with count-aware mean proxies
// ("OpenAttention: One Percent Is Enough with Tail Proxies", method stages
// 04-05: each cluster's unread members fold into one virtual token that
// shares the softmax with the listed rows) for bf16 lists of up to 1024
// entries per (sequence, KV head) -- longer than the one-pass kernel holds
// (the page's 3% read at 32K, 1% at 96K) -- in two launches of one
// 512-thread workgroup per unit:
//
//   proxy_long_logits_kernel  keys only: the listed logits (matrix cores),
//       each cluster's listed count and logit sum, the proxies' mean logits
//       mu_b = (scale <q, sumK_b> - listed logits) / n_b, the exact unit
//       maximum M over listed rows and proxies; then every listed row's
//       weight e^{s - M} - [read member of b] e^{mu_b - M}, the cluster
//       coefficients e^{mu_b - M} and the normaliser
//       sum_listed e^{s - M} + sum_b n_b e^{mu_b - M}, to the workspace.
//   proxy_long_values_kernel  values only: sum_listed w v on the matrix cores
//       (each weight as three bf16 parts, together exact to fp32), plus
//       sum_b e^{mu_b - M} sumV_b in fp32, divided by the normaliser.
//
// A read member's value sits both in its cluster's sumV_b and among the
// listed rows; its weight carries -e^{mu_b - M}, so the read share of sumV_b
// cancels at fp32 accuracy.  Both kernels see the whole unit, so the maximum
// is exact and no split merge is needed.
#include "sda_device.hpp"
#include "sda_kernels.hpp"
#include "sda_proxy_long.hpp"

namespace sda {

namespace {

constexpr int kW = kLongWaves;           // waves per workgroup
constexpr int kNT = kLongMaxPerWave / 16;  // tiles of 16 entries per wave
constexpr int kNS = 4 * kNT;             // value slots per row group
constexpr int kCap = kW * kLongMaxPerWave;  // entries per unit
constexpr int kVRow = 144;               // bf16 elements per staged value row (bank spread)
constexpr int kOOBL = kMaxUnitBytes;     // offset past every row: the load returns zeros
constexpr int kStreamNT = 2;             // non-temporal hint for rows read once

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t rows_of(const void* base, int64_t n, int64_t sn) {
  const int64_t bytes = ((int64_t)(n - 1) * sn + kD) * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int lshfl(int v, int src) { return __shfl(v, src, 64); }

// number of listed entries of unit u (idx_len clamped to [0, m], flagged
// by the logits kernel)
__device__ __forceinline__ int list_len(const AttnParams& p, int u) {
  if (!p.idx_len) return p.m;
  const int L = p.idx_len[u];
  return L < 0 ? 0 : (L > p.m ? p.m : L);
}

// per-unit layout of the coefficient block: C*G cluster coefficients, then
// G maxima (log2 units), then G normalisers
__device__ __forceinline__ float* coef_block(const AttnParams& p, int u, int G) {
  return p.cpart + (int64_t)u * (p.C * G + 2 * G);
}

}  // namespace

template <int G>
__global__ __launch_bounds__(512) void proxy_long_logits_kernel(const AttnParams p) {
  const int u = blockIdx.x;
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int C = p.C;
  const int chunk = p.chunk;  // entries per wave (a multiple of 16, <= 128)

  __shared__ float s_x[G][kCap];         // listed logits (log2 units, with the log-weight), -inf if absent
  __shared__ int s_cl[kCap];             // cluster of each entry, -1 if none
  __shared__ float s_cs[kW][kCmax][G];   // per wave: listed raw logits summed per cluster
  __shared__ int s_cn[kW][kCmax];        // per wave: listed rows per cluster
  __shared__ float s_wm[kW][G];          // per wave: maximum listed logit
  __shared__ float s_qk[kCmax][G];       // scale log2(e) <q_h, sumK_b>
  __shared__ float s_mu[kCmax][G];       // proxy mean logit (log2 units), -inf if no unread member
  __shared__ float s_pi[kCmax][G];       // mu_b + log2 n_b
  __shared__ float s_M[G];
  __shared__ float s_L[kW][G];

  int L = p.m;
  if (p.idx_len) {
    L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
  }
  const int64_t lbase = (int64_t)u * p.m;
  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;

  // ---- this wave's slots start at zero ---------------------------------------
  for (int i = lane; i < kCmax * G; i += 64) (&s_cs[w][0][0])[i] = 0.f;
  for (int i = lane; i < kCmax; i += 64) s_cn[w][i] = 0;

  // ---- list entries of the lane's keys: tile t, key r16 --------------------------
  int jt[kNT], ct[kNT];
  float lwt[kNT];
  bool vt[kNT];
  int bad = 0;
  const bool lookup = p.idx_cluster == nullptr;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int k = 16 * t + r16;
    const int e = w * chunk + k;
    const bool live = k < chunk && e < L;
    const int64_t a = lbase + (live ? e : 0);
    const int j = p.idx[a];
    const int jp = p.idx[lbase + ((live && e > 0) ? e - 1 : 0)];
    const float lw = p.logw ? p.logw[a] : 0.f;
    const int c = lookup ? -1 : p.idx_cluster[a];
    const bool inr = (unsigned)j < (unsigned)p.n;
    if (live && !inr) bad |= SDA_FLAG_IDX_RANGE;
    if (live && e > 0 && jp >= j) bad |= SDA_FLAG_IDX_ORDER;
    if (live && inr && !lookup && (c < -1 || c >= C)) bad |= SDA_FLAG_CLUSTER;
    vt[t] = live && inr;
    jt[t] = vt[t] ? j : 0;
    lwt[t] = lw;
    ct[t] = c;
  }
  if (lookup) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) ct[t] = vt[t] ? p.cluster_id[(int64_t)u * p.n + jt[t]] : -1;
  }
  if (bad) flag_unit(p.flags, u, bad);

  // ---- key rows in the matrix-core operand layout (16 keys x 64 bytes a load) ---
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = rows_of(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  uint4 kt[kNT][4];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int off = vt[t] ? (int)(((int64_t)jt[t] * p.sn + 8 * sub) * 2) : kOOBL;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 64 * st, 0, kStreamNT);
      kt[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

  // ---- while the keys are in flight: q . sumK_b, and the A operand -----------
  for (int i = tid; i < C * G; i += 512) {
    const int b = i / G, h = i - b * G;
    const bf16_t* qh = reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + h) * kD;
    const float* sk = p.sumK + ((int64_t)u * C + b) * kD;
    float a = 0.f;
#pragma unroll 4
    for (int d0 = 0; d0 < kD; d0 += 8) {
      RowChunk<bf16_t> c;
      c.load_cached(qh + d0);
      float f[8], kf[8];
      c.unpack(f);
      load8f(sk + d0, kf);
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) a = fmaf(f[i2], kf[i2], a);
    }
    s_qk[b][h] = a * p.qscale;
  }
  uint4 qa[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qa[st] = make_uint4(0, 0, 0, 0);
    if (r16 < G)
      qa[st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + r16) * kD + 32 * st +
                                                8 * sub);
  }
  wave_lds_sync();  // the wave's zeroed slots

  // ---- logits: d[i] = head 4 sub + i of key r16 -------------------------------
  float bm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                  __builtin_bit_cast(bf16x8_t, kt[t][st]), d, 0, 0, 0);
    const int e = w * chunk + 16 * t + r16;
    const int c = (vt[t] && ct[t] >= 0 && ct[t] < C) ? ct[t] : -1;
    const float lw = p.logw ? lwt[t] * kLog2e : 0.f;
    if (16 * t < chunk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * sub + i;
        if (h < G) {
          const float raw = d[i] * p.qscale;
          const float x = vt[t] ? raw + lw : kNegInf;
          s_x[h][e] = x;
          bm[i] = fmaxf(bm[i], x);
          if (c >= 0) __hip_atomic_fetch_add(&s_cs[w][c][h], raw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      if (sub == 0) {
        s_cl[e] = c;
        if (c >= 0) __hip_atomic_fetch_add(&s_cn[w][c], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = max16(bm[i]);
    if (r16 == 0 && 4 * sub + i < G) s_wm[w][4 * sub + i] = v;
  }
  __syncthreads();

  // ---- the proxies: mean logit of each cluster's unread members ---------------
  for (int i = tid; i < C * G; i += 512) {
    const int b = i / G, h = i - b * G;
    float S = 0.f;
    int cnt = 0;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) {
      S += s_cs[ww][b][h];
      cnt += s_cn[ww][b];
    }
    const int nb = p.count[(int64_t)u * C + b] - cnt;
    if (nb < 0 && h == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
    const bool ok = nb > 0;
    const float mu = ok ? (s_qk[b][h] - S) / (float)nb : kNegInf;
    s_mu[b][h] = mu;
    s_pi[b][h] = ok ? mu + __builtin_amdgcn_logf((float)nb) : kNegInf;
  }
  __syncthreads();
  if (tid < G) {
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmaxf(M, s_wm[ww][tid]);
    for (int b = 0; b < C; ++b) M = fmaxf(M, s_pi[b][tid]);
    s_M[tid] = M;
  }
  __syncthreads();

  // ---- weights, cluster coefficients and the normaliser ------------------------
  const int ncap = kW * chunk;
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = 0.f;
  for (int e = tid; e < ncap; e += 512) {
    const int c = s_cl[e];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float M = s_M[h];
      const float x = s_x[h][e];
      const float ex = (M == kNegInf || x == kNegInf) ? 0.f : fast_exp2(x - M);
      const float mu = c >= 0 ? s_mu[c][h] : kNegInf;
      const float corr = (M == kNegInf || mu == kNegInf) ? 0.f : fast_exp2(mu - M);
      lsum[h] += ex;
      p.part[((int64_t)u * G + h) * ncap + e] = ex - corr;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = sum_rowgroups(sum16(lsum[h]));
    if (lane == 0) s_L[w][h] = v;
  }
  __syncthreads();
  float* cb = coef_block(p, u, G);
  for (int i = tid; i < C * G; i += 512) {
    const int b = i / G, h = i - b * G;
    const float M = s_M[h], mu = s_mu[b][h];
    cb[i] = (M == kNegInf || mu == kNegInf) ? 0.f : fast_exp2(mu - M);
  }
  if (tid < G) {
    const float M = s_M[tid];
    float Lh = 0.f;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) Lh += s_L[ww][tid];
    for (int b = 0; b < C; ++b) {
      const float pi = s_pi[b][tid];
      if (M != kNegInf && pi != kNegInf) Lh += fast_exp2(pi - M);
    }
    cb[C * G + tid] = M;
    cb[C * G + G + tid] = Lh;
  }
}

template <int G>
__global__ __launch_bounds__(512) void proxy_long_values_kernel(const AttnParams p) {
  constexpr int R2 = 2 * G;  // accumulator rows in use: high+middle parts (h), remainders (G + h)
  const int u = blockIdx.x;
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int C = p.C;
  const int chunk = p.chunk;
  const int ncap = kW * chunk;

  __shared__ int s_j[kCap];                       // row of each entry, -1 if absent
  __shared__ __attribute__((aligned(16))) float s_w[G][kCap];  // weights
  __shared__ __attribute__((aligned(16))) bf16_t s_vt[kW][16 * kVRow];  // each wave's value tile
  __shared__ __attribute__((aligned(16))) float s_red[kW][R2][kD];      // each wave's products

  const int L = list_len(p, u);
  const int64_t lbase = (int64_t)u * p.m;
  const float* cb = coef_block(p, u, G);

  // ---- the unit's list and weights into LDS ------------------------------------
  for (int e = tid; e < ncap; e += 512) {
    int j = -1;
    if (e < L) {
      j = p.idx[lbase + e];
      if ((unsigned)j >= (unsigned)p.n) j = -1;  // flagged by the logits kernel
    }
    s_j[e] = j;
  }
  for (int i = tid; i < G * ncap; i += 512) {
    const int h = i / ncap, e = i - h * ncap;
    s_w[h][e] = p.part[((int64_t)u * G + h) * ncap + e];
  }
  __syncthreads();

  // ---- value rows to registers: slot k of row group sub = wave key 4k + sub -------
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rv = rows_of(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);
  uint4 vc[kNS];
#pragma unroll
  for (int k = 0; k < kNS; ++k) {
    const int kk = 4 * k + sub;
    const int j = kk < chunk ? s_j[w * chunk + kk] : -1;
    const int off = j >= 0 ? (int)(((int64_t)j * p.sn + 8 * r16) * 2) : kOOBL;
    auto v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kStreamNT);
    vc[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }

  // ---- while they fly: the cluster terms sum_b e^{mu_b - M} sumV_b (fp32) ------
  float cterm[(G * kD + 511) / 512];
#pragma unroll
  for (int q = 0; q < (G * kD + 511) / 512; ++q) {
    const int i = tid + 512 * q;
    float a = 0.f;
    if (i < G * kD) {
      const int h = i / kD, dim = i - h * kD;
      for (int b = 0; b < C; ++b) a = fmaf(cb[b * G + h], p.sumV[((int64_t)u * C + b) * kD + dim], a);
    }
    cterm[q] = a;
  }

  // ---- weighted values on the matrix cores ------------------------------------
  floatx4_t oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  bf16_t* vt = s_vt[w];
  const int hr = r16 < G ? r16 : (r16 < R2 ? r16 - G : 0);
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (16 * t >= chunk) break;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
      *reinterpret_cast<uint4*>(vt + (4 * kq + sub) * kVRow + 8 * r16) = vc[4 * t + kq];
    wave_lds_sync();  // the tile's rows, staged by other lanes
    // A: the weights of keys 16t + 4 sub + j; rows h take the high and middle
    // parts (K halves), rows G + h the remainder
    const float4 w4 = *reinterpret_cast<const float4*>(&s_w[hr][w * chunk + 16 * t + 4 * sub]);
    const float ws[4] = {w4.x, w4.y, w4.z, w4.w};
    bf16x8_t a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = ws[j];
      const __bf16 hi = (__bf16)x;
      const float r1 = x - (float)hi;
      const __bf16 mid = (__bf16)r1;
      const __bf16 lo = (__bf16)(r1 - (float)mid);
      if (r16 < G) {
        a[j] = hi;
        a[4 + j] = mid;
      } else if (r16 < R2) {
        a[j] = lo;
        a[4 + j] = (__bf16)0.f;
      } else {
        a[j] = (__bf16)0.f;
        a[4 + j] = (__bf16)0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      auto src = (__attribute__((address_space(3))) bf16x4_t*)(vt + (4 * sub + (r16 >> 2)) * kVRow + 16 * nb +
                                                               4 * (r16 & 3));
      const bf16x4_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src);
      const bf16x8_t b = {b4[0], b4[1], b4[2], b4[3], b4[0], b4[1], b4[2], b4[3]};
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[nb], 0, 0, 0);
    }
  }

  // ---- the waves' products, then out = (products + cluster terms) / normaliser ---
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * sub + i;
    if (r < R2) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) s_red[w][r][16 * nb + r16] = oacc[nb][i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < (G * kD + 511) / 512; ++q) {
    const int i = tid + 512 * q;
    if (i < G * kD) {
      const int h = i / kD, dim = i - h * kD;
      float a = cterm[q];
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) a += s_red[ww][h][dim] + s_red[ww][G + h][dim];
      const float M = cb[C * G + h], Lh = cb[C * G + G + h];
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      p.out[qh * kD + dim] = Lh > 0.f ? a / Lh : 0.f;
      if (dim == 0 && p.lse) p.lse[qh] = Lh > 0.f ? (M + __builtin_amdgcn_logf(Lh)) * kLn2 : kNegInf;
    }
  }
}

template <int G>
static hipError_t launch_long_g(const AttnParams& p, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  hipLaunchKernelGGL((proxy_long_logits_kernel<G>), grid, block, 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((proxy_long_values_kernel<G>), grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_proxy_long(const AttnParams& p, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_long_g<1>(p, st);
    case 2: return launch_long_g<2>(p, st);
    case 4: return launch_long_g<4>(p, st);
    case 8: return launch_long_g<8>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sda
