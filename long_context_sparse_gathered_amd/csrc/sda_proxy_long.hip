// sda_proxy_long.hip -- the decode step with count-aware mean proxies
// ("OpenAttention: One Percent Is Enough with Tail Proxies", method stages
// 04-05: each cluster's unread members fold into one virtual token that
// shares the softmax with the listed rows) for bf16 lists of up to 1024
// entries per (sequence, KV head) -- longer than the one-pass kernel holds
// (the page's 3% read at 32K, 1% at 96K) -- in one 512-thread workgroup per
// unit.  Each wave owns up to 128 consecutive entries:
//
//   1. every key row is requested at once (matrix-core operand layout);
//   2. per tile of 16 keys: the logits on the matrix cores, then the tile's
//      value rows requested into the registers its keys held, then the
//      tile's runs of equal cluster id summed with DPP row shifts (one LDS
//      add per run and head into the wave's own slots);
//   3. the proxies' mean logits mu_b = (scale <q, sumK_b> - listed logits)
//      / n_b and the exact unit maximum M over listed rows and proxies;
//   4. every listed row's weight e^{s - M} - [read member of b] e^{mu_b - M}
//      in LDS, the normaliser sum_listed e^{s - M} + sum_b n_b e^{mu_b - M},
//      the cluster terms sum_b e^{mu_b - M} sumV_b in fp32;
//   5. the weighted values on the matrix cores, each weight as three bf16
//      parts (together exact to fp32).
//
// A read member's value sits both in its cluster's sumV_b and among the
// listed rows; its weight carries -e^{mu_b - M}, so the read share of sumV_b
// cancels at fp32 accuracy.  The value rows stream while later key tiles
// are still being turned into logits, so the two streams overlap.
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

}  // namespace

// Run structure of the 16 keys of a row group (lane r16 = key, in list
// order): the inclusive sum of v over the run of equal cluster ids that ends
// at this lane (DPP row shifts; lanes before the row start see zero).
template <int K>
__device__ __forceinline__ float row_shr_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + K, 0xF, 0xF, true));
}
template <int K>
__device__ __forceinline__ int row_shr_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + K, 0xF, 0xF, true);
}
__device__ __forceinline__ float run_sum(float v, int start) {
  int f = start;
  float vp = row_shr_f<1>(v);
  int fp = row_shr_i<1>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_f<2>(v);
  fp = row_shr_i<2>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_f<4>(v);
  fp = row_shr_i<4>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_f<8>(v);
  v = f ? v : v + vp;
  return v;
}
__device__ __forceinline__ int run_count(int v, int start) {
  int f = start;
  int vp = row_shr_i<1>(v);
  int fp = row_shr_i<1>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_i<2>(v);
  fp = row_shr_i<2>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_i<4>(v);
  fp = row_shr_i<4>(f);
  v = f ? v : v + vp;
  f |= fp;
  vp = row_shr_i<8>(v);
  v = f ? v : v + vp;
  return v;
}

template <int G>
__global__ __launch_bounds__(512) void proxy_long_kernel(const AttnParams p) {
  constexpr int R2 = 2 * G;  // accumulator rows in use: high+middle parts (h), remainders (G + h)
  constexpr int kTileBytes = 16 * kVRow * 2;
  constexpr int kPool = kW * kTileBytes > kW * R2 * kD * 4 ? kW * kTileBytes : kW * R2 * kD * 4;
  const int u = blockIdx.x;
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int C = p.C;
  const int chunk = p.chunk;  // entries per wave (a multiple of 16, <= 128)
  const int ncap = kW * chunk;

  __shared__ __attribute__((aligned(16))) float s_x[G][kCap];  // listed logits (log2 units, with the log-weight), then the weights
  __shared__ int s_cl[kCap];             // cluster of each entry, -1 if none
  __shared__ float s_cs[kW][kCmax][G];   // per wave: listed raw logits summed per cluster
  __shared__ int s_cn[kW][kCmax];        // per wave: listed rows per cluster
  __shared__ float s_wm[kW][G];          // per wave: maximum listed logit
  __shared__ float s_qk[kCmax][G];       // scale log2(e) <q_h, sumK_b>
  __shared__ float s_mu[kCmax][G];       // proxy mean logit (log2 units), -inf if no unread member
  __shared__ float s_pi[kCmax][G];       // mu_b + log2 n_b, -inf if none
  __shared__ float s_cb[kCmax][G];       // e^{mu_b - M}, zero past C
  __shared__ float s_M[G], s_Lt[G];
  __shared__ float s_L[kW][G];
  __shared__ __attribute__((aligned(16))) unsigned char s_pool[kPool];  // value tiles, then the waves' products

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

  // ---- key rows in the matrix-core operand layout (16 keys x 64 bytes a load);
  // tile t's registers take its value rows once its logits are formed --------
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = rows_of(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = rows_of(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);
  uint4 rg[kNT][4];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int off = vt[t] ? (int)(((int64_t)jt[t] * p.sn + 8 * sub) * 2) : kOOBL;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 64 * st, 0, kStreamNT);
      rg[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
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

  // ---- per tile: logits (d[i] = head 4 sub + i of key r16), then the tile's
  // value rows into the freed registers, then its cluster runs ----------------
  float bm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (16 * t >= chunk) break;  // uniform across the workgroup
    floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                  __builtin_bit_cast(bf16x8_t, rg[t][st]), d, 0, 0, 0);
    // value slot 4t + kq of row group sub = key 16t + 4kq + sub
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const int src = 4 * kq + sub;
      const int j = __shfl(jt[t], src, 64);
      const bool ok = __shfl(vt[t] ? 1 : 0, src, 64) != 0;
      const int off = ok ? (int)(((int64_t)j * p.sn + 8 * r16) * 2) : kOOBL;
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kStreamNT);
      rg[t][kq] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    const int e = w * chunk + 16 * t + r16;
    const int c = (vt[t] && ct[t] >= 0 && ct[t] < C) ? ct[t] : -1;
    const float lw = p.logw ? lwt[t] * kLog2e : 0.f;
    const int cprev = __builtin_amdgcn_update_dpp(0, c, 0x111, 0xF, 0xF, true);  // row_shr:1
    const int cnext = __builtin_amdgcn_update_dpp(0, c, 0x101, 0xF, 0xF, true);  // row_shl:1
    const int start = (r16 == 0 || c != cprev) ? 1 : 0;
    const bool last = r16 == 15 || c != cnext;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * sub + i;
      const float raw = d[i] * p.qscale;
      const float x = vt[t] ? raw + lw : kNegInf;
      if (h < G) {
        s_x[h][e] = x;
        bm[i] = fmaxf(bm[i], x);
      }
      const float rs = run_sum(c >= 0 ? raw : 0.f, start);
      if (h < G && last && c >= 0) __hip_atomic_fetch_add(&s_cs[w][c][h], rs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const int rn = run_count(c >= 0 ? 1 : 0, start);
    if (sub == 0) {
      s_cl[e] = c;
      if (last && c >= 0) __hip_atomic_fetch_add(&s_cn[w][c], rn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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

  // ---- weights in place of the logits, coefficients, the normaliser ----------
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
      s_x[h][e] = ex - corr;
    }
  }
  for (int i = tid; i < kCmax * G; i += 512) {
    const int b = i / G, h = i - b * G;
    const float M = s_M[h], mu = b < C ? s_mu[b][h] : kNegInf;
    s_cb[b][h] = (M == kNegInf || mu == kNegInf) ? 0.f : fast_exp2(mu - M);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = sum_rowgroups(sum16(lsum[h]));
    if (lane == 0) s_L[w][h] = v;
  }
  __syncthreads();
  if (tid < G) {
    const float M = s_M[tid];
    float Lh = 0.f;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) Lh += s_L[ww][tid];
    for (int b = 0; b < C; ++b) {
      const float pi = s_pi[b][tid];
      if (M != kNegInf && pi != kNegInf) Lh += fast_exp2(pi - M);
    }
    s_Lt[tid] = Lh;
  }

  // ---- the cluster terms sum_b e^{mu_b - M} sumV_b (fp32), sixteen clusters'
  // sums requested at once (past C: the last cluster's, times a zero) ---------
  float cterm[(G * kD + 511) / 512];
#pragma unroll
  for (int q = 0; q < (G * kD + 511) / 512; ++q) {
    const int i = tid + 512 * q;
    const int h = (i < G * kD ? i : 0) / kD, dim = i - (i / kD) * kD;
    const float* sv = p.sumV + (int64_t)u * C * kD + dim;
    float a = 0.f;
    for (int b0 = 0; b0 < C; b0 += 16) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = sv[(int64_t)min(b0 + k, C - 1) * kD];
#pragma unroll
      for (int k = 0; k < 16; ++k) a = fmaf(s_cb[b0 + k][h], v[k], a);
    }
    cterm[q] = i < G * kD ? a : 0.f;
  }

  // ---- weighted values on the matrix cores ------------------------------------
  floatx4_t oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  bf16_t* vtile = reinterpret_cast<bf16_t*>(s_pool + w * kTileBytes);
  const int hr = r16 < G ? r16 : (r16 < R2 ? r16 - G : 0);
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (16 * t >= chunk) break;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
      *reinterpret_cast<uint4*>(vtile + (4 * kq + sub) * kVRow + 8 * r16) = rg[t][kq];
    wave_lds_sync();  // the tile's rows, staged by other lanes
    // A: the weights of keys 16t + 4 sub + j; rows h take the high and middle
    // parts (K halves), rows G + h the remainder
    const float4 w4 = *reinterpret_cast<const float4*>(&s_x[hr][w * chunk + 16 * t + 4 * sub]);
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
      auto src = (__attribute__((address_space(3))) bf16x4_t*)(vtile + (4 * sub + (r16 >> 2)) * kVRow + 16 * nb +
                                                               4 * (r16 & 3));
      const bf16x4_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src);
      const bf16x8_t b = {b4[0], b4[1], b4[2], b4[3], b4[0], b4[1], b4[2], b4[3]};
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[nb], 0, 0, 0);
    }
  }

  // ---- the waves' products, then out = (products + cluster terms) / normaliser ---
  __syncthreads();  // every wave's tiles are consumed: the pool takes the products
  float* red = reinterpret_cast<float*>(s_pool);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * sub + i;
    if (r < R2) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) red[(w * R2 + r) * kD + 16 * nb + r16] = oacc[nb][i];
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
      for (int ww = 0; ww < kW; ++ww) a += red[(ww * R2 + h) * kD + dim] + red[(ww * R2 + G + h) * kD + dim];
      const float M = s_M[h], Lh = s_Lt[h];
      const int64_t qh = qrow0 + h;
      p.out[qh * kD + dim] = Lh > 0.f ? a / Lh : 0.f;
      if (dim == 0 && p.lse) p.lse[qh] = Lh > 0.f ? (M + __builtin_amdgcn_logf(Lh)) * kLn2 : kNegInf;
    }
  }
}

template <int G>
static hipError_t launch_long_g(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL((proxy_long_kernel<G>), dim3(p.B * p.Hkv), dim3(512), 0, st, p);
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
