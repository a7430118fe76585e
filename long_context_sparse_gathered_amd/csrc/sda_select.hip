// sda_select.hip -- the selector in front of the proxy decode ("OpenAttention:
// One Percent Is Enough with Tail Proxies", method stages 01-03 and the
// settings list): int8 key codes in an r = 32 query subspace (QGS), a read
// budget per cluster from the estimated weight error of its mean proxy
// (ErrorGate), and each cluster's best-scoring rows.
//
// Every step that decides an integer is fixed so that it is reproducible:
// projections are fp64 sums, in dimension order, of exact products (a bf16 or
// fp32 element times an fp32 basis entry); codes and query weights use IEEE
// division and round half to even; scores are exact integer dot products
// (v_dot4_i32_i8); a row's selection key orders by score, then by lower
// position, so the rows a cluster reads are unique.
#include <math.h>

#include "sda_device.hpp"
#include "sda_kernels.hpp"
#include "sda_select.hpp"

namespace sda {

// Wave reductions from register-to-register lane moves (no LDS round trips):
// DPP quad permutes and mirrors within each 16-lane row, then the row-swap
// instructions across rows. Each step combines a pair of lanes in both
// orders, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ int dpp_int(int v) {
  return (int)dpp_u32<CTRL>((uint32_t)v);
}
// Integer DPP move whose lanes with a source outside the row receive zero.
template <int CTRL>
__device__ __forceinline__ int dppz_int(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// (even-row value, odd-row value) for row pairs 0-1 and 2-3 (16-lane swap)
// or 0-2 and 1-3 (32-lane swap), the same on every lane of a pair.
template <bool S32>
__device__ __forceinline__ void row_pair_u32(uint32_t v, uint32_t& e, uint32_t& o) {
  if constexpr (S32) {
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    e = r[0];
    o = r[1];
  } else {
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    e = r[0];
    o = r[1];
  }
}
template <bool S32>
__device__ __forceinline__ void row_pair(double v, double& e, double& o) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  uint32_t el, ol, eh, oh;
  row_pair_u32<S32>((uint32_t)b, el, ol);
  row_pair_u32<S32>((uint32_t)(b >> 32), eh, oh);
  e = __longlong_as_double((long long)(((uint64_t)eh << 32) | el));
  o = __longlong_as_double((long long)(((uint64_t)oh << 32) | ol));
}
template <bool S32>
__device__ __forceinline__ void row_pair(int v, int& e, int& o) {
  uint32_t a, b;
  row_pair_u32<S32>((uint32_t)v, a, b);
  e = (int)a;
  o = (int)b;
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  if constexpr (sizeof(T) == 8) {
    v = op(v, dpp_f64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_f64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_f64<0x141>(v));  // row_half_mirror
    v = op(v, dpp_f64<0x140>(v));  // row_mirror
  } else {
    v = op(v, dpp_int<0xB1>(v));
    v = op(v, dpp_int<0x4E>(v));
    v = op(v, dpp_int<0x141>(v));
    v = op(v, dpp_int<0x140>(v));
  }
  T e, o;
  row_pair<false>(v, e, o);
  v = op(e, o);
  row_pair<true>(v, e, o);
  return op(e, o);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  return wave_reduce(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  return wave_reduce(v, [](int a, int b) { return a + b; });
}

// 16 bytes read once (non-temporal).
__device__ __forceinline__ uint4 load_nt_u4(const void* p) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ double wave_max_f64(double v) {
  return wave_reduce(v, [](double a, double b) { return fmax(a, b); });
}

// ---------------------------------------------------------------------------
// Build: projections y_j = U^T k_j and their int8 codes, in three launches:
// pass 1 (QUANT = false) writes each (unit, chunk)'s maxima of |y_i| and,
// when the workspace holds them, the projections themselves (fp64); a small
// kernel reduces the maxima to kmax_i per unit; pass 2 reads the kept
// projections (or recomputes them, bit for bit the same) and writes
// code_ji = rint(127 y_ji / kmax_i).  The basis sits in LDS in
// fp64; the chunk's keys pass through LDS 32 dimensions at a time (read from
// HBM once, coalesced).  A lane owns 4 rows x 8 coordinates (lane & 3 picks
// the coordinates), so every LDS read serves several products; each
// (row, coordinate) sum runs over d in order.
constexpr int kCodeDims = 32;   // key dimensions staged per step

template <typename T, bool QUANT>
__global__ __launch_bounds__(256) void qgs_code_kernel(const QgsBuildParams p) {
  __shared__ double s_u[kD * kQgsRank];
  __shared__ float s_k[kQgsRows][kCodeDims + 1];   // +1: the four rows of a lane group hit different banks
  __shared__ double s_max[4][kQgsRank];
  __shared__ double s_kmax[kQgsRank];
  const int u = blockIdx.x / p.chunks;
  const int ch = blockIdx.x - u * p.chunks;
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid & 3, rg = tid >> 2;    // coordinates 8cg..8cg+7, rows 4rg..4rg+3 of the chunk

  const float* Uu = p.U + (int64_t)u * kD * kQgsRank;
  if (!(QUANT && p.y))
    for (int i = tid; i < kD * kQgsRank; i += 256) s_u[i] = (double)Uu[i];
  if (QUANT && tid < kQgsRank) s_kmax[tid] = p.kmax[(int64_t)u * kQgsRank + tid];

  const int row0 = ch * kQgsRows;
  const int j0 = row0 + 4 * rg;
  const T* kbase = reinterpret_cast<const T*>(p.K) + (int64_t)s * p.sb + (int64_t)g * p.sh;
  double acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[r][i] = 0.0;
  if (QUANT && p.y) {
    // the projections pass 1 kept
    __syncthreads();  // s_kmax in place
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = min(j0 + r, p.n - 1);
      const double* yr = p.y + ((int64_t)u * p.n + j) * kQgsRank + 8 * cg;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[r][i] = __builtin_nontemporal_load(yr + i);
    }
  } else {
  for (int d0 = 0; d0 < kD; d0 += kCodeDims) {
    __syncthreads();   // the previous step's keys are consumed (and the basis is in place)
    // 256 rows x 32 dims: four lanes per row, 8 elements each, in 4 sweeps of 64 rows
#pragma unroll
    for (int sw = 0; sw < 4; ++sw) {
      const int rr = sw * 64 + (tid >> 2);
      const int part = tid & 3;
      const int j = min(row0 + rr, p.n - 1);
      RowChunk<T> c;
      c.load_cached(kbase + (int64_t)j * p.sn + d0 + 8 * part);
      float f[8];
      c.unpack(f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s_k[rr][8 * part + e] = f[e];
    }
    __syncthreads();
#pragma unroll 4
    for (int e = 0; e < kCodeDims; ++e) {
      const double* ur = &s_u[(d0 + e) * kQgsRank + 8 * cg];
      double uv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) uv[i] = ur[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double kd = (double)s_k[4 * rg + r][e];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] = fma(kd, uv[i], acc[r][i]);  // exact product: one rounding
      }
    }
  }
  }  // projections computed

  if constexpr (!QUANT) {
    if (p.y) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j0 + r >= p.n) break;
        double* yr = p.y + ((int64_t)u * p.n + j0 + r) * kQgsRank + 8 * cg;
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(acc[r][i], yr + i);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double v = 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) v = fmax(v, j0 + r < p.n ? fabs(acc[r][i]) : 0.0);
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) v = fmax(v, __shfl_xor(v, off, 64));
      if (lane < 4) s_max[w][8 * lane + i] = v;
    }
    __syncthreads();
    if (tid < kQgsRank) {
      const double m = fmax(fmax(s_max[0][tid], s_max[1][tid]), fmax(s_max[2][tid], s_max[3][tid]));
      p.part[((int64_t)u * p.chunks + ch) * kQgsRank + tid] = m;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (j0 + r >= p.n) break;
      uint32_t word[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double km = s_kmax[8 * cg + i];
        const int code = km > 0.0 ? (int)rint((acc[r][i] * 127.0) / km) : 0;
        word[i >> 2] |= ((uint32_t)code & 0xffu) << (8 * (i & 3));
      }
      *reinterpret_cast<uint2*>(p.codes + ((int64_t)u * p.n + j0 + r) * kQgsRank + 8 * cg) =
          make_uint2(word[0], word[1]);
    }
  }
}

// kmax_i of each unit: the maximum over its chunks.
__global__ __launch_bounds__(64) void qgs_kmax_kernel(const QgsBuildParams p) {
  const int u = blockIdx.x, i = threadIdx.x;
  if (i >= kQgsRank) return;
  double m = 0.0;
  for (int c = 0; c < p.chunks; ++c) m = fmax(m, p.part[((int64_t)u * p.chunks + c) * kQgsRank + i]);
  p.kmax[(int64_t)u * kQgsRank + i] = m;
}

hipError_t launch_qgs_build(const QgsBuildParams& p, int dtype, int units, hipStream_t st) {
  const dim3 grid(units * p.chunks), block(256);
  if (dtype == SDA_BF16) {
    hipLaunchKernelGGL((qgs_code_kernel<bf16_t, false>), grid, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((qgs_code_kernel<float, false>), grid, block, 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qgs_kmax_kernel, dim3(units), dim3(64), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == SDA_BF16) {
    hipLaunchKernelGGL((qgs_code_kernel<bf16_t, true>), grid, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((qgs_code_kernel<float, true>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per step, per unit, first part: the integer query weights, the clusters'
// weight errors and the budget of each cluster.
//
//   qt_h = U^T q_h (fp64, dimension order), w_hi = qt_hi * kmax_i,
//   wmax = max |w|, wq_hi = rint(127 w_hi / wmax)                (QGS)
//   zbar = scale <q_h, mu_b>, s2 = scale^2 sum_d q_hd^2 nu_bd,
//   e_hb = N_b e^{zbar} (e^{s2/2} - 1), Z_h = sum_b N_b e^{zbar + s2/2},
//   eps_b = sum_h e_hb / Z_h                                     (ErrorGate)
//   q_b: E split in proportion to eps_b by the largest remainder, capped at
//   the eligible rows A_b, capped clusters fixed and the rest split again;
//   with no error left anywhere the remaining capacity is the weight.
//
// The unit's query, basis and cluster sums are first staged in LDS with
// coalesced loads; the fp64 loops then read LDS only.
// Rows of the query and of the staged cluster sums in LDS: dims 0-63, four
// pad floats, dims 64-127 (and four spare), so that the lanes of a wave that
// read the same dim of different clusters, heads and 32-dim parts hit
// distinct banks.
constexpr int kPadRow = kD + 8;
static_assert(kD == 128, "the padded rows assume 128 dims");
__device__ __forceinline__ int pad_at(int d) { return d + ((d >> 6) << 2); }

struct PrepLds {
  float qf[kQgsMaxG][kPadRow];
  float u[kD * kQgsRank];
  double w[kQgsMaxG][kQgsRank];
  double top[kCmax][kQgsMaxG];
  double e[kCmax][kQgsMaxG];
  double s2[kCmax][kQgsMaxG];
  double M[kQgsMaxG], Z[kQgsMaxG];
  double eps[kCmax], frac[kCmax], wv[kCmax];
  double wmax;
  int loc[kCmax];
  int avail[kCmax];
  int cnt[kCmax];  // cluster sizes N_b
  // followed in LDS by the cluster sums: sumK [C][kPadRow], then sumK2 [C][kPadRow] (fp32)
};

__host__ __device__ inline size_t prep_lds_bytes(int C) {
  return (sizeof(PrepLds) + 15) / 16 * 16 + (size_t)2 * C * kPadRow * sizeof(float);
}

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float elem_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i].bits << 16);
}
template <>
__device__ __forceinline__ float elem_f32<float>(const float* p, int64_t i) {
  return p[i];
}

// wq_out [G][r/4] packed int8, budget_out / avail_out [C]: global or LDS.
// Ends with the budgets written by wave 0; the caller synchronises.
template <typename T>
__device__ void prep_unit(const QgsSelectParams& p, int u, PrepLds& L, float* sums, uint32_t* wq_out,
                          int* budget_out, int* avail_out) {
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int G = p.G, C = p.C;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const T* q = reinterpret_cast<const T*>(p.q) + ((int64_t)s * p.Hq + (int64_t)g * G) * kD;
  const double* km = p.kmax + (int64_t)u * kQgsRank;
  float* sk = sums;
  float* sk2 = sums + C * kPadRow;

  for (int t = tid; t < G * kD; t += nt) L.qf[t / kD][pad_at(t % kD)] = elem_f32<T>(q, t);
  {
    const float4* src = reinterpret_cast<const float4*>(p.U + (int64_t)u * kD * kQgsRank);
    for (int t = tid; t < kD * kQgsRank / 4; t += nt) reinterpret_cast<float4*>(L.u)[t] = src[t];
    const float4* s1 = reinterpret_cast<const float4*>(p.sumK + (int64_t)u * C * kD);
    const float4* s2 = reinterpret_cast<const float4*>(p.sumK2 + (int64_t)u * C * kD);
    for (int t = tid; t < C * kD / 4; t += nt) {
      const int c4 = t & 31, at = (t >> 5) * (kPadRow / 4) + c4 + (c4 >> 4);
      reinterpret_cast<float4*>(sk)[at] = s1[t];
      reinterpret_cast<float4*>(sk2)[at] = s2[t];
    }
  }
  for (int c = tid; c < C; c += nt) {
    L.loc[c] = 0;
    L.cnt[c] = p.count[(int64_t)u * C + c];
  }
  // cluster ids of the always-read sink and local window (counted below)
  const int32_t* cidu = p.cid + (int64_t)u * p.n;
  const int sink_end = min(p.n_sink, p.n);
  const int loc_begin = max(sink_end, p.n - p.n_local);
  const int nfix = sink_end + (p.n - loc_begin);
  int fixc[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int t = tid + k * nt;
    const int j = t < sink_end ? t : loc_begin + (t - sink_end);
    fixc[k] = t < nfix ? cidu[j] : -1;
  }
  __syncthreads();

  // query weights (unscaled) and the clusters' logit moments
  for (int t = tid; t < G * kQgsRank; t += nt) {
    const int h = t / kQgsRank, i = t - h * kQgsRank;
    double acc = 0.0;
    for (int d0 = 0; d0 < kD; d0 += 16) {
      float qv[16], uv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        qv[e] = L.qf[h][pad_at(d0) + e];
        uv[e] = L.u[(d0 + e) * kQgsRank + i];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) acc = fma((double)qv[e], (double)uv[e], acc);  // in dimension order
    }
    L.w[h][i] = acc * km[i];
  }
  // Logit moments: four lanes per (cluster, head), 32 dimensions each, the
  // partial sums added in a fixed order (every lane of the four ends with the
  // same bits).
  const double sc = (double)p.scale;
  for (int t0 = 0; t0 < C * G * 4; t0 += nt) {
    const int t = t0 + tid;
    const bool on = t < C * G * 4;
    const int pair = on ? t >> 2 : 0, part = t & 3;
    const int b = pair / G, h = pair - b * G;
    const int N = on ? L.cnt[b] : 0;
    const double inv = N > 0 ? 1.0 / (double)N : 0.0;
    double zb = 0.0, v2 = 0.0;
    if (N > 0) {
#pragma unroll 8
      for (int d = 32 * part; d < 32 * part + 32; ++d) {
        const double qd = (double)L.qf[h][pad_at(d)];
        const double mu = (double)sk[b * kPadRow + pad_at(d)] * inv;
        const double nu = fmax((double)sk2[b * kPadRow + pad_at(d)] * inv - mu * mu, 0.0);
        zb = fma(qd, mu, zb);
        v2 = fma(qd * qd, nu, v2);
      }
    }
    zb += __shfl_xor(zb, 1, 64);
    zb += __shfl_xor(zb, 2, 64);
    v2 += __shfl_xor(v2, 1, 64);
    v2 += __shfl_xor(v2, 2, 64);
    if (on && part == 0) {
      if (N > 0) {
        const double zbar = sc * zb;
        const double s2 = (sc * sc) * v2;
        const double lnN = log((double)N);
        L.top[b][h] = lnN + zbar + 0.5 * s2;
        L.e[b][h] = lnN + zbar;
        L.s2[b][h] = s2;
      } else {
        L.top[b][h] = -INFINITY;
        L.e[b][h] = -INFINITY;
        L.s2[b][h] = 0.0;
      }
    }
  }
  // members of each cluster inside the always-read sink and local window
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (fixc[k] >= 0 && fixc[k] < C) atomicAdd(&L.loc[fixc[k]], 1);
  for (int t = tid + 2 * nt; t < nfix; t += nt) {
    const int j = t < sink_end ? t : loc_begin + (t - sink_end);
    const int c = cidu[j];
    if (c >= 0 && c < C) atomicAdd(&L.loc[c], 1);
  }
  __syncthreads();
  // wave h < G: the head's largest cluster weight exponent M_h (lane b holds
  // cluster b); the last wave: the largest |w|
  {
    const int wv_ = tid >> 6, nw_ = nt >> 6;
    for (int h = wv_; h < G; h += nw_) {
      const double v = lane < C ? L.top[lane][h] : -INFINITY;
      const double M = wave_max_f64(v);
      if (lane == 0) L.M[h] = M;
    }
    if (wv_ == nw_ - 1) {
      double m = 0.0;
      for (int t = lane; t < G * kQgsRank; t += 64) m = fmax(m, fabs(L.w[t / kQgsRank][t % kQgsRank]));
      m = wave_max_f64(m);
      if (lane == 0) L.wmax = m;
    }
  }
  __syncthreads();
  // each cluster's estimated weight (over e^M) and proxy weight error, per head
  for (int t = tid; t < C * G; t += nt) {
    const int b = t / G, h = t - b * G;
    const double M = L.M[h];
    const bool live = L.top[b][h] != -INFINITY;
    L.top[b][h] = live ? exp(L.top[b][h] - M) : 0.0;
    L.e[b][h] = live ? exp(L.e[b][h] - M) * expm1(0.5 * L.s2[b][h]) : 0.0;
  }
  __syncthreads();
  for (int h = tid >> 6; h < G; h += nt >> 6) {
    const double Z = wave_sum_f64(lane < C ? L.top[lane][h] : 0.0);
    if (lane == 0) L.Z[h] = Z;
  }
  __syncthreads();
  for (int t = tid; t < G * kQgsRank / 4; t += nt) {
    const int h = t / (kQgsRank / 4), k = t - h * (kQgsRank / 4);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double wv = L.w[h][4 * k + e];
      const int v = L.wmax > 0.0 ? (int)rint((wv * 127.0) / L.wmax) : 0;
      word |= ((uint32_t)v & 0xffu) << (8 * e);
    }
    wq_out[h * (kQgsRank / 4) + k] = word;
  }
  if (tid < C) {
    const int N = L.cnt[tid];
    double eps = 0.0;
    if (N > 0) {
      for (int h = 0; h < G; ++h) eps += L.e[tid][h] / L.Z[h];
    }
    L.eps[tid] = eps;
    const int A = N - L.loc[tid];
    L.avail[tid] = A > 0 ? A : 0;
  }
  __syncthreads();

  // allocation, one wave: lane b owns cluster b
  if (tid < 64) {
    const bool has = lane < C;
    const double eb = has ? L.eps[lane] : 0.0;
    const int Ab = has ? L.avail[lane] : 0;
    bool fixed = !has || Ab <= 0;
    int qb = 0;
    const long long sumA = wave_sum_i32(Ab);
    int R = (int)min((long long)p.E, sumA);
    while (R > 0) {
      const bool act = !fixed;
      if (__ballot(act) == 0) break;
      const bool anypos = __ballot(act && eb > 0.0) != 0;
      const double wv = act ? (anypos ? eb : (double)Ab) : 0.0;
      const double tot = wave_sum_f64(wv);
      const double quota = act ? ((double)R * wv) / tot : 0.0;
      const double base = floor(quota);
      const double frac = quota - base;
      const int ib = (int)base;
      const int rem = R - wave_sum_i32(ib);
      const double fr = act ? frac : -1.0;
      // rank of this lane's remainder among the active ones (larger first,
      // ties to the lower cluster), from LDS broadcast reads
      L.frac[lane] = fr;
      wave_lds_sync();
      // (eight reads in flight, then branch-free compares; every lane wrote
      // its entry, -1 when inactive)
      int rank = 0;
#pragma unroll
      for (int b0 = 0; b0 < kCmax; b0 += 8) {
        if (b0 >= C) break;
        double f8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f8[k] = L.frac[b0 + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const double fb = f8[k];
          rank += (int)((fb >= 0.0) & ((fb > frac) | ((fb == frac) & (b0 + k < lane))));
        }
      }
      wave_lds_sync();
      const int tent = ib + ((act && rank < rem) ? 1 : 0);
      const bool over = act && tent > Ab;
      if (__ballot(over) == 0) {
        if (act) qb = tent;
        break;
      }
      const int capped = wave_sum_i32(over ? Ab : 0);
      if (over) {
        qb = Ab;
        fixed = true;
      }
      R -= capped;
    }
    if (has) {
      budget_out[lane] = qb;
      avail_out[lane] = Ab;
      if (p.budget) p.budget[(int64_t)u * C + lane] = qb;
    }
  }
}

// Standalone form (the three-launch path): results to the workspace.
template <typename T>
__global__ __launch_bounds__(256) void qgs_prep_kernel(const QgsSelectParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_prep[];
  PrepLds& L = *reinterpret_cast<PrepLds*>(s_prep);
  float* sums = reinterpret_cast<float*>(s_prep + (sizeof(PrepLds) + 15) / 16 * 16);
  const int u = blockIdx.x;
  prep_unit<T>(p, u, L, sums, p.wq + (int64_t)u * p.G * (kQgsRank / 4), p.wbudget + (int64_t)u * p.C,
               p.wavail + (int64_t)u * p.C);
}

// ---------------------------------------------------------------------------
// Score of one row: S_j = max over the group's heads of the int8 dot product
// of its 32 codes with the head's weights (eight v_dot4_i32_i8 per head).
template <int G>
__device__ __forceinline__ int qgs_score(const uint32_t (&wv)[G][kQgsRank / 4], const uint4 c0, const uint4 c1) {
  const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  int S = -(1 << 30);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    int dot = 0;
#pragma unroll
    for (int k = 0; k < kQgsRank / 4; ++k) dot = __builtin_amdgcn_sdot4((int)wv[h][k], (int)cw[k], dot, false);
    S = max(S, dot);
  }
  return S;
}

// ---------------------------------------------------------------------------
// Three-launch path, second part: every row's 64-bit selection key.  Four
// rows per thread.
constexpr int kScoreRows = 1024;

template <int G>
__global__ __launch_bounds__(256) void qgs_score_kernel(const QgsSelectParams p) {
  const int chunks = (p.n + kScoreRows - 1) / kScoreRows;
  const int u = blockIdx.x / chunks;
  const int ch = blockIdx.x - u * chunks;
  uint32_t wv[G][kQgsRank / 4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < kQgsRank / 4; ++k) wv[h][k] = p.wq[((int64_t)u * G + h) * (kQgsRank / 4) + k];
  const int lo = p.n_sink, hi = p.n - p.n_local;
  bool bad = false;
#pragma unroll
  for (int rr = 0; rr < kScoreRows / 256; ++rr) {
    const int j = ch * kScoreRows + rr * 256 + threadIdx.x;
    if (j >= p.n) break;
    const int64_t row = (int64_t)u * p.n + j;
    const uint4* cp = reinterpret_cast<const uint4*>(p.codes + row * kQgsRank);
    const int S = qgs_score<G>(wv, cp[0], cp[1]);
    const int c = p.cid[row];
    if (c < -1 || c >= p.C) bad = true;
    const int cl = (c >= 0 && c < p.C) ? c : kNoCluster;
    const bool el = cl != kNoCluster && j >= lo && j < hi;
    const uint64_t key = (el ? (1ull << 47) : 0ull) | ((uint64_t)cl << kKeyBits) |
                         ((uint64_t)(uint32_t)(S + (1 << 19)) << 20) | (uint64_t)(kQgsMaxN - 1 - j);
    p.keys[row] = key;
  }
  if (bad) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
}

// ---------------------------------------------------------------------------
// Per-cluster radix select over 40-bit keys (score, then lower position):
// 7-bit digits from the top, one LDS histogram per cluster; a cluster is done
// once the boundary digit holds exactly the rows it still needs, and its
// threshold T_b is then the q_b-th largest key's prefix (every key of the
// cluster >= T_b is listed).
struct SelState {
  uint64_t pref[kCmax];
  uint64_t T[kCmax];
  int need[kCmax];
  int done[kCmax];
  int left;
  int cnt[16];
};

__device__ __forceinline__ void sel_init(SelState& S, const int* budget, const int* avail, int C) {
  const int tid = threadIdx.x;
  if (tid < C) {
    const int qb = budget[tid];
    const int Ab = avail[tid];
    S.pref[tid] = 0;
    S.need[tid] = qb;
    if (qb <= 0) {
      S.done[tid] = 1;
      S.T[tid] = 1ull << kKeyBits;  // above every key: nothing
    } else if (qb >= Ab) {
      S.done[tid] = 1;
      S.T[tid] = 0;                 // every eligible row
    } else {
      S.done[tid] = 0;
      S.T[tid] = 0;
    }
  }
}

// One pass's resolution, after its histograms are complete.
// Histograms hold nb = 2^W bins per cluster (W = 7 or 6).
__device__ __forceinline__ void sel_resolve(SelState& S, const int* hist, int C, int shift, int nb = 128) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  for (int c = w; c < C; c += nw) {
    if (S.done[c]) continue;
    const int need = S.need[c];
    const int chi = 2 * lane + 1 < nb ? hist[c * nb + 2 * lane + 1] : 0;
    const int clo = 2 * lane < nb ? hist[c * nb + 2 * lane] : 0;
    const int pair = chi + clo;
    // rows in this lane's bins and every higher bin: a suffix scan within
    // each 16-lane row (DPP shifts toward lower lanes, zero past the row),
    // then the totals of the rows above, read from their first lanes
    int incl = pair;
    incl += dppz_int<0x101>(incl);  // row_shl:1
    incl += dppz_int<0x102>(incl);  // row_shl:2
    incl += dppz_int<0x104>(incl);  // row_shl:4
    incl += dppz_int<0x108>(incl);  // row_shl:8
    {
      const int t1 = __builtin_amdgcn_readlane(incl, 16), t2 = __builtin_amdgcn_readlane(incl, 32),
                t3 = __builtin_amdgcn_readlane(incl, 48);
      const int row = lane >> 4;
      incl += (row < 1 ? t1 : 0) + (row < 2 ? t2 : 0) + (row < 3 ? t3 : 0);
    }
    const int excl = incl - pair;
    int t = -1, above = 0;
    if (excl < need && excl + chi >= need) {
      t = 2 * lane + 1;
      above = excl;
    } else if (excl + chi < need && incl >= need) {
      t = 2 * lane;
      above = excl + chi;
    }
    const uint64_t hit = __ballot(t >= 0);
    if (hit == 0) {
      // fewer candidates than the budget (counts that disagree with the
      // cluster ids): list every candidate
      if (lane == 0) {
        S.T[c] = S.pref[c];
        S.done[c] = 1;
      }
      continue;
    }
    const int src = __builtin_ctzll(hit);
    const int tb = __builtin_amdgcn_readlane(t, src);
    const int ab = __builtin_amdgcn_readlane(above, src);
    if (lane == 0) {
      const int rest = need - ab;
      const uint64_t pref = S.pref[c] | ((uint64_t)tb << shift);
      S.pref[c] = pref;
      S.need[c] = rest;
      if (hist[c * nb + tb] == rest) {
        S.T[c] = pref;
        S.done[c] = 1;
      }
    }
  }
}

// Pass p of a W-bit radix select covers key bits [shift, top), top = 40 - W p.
__device__ __forceinline__ void pass_digits(int pass, int& top, int& shift, int& width, int W = 7) {
  top = kKeyBits - W * pass;
  shift = top > W ? top - W : 0;
  width = top - shift;
}

// Listed rows in position order: per-wave counts, then ballot compaction.
// key_of(j) gives (eligible, cluster, 40-bit key) of row j.  Eight rows per
// lane per step, read before any is used (straight-line code).
template <typename KeyOf>
__device__ void emit_listed(const QgsSelectParams& p, int u, SelState& S, KeyOf key_of) {
  const int n = p.n, C = p.C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  const int lo = p.n_sink, hi = p.n - p.n_local;
  const int span = ((n + nw - 1) / nw + 63) / 64 * 64;
  const int r0 = w * span, r1 = min(n, r0 + span);
  auto flags8 = [&](int j0, bool (&on)[8], int (&cl)[8]) {
    bool el[8];
    uint64_t k40[8], T[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) key_of(min(j0 + 64 * k + lane, r1 - 1), el[k], cl[k], k40[k]);
#pragma unroll
    for (int k = 0; k < 8; ++k) T[k] = S.T[cl[k] < C ? cl[k] : 0];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + 64 * k + lane;
      on[k] = (j < r1) & ((j < lo) | (j >= hi) | (el[k] & (cl[k] < C) & (k40[k] >= T[k])));
    }
  };
  int cnt = 0;
  for (int j0 = r0; j0 < r1; j0 += 512) {
    bool on[8];
    int cl[8];
    flags8(j0, on, cl);
#pragma unroll
    for (int k = 0; k < 8; ++k) cnt += __popcll(__ballot(on[k]));
  }
  if (lane == 0) S.cnt[w] = cnt;
  __syncthreads();
  int base = 0, total = 0;
  for (int ww = 0; ww < nw; ++ww) {
    if (ww < w) base += S.cnt[ww];
    total += S.cnt[ww];
  }
  int32_t* idx = p.idx + (int64_t)u * p.m;
  int32_t* icl = p.idx_cluster + (int64_t)u * p.m;
  for (int j0 = r0; j0 < r1; j0 += 512) {
    bool on[8];
    int cl[8];
    flags8(j0, on, cl);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t bal = __ballot(on[k]);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (on[k] && pos < p.m) {
        idx[pos] = j0 + 64 * k + lane;
        icl[pos] = cl[k] == kNoCluster ? -1 : cl[k];
      }
      base += __popcll(bal);
    }
  }
  for (int pos = total + tid; pos < p.m; pos += blockDim.x) {
    idx[pos] = 0;
    icl[pos] = -1;
  }
  if (tid == 0) {
    p.idx_len[u] = min(total, p.m);
    if (total > p.m) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  }
}

// Three-launch path, third part: one workgroup per unit over the keys in the
// workspace.
constexpr int kSelThreads = 512;

__global__ __launch_bounds__(kSelThreads) void qgs_select_kernel(const QgsSelectParams p) {
  __shared__ int s_hist[kCmax * 128];
  __shared__ SelState S;
  const int u = blockIdx.x;
  const int n = p.n, C = p.C;
  const int tid = threadIdx.x;
  const uint64_t* keys = p.keys + (int64_t)u * n;

  sel_init(S, p.wbudget + (int64_t)u * C, p.wavail + (int64_t)u * C, C);
  __syncthreads();
  for (int pass = 0; pass < 6; ++pass) {
    int top, shift, width;
    pass_digits(pass, top, shift, width);
    if (tid < 64) {
      const int left = __popcll(__ballot(tid < C && !S.done[tid]));
      if (tid == 0) S.left = left;
    }
    for (int i = tid; i < C * 128; i += kSelThreads) s_hist[i] = 0;
    __syncthreads();
    if (S.left == 0) break;
    for (int j0 = 0; j0 < n; j0 += 8 * kSelThreads) {
      uint64_t kk[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = j0 + r * kSelThreads + tid;
        kk[r] = j < n ? keys[j] : 0ull;
      }
      int dn[8];
      uint64_t pf[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int c = (int)((kk[r] >> kKeyBits) & 127);
        const int cs = c < C ? c : 0;
        dn[r] = S.done[cs];
        pf[r] = S.pref[cs];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint64_t key = kk[r];
        const int c = (int)((key >> kKeyBits) & 127);
        const uint64_t k40 = key & kKeyMask;
        const bool hit = ((key >> 47) & 1) & (c < C) & (dn[r] == 0) & ((k40 >> top) == (pf[r] >> top));
        if (hit) atomicAdd(&s_hist[c * 128 + (int)((k40 >> shift) & ((1u << width) - 1))], 1);
      }
    }
    __syncthreads();
    sel_resolve(S, s_hist, C, shift);
    __syncthreads();
  }
  emit_listed(p, u, S, [&](int j, bool& el, int& c, uint64_t& k40) {
    const uint64_t key = keys[j];
    el = (key >> 47) & 1;
    c = (int)((key >> kKeyBits) & 127);
    k40 = key & kKeyMask;
  });
}

// ---------------------------------------------------------------------------
// One-launch path (n <= 32768, C <= 32): one workgroup per unit does the
// first part, scores every row straight from its codes into a 4-byte LDS
// record (eligible, cluster, score) while building the first histogram, then
// selects and lists from LDS.  HBM traffic: the codes and cluster ids once.
//   record: [19:0] S + 2^19, [26:20] cluster (127 = none), [27] eligible
constexpr int kFusedMaxN = 32768;
constexpr int kFusedMaxC = kCmax;

constexpr int kFusedSel = 1024;    // picked rows collected in LDS before they are ordered
constexpr int kFusedCand = 1024;   // rows on a pending cluster's boundary after two digits

struct FusedState {
  SelState sel;
  uint32_t wq[kQgsMaxG][kQgsRank / 4];
  int budget[kCmax];
  int avail[kCmax];
  int match[kCmax];
  int2 thr[kCmax];  // (score threshold of a pick, boundary prefix of a candidate)
  int nsel, ncand;
  int picked[kFusedSel];
  int cand[kFusedCand];
};

// LDS layout: [0, big) records or (first part) PrepLds + sums; then the
// histograms [C][128]; then FusedState.
__host__ __device__ inline size_t fused_big(int n, int C) {
  const size_t rec = (size_t)n * 4;
  const size_t prep = prep_lds_bytes(C);
  return ((rec > prep ? rec : prep) + 15) / 16 * 16;
}
__host__ __device__ inline size_t fused_lds_bytes(int n, int C) {
  return fused_big(n, C) + (size_t)C * (C <= 32 ? 128 : 64) * 4 + sizeof(FusedState);
}

__device__ __forceinline__ uint64_t rec_key(uint32_t r, int j) {
  return ((uint64_t)(r & 0xfffffu) << 20) | (uint64_t)(kQgsMaxN - 1 - j);
}

template <typename T, int G>
__global__ __launch_bounds__(kSelThreads) void qgs_fused_kernel(const QgsSelectParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
  const int n = p.n, C = p.C;
  const size_t big = fused_big(n, C);
  uint32_t* rec = reinterpret_cast<uint32_t*>(s_raw);
  int* hist = reinterpret_cast<int*>(s_raw + big);
  // digits of W bits: 7 up to 32 clusters, 6 up to 64 (histograms C x 2^W)
  const int W = C <= 32 ? 7 : 6, NB = 1 << W;
  FusedState& F = *reinterpret_cast<FusedState*>(s_raw + big + (size_t)C * NB * 4);
  SelState& S = F.sel;
  const int u = blockIdx.x;
  const int tid = threadIdx.x;

  {
    PrepLds& L = *reinterpret_cast<PrepLds*>(s_raw);
    float* sums = reinterpret_cast<float*>(s_raw + (sizeof(PrepLds) + 15) / 16 * 16);
    prep_unit<T>(p, u, L, sums, &F.wq[0][0], F.budget, F.avail);
  }
  __syncthreads();
  sel_init(S, F.budget, F.avail, C);
  for (int i = tid; i < C * NB; i += kSelThreads) hist[i] = 0;
  __syncthreads();

  // scores, records and the first digit's histograms
  uint32_t wv[G][kQgsRank / 4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < kQgsRank / 4; ++k) wv[h][k] = F.wq[h][k];
  const int lo = p.n_sink, hi = p.n - p.n_local;
  const int8_t* codes = p.codes + (int64_t)u * n * kQgsRank;
  const int32_t* cid = p.cid + (int64_t)u * n;
  bool bad = false;
  constexpr int RB = 8;  // rows in flight per thread
  for (int j0 = 0; j0 < n; j0 += RB * kSelThreads) {
    uint4 c0[RB], c1[RB];
    int cc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int j = min(j0 + r * kSelThreads + tid, n - 1);
      const uint4* cp = reinterpret_cast<const uint4*>(codes + (int64_t)j * kQgsRank);
      c0[r] = load_nt_u4(cp);
      c1[r] = load_nt_u4(cp + 1);
      cc[r] = __builtin_nontemporal_load(cid + j);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int j = j0 + r * kSelThreads + tid;
      if (j >= n) continue;
      const int Sc = qgs_score<G>(wv, c0[r], c1[r]);
      const int c = cc[r];
      if (c < -1 || c >= C) bad = true;
      const int cl = (c >= 0 && c < C) ? c : kNoCluster;
      const bool el = cl != kNoCluster && j >= lo && j < hi;
      const uint32_t s20 = (uint32_t)(Sc + (1 << 19));
      rec[j] = (el ? (1u << 27) : 0u) | ((uint32_t)cl << 20) | s20;
      if (el && !S.done[cl]) atomicAdd(&hist[cl * NB + (int)(s20 >> (20 - W))], 1);
    }
  }
  if (bad) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  __syncthreads();

  // pass 0: its histograms came with the scores (key bits [40 - W, 40) = S20 >> (20 - W))
  sel_resolve(S, hist, C, kKeyBits - W, NB);
  __syncthreads();

  // pass 1: key bits [40 - 2W, 40 - W) = (S20 >> (20 - 2W)) & (NB - 1) of the
  // rows in each pending cluster's boundary digit; 32-bit arithmetic on the
  // records
  if (tid < C) F.match[tid] = S.done[tid] ? -1 : (int)(S.pref[tid] >> (kKeyBits - W));
  for (int i = tid; i < C * NB; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  for (int j0 = tid; j0 < n; j0 += 8 * kSelThreads) {
    uint32_t rr[8];
    int mt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rr[k] = rec[min(j0 + k * kSelThreads, n - 1)];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = (int)((rr[k] >> 20) & 127);
      mt[k] = F.match[c < C ? c : 0];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t r = rr[k], s20 = r & 0xfffffu;
      const bool hit = (j0 + k * kSelThreads < n) & ((r >> 27) & 1) & ((int)(s20 >> (20 - W)) == mt[k]);
      if (hit) atomicAdd(&hist[(int)((r >> 20) & 127) * NB + (int)((s20 >> (20 - 2 * W)) & (NB - 1))], 1);
    }
  }
  __syncthreads();
  sel_resolve(S, hist, C, kKeyBits - 2 * W, NB);
  __syncthreads();

  // Classify the rows between sink and local window once: a row of a done
  // cluster is picked when S20 >= A_c (its threshold's score part; those
  // thresholds have zero position bits); for a pending cluster, a row above
  // its boundary (S20 >> (20 - 2W) > P_c) is picked and a row on it (== P_c)
  // is a candidate for the remaining digits.
  const int lane = tid & 63, w = tid >> 6;
  if (tid < C) {
    if (S.done[tid]) {
      F.thr[tid] = make_int2((int)(S.T[tid] >> 20), -1);
    } else {
      const int P = (int)(S.pref[tid] >> (kKeyBits - 2 * W));
      F.thr[tid] = make_int2((P + 1) << (20 - 2 * W), P);
    }
  }
  if (tid == 0) {
    F.nsel = 0;
    F.ncand = 0;
  }
  __syncthreads();
  auto push = [&](bool on, int* cnt, int* list, int cap, int j) {
    const uint64_t bal = __ballot(on);
    if (bal) {
      int base = 0;
      if (lane == 0) base = atomicAdd(cnt, __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (on && pos < cap) list[pos] = j;
    }
  };
  {
    const int mid = max(0, hi - lo);
    const int span = ((mid + 7) / 8 + 63) / 64 * 64;
    const int r0 = lo + w * span, r1 = min(hi, r0 + span);
    for (int j0 = r0; j0 < r1; j0 += 512) {
      uint32_t rr[8];
      int ta[8], tb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) rr[k] = rec[min(j0 + 64 * k + lane, r1 - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = (int)((rr[k] >> 20) & 127);
        const int2 th = F.thr[c < C ? c : 0];
        ta[k] = th.x;
        tb[k] = th.y;
      }
      // all eight rows' decisions, then one reservation per list for the
      // step (a reservation is an LDS round trip); rows are written only
      // for the ballots that hold any
      uint64_t bp[8], bc[8];
      int np = 0, nc = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = j0 + 64 * k + lane;
        const int s20 = (int)(rr[k] & 0xfffffu);
        const bool el = (j < r1) & ((rr[k] >> 27) & 1);
        bp[k] = __ballot(el & (s20 >= ta[k]));
        bc[k] = __ballot(el & ((s20 >> (20 - 2 * W)) == tb[k]));
        np += __popcll(bp[k]);
        nc += __popcll(bc[k]);
      }
      if (np + nc > 0) {
        int basep = 0, basec = 0;
        if (lane == 0) {
          if (np) basep = atomicAdd(&F.nsel, np);
          if (nc) basec = atomicAdd(&F.ncand, nc);
        }
        basep = __builtin_amdgcn_readfirstlane(basep);
        basec = __builtin_amdgcn_readfirstlane(basec);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = j0 + 64 * k + lane;
          if (bp[k]) {
            const int pos = basep + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bp[k] >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bp[k], 0));
            if (((bp[k] >> lane) & 1) && pos < kFusedSel) F.picked[pos] = j;
            basep += __popcll(bp[k]);
          }
          if (bc[k]) {
            const int pos = basec + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bc[k] >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bc[k], 0));
            if (((bc[k] >> lane) & 1) && pos < kFusedCand) F.cand[pos] = j;
            basec += __popcll(bc[k]);
          }
        }
      }
    }
  }
  __syncthreads();

  if (F.ncand > kFusedCand || F.nsel > kFusedSel) {
    // too many rows for the LDS lists: the remaining digits over all rows,
    // then the ordered emission by scans
    for (int pass = 2; pass * W < kKeyBits; ++pass) {
      int top, shift, width;
      pass_digits(pass, top, shift, width, W);
      if (tid < 64) {
        const int left = __popcll(__ballot(tid < C && !S.done[tid]));
        if (tid == 0) S.left = left;
      }
      for (int i = tid; i < C * NB; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      if (S.left == 0) break;
      for (int j = tid; j < n; j += kSelThreads) {
        const uint32_t r = rec[j];
        const int c = (int)((r >> 20) & 127);
        const uint64_t k40 = rec_key(r, j);
        const bool hit = ((r >> 27) & 1) && !S.done[c] && (k40 >> top) == (S.pref[c] >> top);
        if (hit) atomicAdd(&hist[c * NB + (int)((k40 >> shift) & ((1u << width) - 1))], 1);
      }
      __syncthreads();
      sel_resolve(S, hist, C, shift, NB);
      __syncthreads();
    }
    emit_listed(p, u, S, [&](int j, bool& el, int& c, uint64_t& k40) {
      const uint32_t r = rec[j];
      el = (r >> 27) & 1;
      c = (int)((r >> 20) & 127);
      k40 = rec_key(r, j);
    });
    return;
  }

  // the remaining digits over the candidates only
  const int ncand = F.ncand;
  for (int pass = 2; pass * W < kKeyBits; ++pass) {
    int top, shift, width;
    pass_digits(pass, top, shift, width, W);
    if (tid < 64) {
      const int left = __popcll(__ballot(tid < C && !S.done[tid]));
      if (tid == 0) S.left = left;
    }
    for (int i = tid; i < C * NB; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    if (S.left == 0) break;
    for (int t = tid; t < ncand; t += kSelThreads) {
      const int j = F.cand[t];
      const uint32_t r = rec[j];
      const int c = (int)((r >> 20) & 127);
      const uint64_t k40 = rec_key(r, j);
      if (!S.done[c] && (k40 >> top) == (S.pref[c] >> top))
        atomicAdd(&hist[c * NB + (int)((k40 >> shift) & ((1u << width) - 1))], 1);
    }
    __syncthreads();
    sel_resolve(S, hist, C, shift, NB);
    __syncthreads();
  }
  for (int t0 = 0; t0 < ncand; t0 += kSelThreads) {
    const int t = t0 + tid;
    int j = 0;
    bool on = false;
    if (t < ncand) {
      j = F.cand[t];
      const uint32_t r = rec[j];
      const int c = (int)((r >> 20) & 127);
      on = rec_key(r, j) >= S.T[c];
    }
    push(on, &F.nsel, F.picked, kFusedSel, j);
  }
  __syncthreads();
  const int nsel = F.nsel;
  if (nsel > kFusedSel) {
    emit_listed(p, u, S, [&](int j, bool& el, int& c, uint64_t& k40) {
      const uint32_t r = rec[j];
      el = (r >> 27) & 1;
      c = (int)((r >> 20) & 127);
      k40 = rec_key(r, j);
    });
    return;
  }

  // The listed rows are the sink, the picked rows (all inside
  // [n_sink, n - n_local)) and the local window, in that position order:
  // each picked row goes to its rank among the picked.
  const int sink_end = min(lo, n);
  const int loc_begin = max(sink_end, hi);
  const int total = sink_end + nsel + (n - loc_begin);
  int32_t* idx = p.idx + (int64_t)u * p.m;
  int32_t* icl = p.idx_cluster + (int64_t)u * p.m;
  auto put = [&](int pos, int j) {
    if (pos < p.m) {
      const int c = (int)((rec[j] >> 20) & 127);
      idx[pos] = j;
      icl[pos] = c == kNoCluster ? -1 : c;
    }
  };
  for (int t = tid; t < sink_end; t += kSelThreads) put(t, t);
  for (int t = tid; t < n - loc_begin; t += kSelThreads) put(sink_end + nsel + t, loc_begin + t);
  for (int t = tid; t < nsel; t += kSelThreads) {
    const int j = F.picked[t];
    int rank = 0;
    for (int k = 0; k < nsel; ++k) rank += F.picked[k] < j ? 1 : 0;
    put(sink_end + rank, j);
  }
  for (int pos = total + tid; pos < p.m; pos += kSelThreads) {
    idx[pos] = 0;
    icl[pos] = -1;
  }
  if (tid == 0) {
    p.idx_len[u] = min(total, p.m);
    if (total > p.m) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  }
}

template <int G>
static hipError_t launch_score_g(const QgsSelectParams& p, int units, hipStream_t st) {
  const int chunks = (p.n + kScoreRows - 1) / kScoreRows;
  hipLaunchKernelGGL(qgs_score_kernel<G>, dim3(units * chunks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_fused_g(const QgsSelectParams& p, int units, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((qgs_fused_kernel<T, G>), dim3(units), dim3(kSelThreads), lds, st, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fused_t(const QgsSelectParams& p, int units, size_t lds, hipStream_t st) {
  switch (p.G) {
    case 1: return launch_fused_g<T, 1>(p, units, lds, st);
    case 2: return launch_fused_g<T, 2>(p, units, lds, st);
    case 4: return launch_fused_g<T, 4>(p, units, lds, st);
    case 8: return launch_fused_g<T, 8>(p, units, lds, st);
  }
  return hipErrorInvalidValue;
}

bool qgs_select_one_launch(int n, int C) {
  return n <= kFusedMaxN && C <= kFusedMaxC && fused_lds_bytes(n, C) <= 160 * 1024;
}

hipError_t launch_qgs_select(const QgsSelectParams& p, int dtype, hipStream_t st) {
  const int units = p.B * p.Hkv;
  if (qgs_select_one_launch(p.n, p.C)) {
    const size_t lds = fused_lds_bytes(p.n, p.C);
    return dtype == SDA_BF16 ? launch_fused_t<bf16_t>(p, units, lds, st) : launch_fused_t<float>(p, units, lds, st);
  }
  const size_t plds = prep_lds_bytes(p.C);
  if (dtype == SDA_BF16) {
    hipLaunchKernelGGL(qgs_prep_kernel<bf16_t>, dim3(units), dim3(256), plds, st, p);
  } else {
    hipLaunchKernelGGL(qgs_prep_kernel<float>, dim3(units), dim3(256), plds, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.G) {
    case 1: e = launch_score_g<1>(p, units, st); break;
    case 2: e = launch_score_g<2>(p, units, st); break;
    case 4: e = launch_score_g<4>(p, units, st); break;
    case 8: e = launch_score_g<8>(p, units, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qgs_select_kernel, dim3(units), dim3(kSelThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sda
