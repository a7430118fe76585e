// sda_sampled.hip -- sparse decode attention with a sampled tail
// ("vAttention: Verified Sparse Attention via Sampling", method sections
// 1-3): the deterministic set I_f is read exactly, the unread rows are
// sampled uniformly with replacement, each sample weighted n_s / b (eq. 3),
// and the budget b comes from the CLT sample-size lemma applied to the
// numerator and the denominator (b = max(b_N, b_D), Lemma 4.2), with the
// statistics estimated from b0 base draws.
//
// Three launches per call:
//   sampled_stats_kernel  one workgroup per (sequence, KV head): I_f and the
//                         base draws in fp64, the budget b; leaves M, D_f,
//                         N_f and b in the workspace.
//   sampled_draws_kernel  `splits` workgroups per unit share the b fresh
//                         draws: each generates its draws' positions, gathers
//                         the rows and keeps an fp32 online softmax.
//   sampled_merge_kernel  one workgroup per unit: log-sum-exp merge of the
//                         draw partials, then num = N_f + (n_s/b) N_dyn and
//                         den = D_f + (n_s/b) D_dyn in fp64.
// Everything the budget depends on -- logits, weights, sums, variances -- is
// fp64, so the integer budget matches an fp64 reference up to the summation
// order.  The fresh draws feed only the output.
//
// Draw k of unit u: x = output k of SplitMix64 seeded with key_u, where
// key_u = output u of SplitMix64 seeded with `seed` (SplitMix64: the state
// advances by 0x9E3779B97F4A7C15 and each output is the state through the
// published 64-bit finaliser; Steele, Lea & Flood, OOPSLA 2014).  The draw
// picks unread rank floor(x * n_s / 2^64), and rank r maps to the position
// r + #{i : I_f[i] - i <= r} (binary search).
#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

namespace {

constexpr int kW = 8;  // waves per workgroup
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int kOOBs = kMaxUnitBytes;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// output k (0-based) of SplitMix64 seeded with `seed`
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t k) { return mix64(seed + (k + 1) * kGamma); }

// rank -> position over the sorted, distinct list held as A[i] = I_f[i] - i
__device__ __forceinline__ int tail_position(const int* A, int mf, int64_t rank) {
  int lo = 0, hi = mf;  // count of A[i] <= rank
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)A[mid] <= rank) lo = mid + 1; else hi = mid;
  }
  return (int)(rank + lo);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// sum over the 16 lanes of a row group, identical bits on every lane
__device__ __forceinline__ double sum16_d(double v) {
  v += dpp_d<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_d<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_d<0x141>(v);  // row_half_mirror
  v += dpp_d<0x140>(v);  // row_mirror
  return v;
}

// (even-row value, odd-row value) of a 16- or 32-lane row exchange
struct RowPairD {
  double even, odd;
};
template <bool R32>
__device__ __forceinline__ RowPairD swap_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  auto rl = R32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto rh = R32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  return {__builtin_bit_cast(double, ((uint64_t)rh[0] << 32) | rl[0]),
          __builtin_bit_cast(double, ((uint64_t)rh[1] << 32) | rl[1])};
}

// sum over the four row groups, identical bits on every lane
__device__ __forceinline__ double sum_rowgroups_d(double v) {
  const RowPairD a = swap_d<false>(v);
  v = a.even + a.odd;
  const RowPairD b = swap_d<true>(v);
  return b.even + b.odd;
}

// exp(m - M), 0 for an empty partial (m = -inf)
__device__ __forceinline__ double rescale_d(double m, double M) {
  return m == -__builtin_huge_val() ? 0.0 : exp(m - M);
}

// lane H's value, broadcast to the 16 lanes of each row group (row_newbcast)
template <int H>
__device__ __forceinline__ double row_bcast_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x150 + H, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x150 + H, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double row_bcast(double v, int h) {  // h folds to a constant when unrolled
  switch (h) {
    case 0: return row_bcast_d<0>(v);
    case 1: return row_bcast_d<1>(v);
    case 2: return row_bcast_d<2>(v);
    case 3: return row_bcast_d<3>(v);
    case 4: return row_bcast_d<4>(v);
    case 5: return row_bcast_d<5>(v);
    case 6: return row_bcast_d<6>(v);
    default: return row_bcast_d<7>(v);
  }
}

template <typename T>
__device__ __forceinline__ void widen8(const RowChunk<T>& c, double (&d)[8]) {
  float f[8];
  c.unpack(f);
#pragma unroll
  for (int i = 0; i < 8; ++i) d[i] = (double)f[i];
}

using rsrc_t = __amdgpu_buffer_rsrc_t;

template <typename T>
__device__ __forceinline__ rsrc_t rsrc_of(const void* base, int64_t n, int64_t sn) {
  const int64_t bytes = ((int64_t)(n - 1) * sn + kD) * (int64_t)sizeof(T);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void gather(RowChunk<bf16_t>& c, rsrc_t r, int off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  c.raw = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void gather(RowChunk<float>& c, rsrc_t r, int off) {
  auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
  c.a = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
  c.b = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
}

template <typename T>
__device__ __forceinline__ int off_of(int j, int64_t sn, int r16) {
  return (int)(((int64_t)j * sn + 8 * r16) * (int64_t)sizeof(T));
}

// CLT budget of one head from its statistics (the same formula the fp64
// reference uses; contraction off so that every product rounds on its own).
__device__ double budget_of(double z, double eps, double n_s, double varD, double Dhat, double trN,
                            double normN) {
#pragma clang fp contract(off)
  double bD = 0.0, bN = 0.0;
  if (varD > 0.0) {
    const double t = z * n_s * sqrt(varD) / (eps * Dhat);
    bD = t * t;
  }
  if (trN > 0.0) {
    if (normN > 0.0) {
      const double t = z * n_s * sqrt(trN) / (eps * normN);
      bN = t * t;
    } else {
      bN = __builtin_huge_val();
    }
  }
  return bD > bN ? bD : bN;
}

}  // namespace

// Exact part over a share of I_f: rows [c*per, min(mf, (c+1)*per)) of unit u
// for workgroup (u, c), an fp64 online softmax per row group (keys and values
// read together), merged into one record (m, D, N) per head relative to m.
template <typename T, int G>
__global__ __launch_bounds__(512) void sampled_exact_kernel(const AttnParams p) {
  constexpr int NSB = 2;               // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * kW * NSB;   // rows per batch
  constexpr double kInf = __builtin_huge_val();
  const int u = blockIdx.x / p.splits;
  const int c = blockIdx.x - u * p.splits;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ double s_part[kW][G][kD];
  __shared__ double s_pm[kW][G], s_pd[kW][G];
  __shared__ double s_wf[kW][G], s_wM[G];

  int mf = p.m;
  if (p.idx_len) {
    const int L = p.idx_len[u];
    mf = L < 0 ? 0 : (L > p.m ? p.m : L);
  }
  const int per = (mf + p.splits - 1) / p.splits;
  const int r0 = min(mf, c * per), r1 = min(mf, r0 + per);
  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = rsrc_of<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = rsrc_of<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
  const double scale = (double)p.scale;
  float qr[G][8];  // bf16/fp32 query values are exact in fp32 and in fp64
#pragma unroll
  for (int h = 0; h < G; ++h)
    load_q8<T>(p.q, ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16, qr[h]);

  double mh[G], Df[G], Nf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mh[h] = -kInf;
    Df[h] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) Nf[h][i] = 0.0;
  }
  // list entries of the next batch: lane l < 4*NSB holds row rb + 4*((l>>2)*kW + w) + (l&3)
  auto lane_row = [&](int rb) { return rb + 4 * ((lane >> 2) * kW + w) + (lane & 3); };
  auto list_at = [&](int rb) {
    const int r = lane_row(rb);
    int j = -1;
    if (lane < 4 * NSB && r < r1) {
      j = p.idx[lbase + r];
      if ((unsigned)j >= (unsigned)p.n) j = 0;  // flagged by the statistics kernel
    }
    return j;
  };
  auto issue = [&](int lj, RowChunk<T> (&kc)[NSB], RowChunk<T> (&vc)[NSB]) {
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int j = __shfl(lj, 4 * k + sub, 64);
      const int off = j >= 0 ? off_of<T>(j, p.sn, r16) : kOOBs;
      gather(kc[k], rk, off);
      gather(vc[k], rv, off);
    }
  };
  int lj = list_at(r0);
  RowChunk<T> kc[NSB], vc[NSB];
  issue(lj, kc, vc);
  for (int rb = r0; rb < r1; rb += STEP) {
    const int ln = list_at(rb + STEP);
    RowChunk<T> kn[NSB], vn[NSB];
    issue(ln, kn, vn);  // past the end: range-checked zeros, no traffic
    double x[NSB][G], bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) bm[h] = -kInf;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const bool ok = __shfl(lj, 4 * k + sub, 64) >= 0;
      double kd[8];
      widen8(kc[k], kd);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        double a = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fma((double)qr[h][i], kd[i], a);
        x[k][h] = ok ? scale * sum16_d(a) : -kInf;
        bm[h] = fmax(bm[h], x[k][h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (bm[h] > mh[h]) {
        const double f = rescale_d(mh[h], bm[h]);
        Df[h] *= f;
#pragma unroll
        for (int i = 0; i < 8; ++i) Nf[h][i] *= f;
        mh[h] = bm[h];
      }
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      // lane r16 < G evaluates exp for head r16; the row group shares it
      double xo = -kInf, mo = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (r16 == h) {
          xo = x[k][h];
          mo = mh[h];
        }
      const double eo = xo == -kInf ? 0.0 : exp(xo - mo);
      double vd[8];
      widen8(vc[k], vd);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma clang fp contract(off)
        const double e = row_bcast(eo, h);
        Df[h] += e;
#pragma unroll
        for (int i = 0; i < 8; ++i) Nf[h][i] += e * vd[i];
      }
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      kc[k] = kn[k];
      vc[k] = vn[k];
    }
    lj = ln;
  }
  // merge the row groups (log-sum-exp, fp64), then the waves
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const RowPairD mm = pass ? swap_d<true>(mh[h]) : swap_d<false>(mh[h]);
      const double M = fmax(mm.even, mm.odd);
      // the larger side scales by exp(0) = 1: one exponential per pair
      const bool ev_big = mm.even >= mm.odd;
      const double fs = rescale_d(ev_big ? mm.odd : mm.even, M);
      const double fa = ev_big ? (M == -kInf ? 0.0 : 1.0) : fs, fb = ev_big ? fs : 1.0;
      const RowPairD dd = pass ? swap_d<true>(Df[h]) : swap_d<false>(Df[h]);
      Df[h] = dd.even * fa + dd.odd * fb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const RowPairD nn = pass ? swap_d<true>(Nf[h][i]) : swap_d<false>(Nf[h][i]);
        Nf[h][i] = nn.even * fa + nn.odd * fb;
      }
      mh[h] = M;
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_part[w][h][8 * r16 + i] = Nf[h][i];
      if (r16 == 0) {
        s_pm[w][h] = mh[h];
        s_pd[w][h] = Df[h];
      }
    }
  }
  __syncthreads();
  // the waves' scale factors, once per (wave, head)
  if (tid < G) {
    double M = -kInf;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmax(M, s_pm[ww][tid]);
    s_wM[tid] = M;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) s_wf[ww][tid] = rescale_d(s_pm[ww][tid], M);
  }
  __syncthreads();
  double* rec = p.wexact + ((int64_t)u * p.splits + c) * G * (2 + kD);
  for (int e = tid; e < G * kD; e += 512) {
    const int h = e / kD, i = e - h * kD;
    const double M = s_wM[h];
    double a = 0.0, d = 0.0;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) {
      const double f = s_wf[ww][h];
      a += s_part[ww][h][i] * f;
      d += s_pd[ww][h] * f;
    }
    rec[2 * G + e] = a;
    if (i == 0) {
      rec[h] = M;
      rec[G + h] = d;
    }
  }
}

template <typename T, int G>
__global__ __launch_bounds__(512) void sampled_stats_kernel(const AttnParams p) {
  constexpr int NSB = 2;               // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * kW * NSB;   // rows per batch
  constexpr double kInf = __builtin_huge_val();
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ int s_A[kSampMaxList];
  __shared__ int s_bj[kSampMaxB0];
  __shared__ double s_wb[kSampMaxB0][G];  // base draws: logits, then weights exp(s - M)
  __shared__ double s_part[kW][G][kD];    // per-wave partial sums
  __shared__ double s_pm[kW][G];
  __shared__ double s_M[G], s_Mf[G], s_Df[G], s_mD[G];
  __shared__ double s_Nf[G][kD], s_mN[G][kD];
  __shared__ double s_hs[G][4];           // per head: two halves of |Nhat|^2
  __shared__ double s_bh[G];
  __shared__ double s_sf[kSampMaxSplits][G];  // the exact-part splits' scale factors
  __shared__ int s_b;

  // ---- the deterministic set, as A[i] = I_f[i] - i ---------------------------
  int mf = p.m;
  if (p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    mf = L;
  }
  const int64_t lbase = (int64_t)u * p.m;
  {
    int bad = 0;
    for (int i = tid; i < mf; i += 512) {
      int j = p.idx[lbase + i];
      if ((unsigned)j >= (unsigned)p.n) {
        bad |= SDA_FLAG_IDX_RANGE;
        j = 0;
      }
      if (i > 0 && p.idx[lbase + i - 1] >= j) bad |= SDA_FLAG_IDX_ORDER;
      s_A[i] = j - i;
    }
    if (bad) flag_unit(p.flags, u, bad);
  }
  const int64_t n_s = (int64_t)p.n - mf;
  const int b0 = n_s > 0 ? p.b0 : 0;
  const uint64_t key = splitmix_at(p.seed, (uint64_t)u);
  __syncthreads();

  // ---- base draws ---------------------------------------------------------------
  for (int k = tid; k < b0; k += 512) {
    const int64_t rank = (int64_t)__umul64hi(splitmix_at(key, (uint64_t)k), (uint64_t)n_s);
    const int pos = tail_position(s_A, mf, rank);
    s_bj[k] = pos < p.n ? pos : p.n - 1;  // in range whenever the list is valid
  }

  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = rsrc_of<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = rsrc_of<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
  const double scale = (double)p.scale;
  // query chunk (bf16/fp32 values are exact in fp32 and in fp64)
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load_q8<T>(p.q, ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16, qr[h]);
  // fp64 logit of the row chunk in kc for head h (identical on the 16 lanes)
  auto logit = [&](const RowChunk<T>& kc, double (&x)[G]) {
    double kd[8];
    widen8(kc, kd);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fma((double)qr[h][i], kd[i], a);
      x[h] = scale * sum16_d(a);
    }
  };

  // the first batch of base rows (keys and values) goes out now, so that its
  // latency overlaps the merge of the exact-part records below; the values
  // stay in registers for the two passes over them
  __syncthreads();  // the draw positions
  RowChunk<T> kc0[NSB], vc0[NSB];
#pragma unroll
  for (int k = 0; k < NSB; ++k) {
    const int r = 4 * (k * kW + w) + sub;
    const int off = r < b0 ? off_of<T>(s_bj[r], p.sn, r16) : kOOBs;
    gather(kc0[k], rk, off);
    gather(vc0[k], rv, off);
  }

  // ---- I_f: merge the exact-part records of the splits (log-sum-exp, fp64) ---
  {
    const double* rec = p.wexact + (int64_t)u * p.splits * G * (2 + kD);
    // the splits' scale factors, once per (split, head)
    if (tid < G) {
      double M = -kInf;
      for (int c = 0; c < p.splits; ++c) M = fmax(M, rec[(int64_t)c * G * (2 + kD) + tid]);
      s_Mf[tid] = M;
      for (int c = 0; c < p.splits; ++c) s_sf[c][tid] = rescale_d(rec[(int64_t)c * G * (2 + kD) + tid], M);
    }
    __syncthreads();
    for (int e = tid; e < G * kD; e += 512) {
      const int h = e / kD, i = e - h * kD;
      double a = 0.0, d = 0.0;
      for (int c = 0; c < p.splits; ++c) {
        const double* rc = rec + (int64_t)c * G * (2 + kD);
        const double f = s_sf[c][h];
        a += rc[2 * G + e] * f;
        d += rc[G + h] * f;
      }
      s_Nf[h][i] = a;
      if (i == 0) s_Df[h] = d;
    }
  }
  __syncthreads();

  // ---- base draws: fp64 logits, the shift M, the weights --------------------
  double bmx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) bmx[h] = -kInf;
  for (int rb = 0; rb < b0; rb += STEP) {
    RowChunk<T> kc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      if (rb == 0)
        kc[k] = kc0[k];
      else
        gather(kc[k], rk, r < b0 ? off_of<T>(s_bj[r], p.sn, r16) : kOOBs);
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      double x[G];
      logit(kc[k], x);
      if (r < b0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          bmx[h] = fmax(bmx[h], x[h]);
          if (r16 == h) s_wb[r][h] = x[h];
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const RowPairD a = swap_d<false>(bmx[h]);
    const double v = fmax(a.even, a.odd);
    const RowPairD b = swap_d<true>(v);
    bmx[h] = fmax(b.even, b.odd);
    if (lane == 0) s_pm[w][h] = bmx[h];
  }
  __syncthreads();
  if (tid < G) {
    double M = s_Mf[tid];
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmax(M, s_pm[ww][tid]);
    s_M[tid] = M;
  }
  __syncthreads();
  if (tid < G) s_bh[tid] = rescale_d(s_Mf[tid], s_M[tid]);  // (s_bh reused before the budget)
  __syncthreads();
  for (int e = tid; e < G * kD; e += 512) {
    const int h = e / kD, i = e - h * kD;
    const double f = s_bh[h];
    s_Nf[h][i] *= f;
    if (i == 0) s_Df[h] *= f;
  }
  for (int e = tid; e < b0 * G; e += 512) {
    const int k = e / G, h = e - k * G;
    s_wb[k][h] = exp(s_wb[k][h] - s_M[h]);
  }
  __syncthreads();

  // ---- base draws: means of r^D = w and r^N = w v ------------------------------
  auto base_values = [&](int rb, RowChunk<T> (&vc)[NSB]) {
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      if (rb == 0)
        vc[k] = vc0[k];
      else
        gather(vc[k], rv, r < b0 ? off_of<T>(s_bj[r], p.sn, r16) : kOOBs);
    }
  };
  {
    double mn[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) mn[h][i] = 0.0;
    for (int rb = 0; rb < b0; rb += STEP) {
      RowChunk<T> vc[NSB];
      base_values(rb, vc);
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        const int r = rb + 4 * (k * kW + w) + sub;
        if (r < b0) {
          double vd[8];
          widen8(vc[k], vd);
#pragma unroll
          for (int h = 0; h < G; ++h) {
#pragma clang fp contract(off)
            const double e = s_wb[r][h];
#pragma unroll
            for (int i = 0; i < 8; ++i) mn[h][i] += e * vd[i];
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) mn[h][i] = sum_rowgroups_d(mn[h][i]);
      if (sub == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s_part[w][h][8 * r16 + i] = mn[h][i];
      }
    }
    __syncthreads();
    for (int e = tid; e < G * kD; e += 512) {
      const int h = e / kD, i = e - h * kD;
      double a = 0.0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) a += s_part[ww][h][i];
      s_mN[h][i] = b0 > 0 ? a / (double)b0 : 0.0;
    }
    if (tid < G) {
      double a = 0.0;
      for (int k = 0; k < b0; ++k) a += s_wb[k][tid];
      s_mD[tid] = b0 > 0 ? a / (double)b0 : 0.0;
    }
    __syncthreads();
  }

  // ---- base draws: centred second moments --------------------------------------
  {
    double mnr[G][8], sq[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sq[h] = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mnr[h][i] = s_mN[h][8 * r16 + i];
    }
    for (int rb = 0; rb < b0; rb += STEP) {
      RowChunk<T> vc[NSB];
      base_values(rb, vc);
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        const int r = rb + 4 * (k * kW + w) + sub;
        if (r < b0) {
          double vd[8];
          widen8(vc[k], vd);
#pragma unroll
          for (int h = 0; h < G; ++h) {
#pragma clang fp contract(off)
            const double e = s_wb[r][h];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const double dv = e * vd[i] - mnr[h][i];
              sq[h] += dv * dv;
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double v = sum_rowgroups_d(sum16_d(sq[h]));
      if (lane == 0) s_pm[w][h] = v;
    }
    // |N_f + n_s mean(r^N)|^2 per head: 128 dims over two waves' lanes
    for (int e = tid; e < G * kD; e += 512) {
#pragma clang fp contract(off)
      const int h = e / kD, i = e - h * kD;
      const double nh = s_Nf[h][i] + (double)n_s * s_mN[h][i];
      double nn = nh * nh;
      nn = sum_rowgroups_d(sum16_d(nn));
      if ((tid & 63) == 0) s_hs[h][i >> 6] = nn;
    }
    __syncthreads();
  }
  if (tid < G) {
#pragma clang fp contract(off)
    const int h = tid;
    double bh = 0.0;
    if (b0 > 0) {
      const double mD = s_mD[h];
      double varD = 0.0;
      for (int k = 0; k < b0; ++k) {
        const double dv = s_wb[k][h] - mD;
        varD += dv * dv;
      }
      varD /= (double)(b0 - 1);
      double trN = 0.0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) trN += s_pm[ww][h];
      trN /= (double)(b0 - 1);
      const double normN = sqrt(s_hs[h][0] + s_hs[h][1]);
      const double Dhat = s_Df[h] + (double)n_s * mD;
      bh = budget_of(p.z, p.eps, (double)n_s, varD, Dhat, trN, normN);
    }
    s_bh[h] = bh;
  }
  __syncthreads();
  if (tid == 0) {
    double bstar = 0.0;
    for (int h = 0; h < G; ++h)
      if (s_bh[h] > bstar || s_bh[h] != s_bh[h]) bstar = s_bh[h];
    int64_t b = 0;
    if (n_s > 0) {
      if (!(bstar < (double)n_s)) {
        b = n_s;
      } else {
        b = (int64_t)ceil(bstar);
        if (b < 1) b = 1;
        if (b > n_s) b = n_s;
      }
    }
    s_b = (int)b;
    if (p.b_out) p.b_out[u] = (int32_t)b;
    if (p.bstar_out) p.bstar_out[u] = bstar;
    if (p.samples_out && b > p.b_cap) flag_unit(p.flags, u, SDA_FLAG_SAMPLE_CAP);
  }
  __syncthreads();

  // ---- hand the exact part and the budget to the draw workgroups -----------
  double* st = p.wstat + (int64_t)u * G * (2 + kD);
  for (int e = tid; e < G * kD; e += 512) st[2 * G + e] = s_Nf[e / kD][e % kD];
  if (tid < G) {
    st[tid] = s_M[tid];
    st[G + tid] = s_Df[tid];
  }
  if (tid == 0) p.wb[u] = s_b;
}

// the deterministic list as A[i] = I_f[i] - i (entries out of range count as
// position 0; the statistics kernel flags them)
__device__ __forceinline__ int list_len(const AttnParams& p, int u) {
  int mf = p.m;
  if (p.idx_len) {
    const int L = p.idx_len[u];
    mf = L < 0 ? 0 : (L > p.m ? p.m : L);
  }
  return mf;
}

// Exclusive prefix over the units of their work-item counts ceil(b_u / chunk)
// into pref[0..units] (pref[units] = total), by a 256-thread workgroup.
__device__ void work_item_prefix(const int32_t* wb, int units, int* pref, int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (units + 255) / 256;
  const int lo = min(units, tid * per), hi = min(units, lo + per);
  int run = 0;
  for (int u = lo; u < hi; ++u) run += (wb[u] + kDrawChunk - 1) / kDrawChunk;
  // inclusive scan of the per-thread runs: within the wave, then across waves
  int v = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) scratch[w] = v;
  __syncthreads();
  int base = 0;
  for (int ww = 0; ww < w; ++ww) base += scratch[ww];
  int at = base + v - run;  // exclusive start of this thread's run
  for (int u = lo; u < hi; ++u) {
    pref[u] = at;
    at += (wb[u] + kDrawChunk - 1) / kDrawChunk;
  }
  if (tid == 255) pref[units] = base + v;
  __syncthreads();
}

template <typename T, int G>
__global__ __launch_bounds__(256, (G * sizeof(T) >= 16 ? 1 : 3)) void sampled_draws_kernel(const AttnParams p) {
  constexpr int W = 4;              // waves
  constexpr int NSB = 4;            // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * W * NSB; // draws per batch
  const int units = p.B * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ int s_pref[kSampMaxUnits + 1];
  __shared__ int s_A[kSampMaxList];
  __shared__ int s_scan[W];
  __shared__ float s_m[W][G], s_l[W][G];
  __shared__ __attribute__((aligned(16))) float s_acc[W][G][kD];

  work_item_prefix(p.wb, units, s_pref, s_scan);
  const int total = s_pref[units];
  if (blockIdx.x == 0)
    for (int i = tid; i <= units; i += 256) p.wsched[i] = s_pref[i];
  const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
  int wi = blockIdx.x * per;
  const int wend = min(total, wi + per);
  const int maxc = sampled_max_items(p.n);

  while (wi < wend) {
    // the unit holding item wi: last u with pref[u] <= wi (units with no
    // items share their start with the next unit and are skipped)
    int lo = 0, hi = units - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= wi) lo = mid; else hi = mid - 1;
    }
    const int u = lo;
    const int c = wi - s_pref[u];
    const int seg_end = min(wend, s_pref[u + 1]);
    const int b = p.wb[u];
    const int t0 = c * kDrawChunk;
    const int t1 = min(b, (seg_end - s_pref[u]) * kDrawChunk);
    const int s = u / p.Hkv;
    const int g = u - s * p.Hkv;

    const int mf = list_len(p, u);
    const int64_t lbase = (int64_t)u * p.m;
    __syncthreads();  // the previous segment's readers of s_A and s_acc are done
    for (int i = tid; i < mf; i += 256) {
      int j = p.idx[lbase + i];
      if ((unsigned)j >= (unsigned)p.n) j = 0;
      s_A[i] = j - i;
    }
    const int64_t n_s = (int64_t)p.n - mf;
    const uint64_t key = splitmix_at(p.seed, (uint64_t)u);
    __syncthreads();

    // lane l < 4*NSB of wave w generates draw tb + 4*((l>>2)*W + w) + (l&3);
    // slot k of row group sub takes the draw of lane 4k + sub
    auto lane_draw = [&](int tb) { return tb + 4 * ((lane >> 2) * W + w) + (lane & 3); };
    auto position = [&](int t) {
      const int64_t rank = (int64_t)__umul64hi(splitmix_at(key, (uint64_t)(p.b0 + t)), (uint64_t)n_s);
      const int j = tail_position(s_A, mf, rank);
      return j < p.n ? j : p.n - 1;
    };
    int pj = 0;
    {
      const int t = lane_draw(t0);
      if (lane < 4 * NSB && t < t1) pj = position(t);
    }

    const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
    const rsrc_t rk = rsrc_of<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
    const rsrc_t rv = rsrc_of<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      load_q8<T>(p.q, ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16, qf[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[h][i] *= p.qscale;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }

    for (int tb = t0; tb < t1; tb += STEP) {
      const int t = lane_draw(tb);
      const bool own = lane < 4 * NSB && t < t1;
      if (own && p.samples_out && t < p.b_cap) p.samples_out[(int64_t)u * p.b_cap + t] = pj;
      int off[NSB];
      bool ok[NSB];
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        const int src = 4 * k + sub;
        const int j = __shfl(pj, src, 64);
        ok[k] = __shfl(own ? 1 : 0, src, 64) != 0;
        off[k] = ok[k] ? off_of<T>(j, p.sn, r16) : kOOBs;
      }
      RowChunk<T> kc[NSB], vc[NSB];
#pragma unroll
      for (int k = 0; k < NSB; ++k) gather(kc[k], rk, off[k]);
#pragma unroll
      for (int k = 0; k < NSB; ++k) gather(vc[k], rv, off[k]);
      // next batch's positions while the rows are in flight
      {
        const int tn = lane_draw(tb + STEP);
        if (lane < 4 * NSB && tn < t1) pj = position(tn);
      }
      float x[NSB][G], bm[G];
#pragma unroll
      for (int h = 0; h < G; ++h) bm[h] = kNegInf;
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        float kf[8];
        kc[k].unpack(kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qf[h][i], kf[i], a);
          a = sum16(a);
          x[k][h] = ok[k] ? a : kNegInf;
          bm[h] = fmaxf(bm[h], x[k][h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], bm[h]);
        const float al = rescale(m[h], mn);
        m[h] = mn;
        l[h] *= al;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= al;
      }
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        float vf[8];
        vc[k].unpack(vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float e = (m[h] == kNegInf) ? 0.f : fast_exp2(x[k][h] - m[h]);
          l[h] += e;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(e, vf[i], acc[h][i]);
        }
      }
    }

    // ---- merge the four row groups, then the waves; one record per head ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const RowPair mm = pass ? swap32(m[h]) : swap16(m[h]);
        const float M = fmaxf(mm.even, mm.odd);
        const float fa = rescale(mm.even, M), fb = rescale(mm.odd, M);
        const RowPair ll = pass ? swap32(l[h]) : swap16(l[h]);
        l[h] = ll.even * fa + ll.odd * fb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const RowPair aa = pass ? swap32(acc[h][i]) : swap16(acc[h][i]);
          acc[h][i] = aa.even * fa + aa.odd * fb;
        }
        m[h] = M;
      }
      if (sub == 0) {
        *reinterpret_cast<float4*>(&s_acc[w][h][8 * r16]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4*>(&s_acc[w][h][8 * r16 + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        if (r16 == 0) {
          s_m[w][h] = m[h];
          s_l[w][h] = l[h];
        }
      }
    }
    __syncthreads();
    float* rec = p.part + ((int64_t)u * maxc + c) * G * kDrawRec;
    for (int e = tid; e < G * kD; e += 256) {
      const int h = e / kD, dim = e - h * kD;
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) M = fmaxf(M, s_m[ww][h]);
      float a = 0.f, L = 0.f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const float f = rescale(s_m[ww][h], M);
        a = fmaf(s_acc[ww][h][dim], f, a);
        L = fmaf(s_l[ww][h], f, L);
      }
      float* rh = rec + h * kDrawRec;
      rh[4 + dim] = a;
      if (dim == 0) {
        rh[0] = M;
        rh[1] = L;
      }
    }
    wi = seg_end;
  }
}

// One workgroup per unit. The unit's draws are items [S, S + nc) of the
// numbering; a record exists for the first item of each draw workgroup's
// segment: item S, and every item k*per in (S, S + nc).
template <int G>
__global__ __launch_bounds__(512) void sampled_merge_kernel(const AttnParams p) {
  constexpr int kBlk = 128;  // records staged per round
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x;
  const int units = p.B * p.Hkv;
  const int mf = list_len(p, u);
  const int64_t n_s = (int64_t)p.n - mf;
  const int b = p.wb[u];
  const int maxc = sampled_max_items(p.n);
  const int S = p.wsched[u], nc = p.wsched[u + 1] - S, total = p.wsched[units];
  const int grid = min(kDrawGrid, units * maxc);
  const int per = (total + grid - 1) / grid;
  const double* st = p.wstat + (int64_t)u * G * (2 + kD);
  const float* rec = p.part + (int64_t)u * maxc * G * kDrawRec;
  const double fw = b > 0 ? (double)n_s / (double)b : 0.0;

  // record r of this unit sits at item chunk rc(r): 0, then k*per - S for the
  // workgroup boundaries k*per inside (S, S + nc)
  const int k0 = per > 0 ? S / per + 1 : 0;
  int nrec = 0;
  if (nc > 0) nrec = 1 + max(0, (S + nc - 1) / per - k0 + 1);
  auto rc = [&](int r) { return r == 0 ? 0 : (k0 + r - 1) * per - S; };

  __shared__ float s_red[512];
  __shared__ float s_md[G];
  __shared__ int s_c[kBlk];
  __shared__ float s_f[kBlk][G], s_rl[kBlk][G];

  // maximum of the record maxima per head (thread tid serves head tid % G)
  {
    float mx = kNegInf;
    for (int e = tid; e < nrec * G; e += 512) mx = fmaxf(mx, rec[((int64_t)rc(e / G) * G + e % G) * kDrawRec]);
    s_red[tid] = mx;
    __syncthreads();
    for (int span = 256; span >= G; span >>= 1) {
      if (tid < span) s_red[tid] = fmaxf(s_red[tid], s_red[tid + span]);
      __syncthreads();
    }
    if (tid < G) s_md[tid] = s_red[tid];
    __syncthreads();
  }

  float a[(G * kD + 511) / 512], L[(G * kD + 511) / 512];
#pragma unroll
  for (int k = 0; k < (G * kD + 511) / 512; ++k) a[k] = L[k] = 0.f;
  for (int r0 = 0; r0 < nrec; r0 += kBlk) {
    const int nb = min(kBlk, nrec - r0);
    for (int e = tid; e < nb * G; e += 512) {
      const int r = e / G, h = e - r * G;
      const int c = rc(r0 + r);
      const float* rh = rec + ((int64_t)c * G + h) * kDrawRec;
      if (h == 0) s_c[r] = c;
      s_f[r][h] = rescale(rh[0], s_md[h]);
      s_rl[r][h] = rh[1];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < (G * kD + 511) / 512; ++k) {
      const int e = tid + 512 * k;
      if (e < G * kD) {
        const int h = e / kD, dim = e - h * kD;
        int r = 0;
        for (; r + 8 <= nb; r += 8) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = rec[((int64_t)s_c[r + j] * G + h) * kDrawRec + 4 + dim];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            a[k] = fmaf(v[j], s_f[r + j][h], a[k]);
            L[k] = fmaf(s_rl[r + j][h], s_f[r + j][h], L[k]);
          }
        }
        for (; r < nb; ++r) {
          a[k] = fmaf(rec[((int64_t)s_c[r] * G + h) * kDrawRec + 4 + dim], s_f[r][h], a[k]);
          L[k] = fmaf(s_rl[r][h], s_f[r][h], L[k]);
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < (G * kD + 511) / 512; ++k) {
    const int e = tid + 512 * k;
    if (e < G * kD) {
      const int h = e / kD, dim = e - h * kD;
      // back to the fp64 shift M (natural units): exp(s - M) = 2^(x' - M log2 e)
      const double M = st[h];
      const double sc = (L[k] > 0.f) ? exp2((double)s_md[h] - M * 1.4426950408889634) : 0.0;
      const double num = st[2 * G + e] + fw * (double)a[k] * sc;
      const double den = st[G + h] + fw * (double)L[k] * sc;
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      p.out[qh * kD + dim] = den > 0.0 ? (float)(num / den) : 0.f;
      if (dim == 0 && p.lse) p.lse[qh] = den > 0.0 ? (float)(M + log(den)) : kNegInf;
    }
  }
}

template <typename T, int G>
static hipError_t launch_sampled_g(const AttnParams& p, hipStream_t st) {
  const int units = p.B * p.Hkv;
  hipLaunchKernelGGL((sampled_exact_kernel<T, G>), dim3(units * p.splits), dim3(512), 0, st, p);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL((sampled_stats_kernel<T, G>), dim3(units), dim3(512), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = std::min(kDrawGrid, units * sampled_max_items(p.n));
  hipLaunchKernelGGL((sampled_draws_kernel<T, G>), dim3(grid), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sampled_merge_kernel<G>), dim3(units), dim3(512), 0, st, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_sampled_t(const AttnParams& p, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_sampled_g<T, 1>(p, st);
    case 2: return launch_sampled_g<T, 2>(p, st);
    case 4: return launch_sampled_g<T, 4>(p, st);
    case 8: return launch_sampled_g<T, 8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sampled(const AttnParams& p, int dtype, int G, hipStream_t st) {
  return dtype == SDA_BF16 ? launch_sampled_t<bf16_t>(p, G, st) : launch_sampled_t<float>(p, G, st);
}

}  // namespace sda
