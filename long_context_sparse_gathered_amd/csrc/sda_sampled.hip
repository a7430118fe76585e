// sda_sampled.hip -- sparse decode attention with a sampled tail
// ("vAttention: Verified Sparse Attention via Sampling", method sections
// 1-3): the deterministic set I_f is read exactly, the unread rows are
// sampled uniformly with replacement, each sample weighted n_s / b (eq. 3),
// and the budget b comes from the CLT sample-size lemma applied to the
// numerator and the denominator (b = max(b_N, b_D), Lemma 4.2), with the
// statistics estimated from b0 base draws.
//
// Four launches per call:
//   sampled_exact_kernel  `splits` workgroups per unit share the exact pass
//                         over I_f (an fp64 record per share); B*Hkv more
//                         workgroups, one per (sequence, KV head), check the
//                         list and take the b0 base draws' fp64 moments
//                         relative to their own maximum. About 256 in all,
//                         one per CU.
//   sampled_budget_kernel one workgroup per unit: the records merged at the
//                         unit's maximum M, the base moments rescaled to it,
//                         the budget b; leaves M, D_f, N_f and b in the
//                         workspace.
//   sampled_draws_kernel  one round of workgroups (as many as the chip
//                         holds) shares the b fresh draws of every unit
//                         (work items of kDrawChunk draws): each generates
//                         its draws' positions, gathers the rows and keeps
//                         an fp32 online softmax.
//   sampled_merge_kernel  one workgroup per unit: log-sum-exp merge of the
//                         draw partials, then num = N_f + (n_s/b) N_dyn and
//                         den = D_f + (n_s/b) D_dyn in fp64.
// With a table of delta splits (nz > 0) the budget is the verified one
// (budget_verified: eps and delta bound the output, not each sum).
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
#include <type_traits>

#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

namespace {

constexpr int kW = 8;  // waves per workgroup
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

// Lane moves within 16-lane rows whose every lane reads a lane of its own
// row (permutations and row broadcasts): no lane keeps an old value, so the
// moves take none (an old operand costs two register initialisations per
// move).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
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

// fp32 lane moves within 16-lane rows in which every lane reads a lane of
// its own row (the zero old value lets the compiler fold a move into the
// add that consumes it)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// lane H's value to the 16 lanes of each row group (a plain move, no old value)
template <int H>
__device__ __forceinline__ float bcast_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + H, 0xF, 0xF, false));
}
// Sums over the 16 lanes of a row group of four values a[0..3], reduce-
// scattered: lane r16 returns the sum of a[r16 >> 2]. Partners r16 ^ 8
// (row_ror:8; bit 3 keeps heads 2..3), r16 ^ 7 (row_half_mirror; bit 2 keeps
// the odd one of the pair), then r16 ^ 1 and r16 ^ 2 (quad permutations):
// the four partner sets together cover the row.
__device__ __forceinline__ float sum16_scatter4(const float (&a)[4], int r16) {
  const bool b3 = (r16 & 8) != 0, b2 = (r16 & 4) != 0;
  const float s0 = b3 ? a[0] : a[2], k0 = b3 ? a[2] : a[0];
  const float s1 = b3 ? a[1] : a[3], k1 = b3 ? a[3] : a[1];
  const float c0 = k0 + dpp_f<0x128>(s0);
  const float c1 = k1 + dpp_f<0x128>(s1);
  const float sv = b2 ? c0 : c1, kv = b2 ? c1 : c0;
  float d = kv + dpp_f<0x141>(sv);
  d += dpp_f<0xB1>(d);
  d += dpp_f<0x4E>(d);
  return d;
}

// lane H's value, broadcast to the 16 lanes of each row group (row_newbcast)
template <int H>
__device__ __forceinline__ double row_bcast_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0x150 + H, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0x150 + H, 0xF, 0xF, false);
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

// fp64 sums over the 16 lanes of a row group of four values, reduce-
// scattered as in sum16_scatter4: lane r16 returns the sum of a[r16 >> 2]
__device__ __forceinline__ double sum16_scatter4_d(const double (&a)[4], int r16) {
  const bool b3 = (r16 & 8) != 0, b2 = (r16 & 4) != 0;
  const double s0 = b3 ? a[0] : a[2], k0 = b3 ? a[2] : a[0];
  const double s1 = b3 ? a[1] : a[3], k1 = b3 ? a[3] : a[1];
  const double c0 = k0 + dpp_d<0x128>(s0);
  const double c1 = k1 + dpp_d<0x128>(s1);
  const double sv = b2 ? c0 : c1, kv = b2 ? c1 : c0;
  double d = kv + dpp_d<0x141>(sv);
  d += dpp_d<0xB1>(d);
  d += dpp_d<0x4E>(d);
  return d;
}
// lane 4h's value to the 16 lanes of each row group (h folds to a constant)
__device__ __forceinline__ double row_bcast4(double v, int h) {
  switch (h) {
    case 0: return row_bcast_d<0>(v);
    case 1: return row_bcast_d<4>(v);
    case 2: return row_bcast_d<8>(v);
    default: return row_bcast_d<12>(v);
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

// rows are read once per step: streaming (non-temporal) cache policy
constexpr int kRowNT = 2;
__device__ __forceinline__ void gather(RowChunk<bf16_t>& c, rsrc_t r, int off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kRowNT);
  c.raw = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void gather(RowChunk<float>& c, rsrc_t r, int off) {
  auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kRowNT);
  auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kRowNT);
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

// The verified budget of one head ("vAttention", verified-SDPA: Lemma 4.2
// and Theorem 4.3): for each given split delta = d_N + d_D the split of eps/2
// that balances the numerator's and the denominator's CLT budgets gives
// (2 (z_N a + z_D c) / eps)^2, with a = n_s sqrt(Tr) / |N_hat| and
// c = n_s sigma_D / D_hat; the budget is the smallest over the splits.
__device__ double budget_verified(const double* zs, int nz, double eps, double n_s, double varD, double Dhat,
                                  double trN, double normN) {
#pragma clang fp contract(off)
  double a = 0.0, c = 0.0;
  if (trN > 0.0) a = normN > 0.0 ? n_s * sqrt(trN) / normN : __builtin_huge_val();
  if (varD > 0.0) c = n_s * sqrt(varD) / Dhat;
  double best = __builtin_huge_val();
  for (int k = 0; k < nz; ++k) {
    const double t = 2.0 * (zs[2 * k] * a + zs[2 * k + 1] * c) / eps;
    const double v = t * t;
    if (v < best) best = v;
  }
  if (a == 0.0 && c == 0.0) best = 0.0;
  return best;
}

}  // namespace

// Base draws of unit u, on one extra workgroup of the exact-part launch (they
// need nothing from the exact part): the deterministic list's checks and its
// rank map, the b0 base positions, their fp64 logits, and per head, relative
// to the base draws' own maximum m_b (w' = e^{s - m_b}): S1 = sum w',
// VD = sum (w' - S1/b0)^2, N1 = sum w' v, TN = sum_k |w'_k v_k - N1/b0|^2.
// The budget kernel rescales them to the unit's maximum.  Record per head,
// in wbase: m_b, S1, VD, TN at [h], [G + h], [2G + h], [3G + h], N1 at
// [4G + h*d, 4G + (h+1)*d).
template <typename T, int G>
__device__ void sampled_base_role(const AttnParams& p, int u, double (&s_part)[kW][G][kD], int (&s_A)[kSampMaxList]) {
  constexpr int NSB = 2;               // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * kW * NSB;   // rows per batch
  constexpr double kInf = __builtin_huge_val();
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ int s_bj[kSampMaxB0];
  __shared__ double s_wb[kSampMaxB0][G];  // base draws: logits, then weights e^{s - m_b}
  __shared__ double s_pm[kW][G];
  __shared__ double s_mb[G], s_S1[G];
  __shared__ double s_N1[G][kD];

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
  __syncthreads();  // the draw positions

  // the first batch of base rows (keys and values) in one round trip; the
  // values stay in registers for the two passes over them
  RowChunk<T> kc0[NSB], vc0[NSB];
#pragma unroll
  for (int k = 0; k < NSB; ++k) {
    const int r = 4 * (k * kW + w) + sub;
    const int off = r < b0 ? off_of<T>(s_bj[r], p.sn, r16) : kOOBs;
    gather(kc0[k], rk, off);
    gather(vc0[k], rv, off);
  }

  // ---- fp64 logits and their maximum m_b ----------------------------------------
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
    double M = -kInf;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmax(M, s_pm[ww][tid]);
    s_mb[tid] = M;
  }
  __syncthreads();
  for (int e = tid; e < b0 * G; e += 512) {
    const int k = e / G, h = e - k * G;
    s_wb[k][h] = exp(s_wb[k][h] - s_mb[h]);
  }
  __syncthreads();

  // ---- S1 = sum w' and N1 = sum w' v ---------------------------------------------
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
    if (w < G) {  // wave h sums head h's base weights
      double a = 0.0;
      for (int k = lane; k < b0; k += 64) a += s_wb[k][w];
      a = sum_rowgroups_d(sum16_d(a));
      if (lane == 0) s_S1[w] = a;
    }
    __syncthreads();
    for (int e = tid; e < G * kD; e += 512) {
      const int h = e / kD, i = e - h * kD;
      double a = 0.0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) a += s_part[ww][h][i];
      s_N1[h][i] = a;
    }
    __syncthreads();
  }

  // ---- centred second moments: TN and VD -------------------------------------------
  double* rec = p.wbase + (int64_t)u * G * (4 + kD);
  {
    double mnr[G][8], sq[G];
    const double inv = b0 > 0 ? 1.0 / (double)b0 : 0.0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sq[h] = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mnr[h][i] = s_N1[h][8 * r16 + i] * inv;
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
    if (w < G) {  // wave h: head h's centred weight sum of squares
#pragma clang fp contract(off)
      const double mD = s_S1[w] * inv;
      double vd2 = 0.0;
      for (int k = lane; k < b0; k += 64) {
        const double dv = s_wb[k][w] - mD;
        vd2 += dv * dv;
      }
      vd2 = sum_rowgroups_d(sum16_d(vd2));
      if (lane == 0) rec[2 * G + w] = vd2;
    }
    __syncthreads();
  }
  if (tid < G) {
    double tn = 0.0;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) tn += s_pm[ww][tid];
    rec[tid] = s_mb[tid];
    rec[G + tid] = s_S1[tid];
    rec[3 * G + tid] = tn;
  }
  for (int e = tid; e < G * kD; e += 512) rec[4 * G + e] = s_N1[e / kD][e % kD];
}

// Exact part over a share of I_f: rows [c*per, min(mf, (c+1)*per)) of unit u
// for workgroup (u, c), an fp64 online softmax per row group (keys and values
// read together), merged into one record (m, D, N) per head relative to m.
// The first B*Hkv workgroups of the launch take the base draws instead, one
// unit each (sampled_base_role).
template <typename T, int G>
__global__ __launch_bounds__(512) void sampled_exact_kernel(const AttnParams p) {
  constexpr int NSB = 2;               // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * kW * NSB;   // rows per batch
  constexpr double kInf = __builtin_huge_val();
  __shared__ double s_part[kW][G][kD];
  __shared__ int s_list[kSampMaxList];  // the base role's A[i]; the exact role's share of I_f
  const int units = p.B * p.Hkv;
  if ((int)blockIdx.x < units) {
    sampled_base_role<T, G>(p, blockIdx.x, s_part, s_list);
    return;
  }
  const int u = (blockIdx.x - units) / p.splits;
  const int c = (blockIdx.x - units) - u * p.splits;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

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
  // this workgroup's share of the list, staged in LDS at once (entries out
  // of range count as row 0; the base-draw workgroup flags them)
  for (int r = r0 + tid; r < r1; r += 512) {
    const int j = p.idx[lbase + r];
    s_list[r - r0] = (unsigned)j < (unsigned)p.n ? j : 0;
  }
  __syncthreads();
  // list entries of the next batch: lane l < 4*NSB holds row rb + 4*((l>>2)*kW + w) + (l&3)
  auto lane_row = [&](int rb) { return rb + 4 * ((lane >> 2) * kW + w) + (lane & 3); };
  auto list_at = [&](int rb) {
    const int r = lane_row(rb);
    return lane < 4 * NSB && r < r1 ? s_list[r - r0] : -1;
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
    if constexpr (G == 4) {
      // every slot's dot products unconditionally (a slot past the list
      // holds zero rows), so that they and their row sums interleave; the
      // empty slots are masked afterwards
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        double kd[8];
        widen8(kc[k], kd);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          double a = 0.0;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fma((double)qr[h][i], kd[i], a);
          x[k][h] = a;
        }
      }
      // the four heads' sums reduce-scattered over the row group: lane r16
      // holds head ho = r16 >> 2's logit of each slot and takes its one
      // exponential; lanes 4h of the row group hand head h's values on
      const int ho = r16 >> 2;
      double xo[NSB], bmo = -kInf;
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        const bool ok = __shfl(lj, 4 * k + sub, 64) >= 0;
        const double a4[4] = {x[k][0], x[k][1], x[k][2], x[k][3]};
        xo[k] = ok ? scale * sum16_scatter4_d(a4, r16) : -kInf;
        bmo = fmax(bmo, xo[k]);
      }
      const double mo = ho == 0 ? mh[0] : ho == 1 ? mh[1] : ho == 2 ? mh[2] : mh[3];
      const double fo = bmo > mo ? rescale_d(mo, bmo) : 1.0;  // 1 where the maximum stays
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const double f = row_bcast4(fo, h);
        Df[h] *= f;
#pragma unroll
        for (int i = 0; i < 8; ++i) Nf[h][i] *= f;
        mh[h] = fmax(mh[h], row_bcast4(bmo, h));
      }
      const double mn = fmax(mo, bmo);
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        const double eo = xo[k] == -kInf ? 0.0 : exp(xo[k] - mn);
        double vd[8];
        widen8(vc[k], vd);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const double e = row_bcast4(eo, h);
          Df[h] += e;
#pragma unroll
          for (int i = 0; i < 8; ++i) Nf[h][i] = fma(e, vd[i], Nf[h][i]);
        }
      }
    } else {
      // (other group sizes: one head at a time, which keeps fewer values live)
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
      {
        // a new maximum rescales the running sums: lane r16 < G takes the one
        // exponential of head r16 and the row group shares it (1 where the
        // maximum stays)
        double mo = 0.0, bo = 0.0;
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (r16 == h) {
            mo = mh[h];
            bo = bm[h];
          }
        const double fo = bo > mo ? rescale_d(mo, bo) : 1.0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const double f = row_bcast(fo, h);
          Df[h] *= f;
#pragma unroll
          for (int i = 0; i < 8; ++i) Nf[h][i] *= f;
          mh[h] = fmax(mh[h], bm[h]);
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
          const double e = row_bcast(eo, h);
          Df[h] += e;
#pragma unroll
          for (int i = 0; i < 8; ++i) Nf[h][i] = fma(e, vd[i], Nf[h][i]);
        }
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

// The budget of each unit (one workgroup per unit): the exact part's
// records merged at the unit's maximum M = max(M_f, m_b) (fp64 log-sum-exp),
// the base draws' moments rescaled by e^{m_b - M}, the CLT budget per head
// (b = max over the group's heads, Lemma 4.2); M, D_f, N_f and b go to the
// workspace for the draw and merge kernels.
template <int G>
__global__ __launch_bounds__(256) void sampled_budget_kernel(const AttnParams p) {
  constexpr int NE = (G * kD + 255) / 256;  // vector elements per thread
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  // per head: the splits' (M_c, D_c), then the base draws' (m_b, S1, VD, TN)
  __shared__ double s_sc[2 * kSampMaxSplits + 4][G];
  __shared__ double s_sf[kSampMaxSplits][G];  // the exact-part splits' scale factors to M
  __shared__ double s_M[G], s_fb[G], s_Df[G];
  __shared__ double s_hs[G][2];               // per head: two halves of |Nhat|^2
  __shared__ double s_bh[G];

  int mf = p.m;
  if (p.idx_len) {
    const int L = p.idx_len[u];
    mf = L < 0 ? 0 : (L > p.m ? p.m : L);
  }
  const int64_t n_s = (int64_t)p.n - mf;
  const int b0 = n_s > 0 ? p.b0 : 0;
  const double inv = b0 > 0 ? 1.0 / (double)b0 : 0.0;
  const int splits = p.splits;
  const double* rec = p.wexact + (int64_t)u * splits * G * (2 + kD);
  const double* bs = p.wbase + (int64_t)u * G * (4 + kD);

  // every load in one round trip: the scalars to LDS, the vectors to registers
  if (tid < (2 * splits + 4) * G) {
    const int k = tid / G, h = tid - k * G;
    s_sc[k][h] = k < 2 * splits ? rec[(int64_t)(k >> 1) * G * (2 + kD) + (k & 1) * G + h]
                                : bs[(k - 2 * splits) * G + h];
  }
  double nv[NE][kSampMaxSplits], bv[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    bv[j] = e < G * kD ? bs[4 * G + e] : 0.0;
#pragma unroll
    for (int c = 0; c < kSampMaxSplits; ++c)
      nv[j][c] = e < G * kD && c < splits ? rec[(int64_t)c * G * (2 + kD) + 2 * G + e] : 0.0;
  }
  __syncthreads();
  if (tid < G) {
    const double mb = s_sc[2 * splits][tid];
    double M = mb;
    for (int c = 0; c < splits; ++c) M = fmax(M, s_sc[2 * c][tid]);
    s_M[tid] = M;
    double d = 0.0;
    for (int c = 0; c < splits; ++c) {
      const double f = rescale_d(s_sc[2 * c][tid], M);
      s_sf[c][tid] = f;
      d += s_sc[2 * c + 1][tid] * f;
    }
    s_Df[tid] = d;
    s_fb[tid] = rescale_d(mb, M);
  }
  __syncthreads();
  double* st = p.wstat + (int64_t)u * G * (2 + kD);
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < G * kD) {  // a wave covers 64 dims of one head
#pragma clang fp contract(off)
      const int h = e / kD, i = e - h * kD;
      double a = 0.0;
#pragma unroll
      for (int c = 0; c < kSampMaxSplits; ++c)
        if (c < splits) a += nv[j][c] * s_sf[c][h];
      st[2 * G + e] = a;
      const double mN = s_fb[h] * bv[j] * inv;
      const double nh = a + (double)n_s * mN;
      double nn = nh * nh;
      nn = sum_rowgroups_d(sum16_d(nn));
      if (lane == 0) s_hs[h][i >> 6] = nn;
    }
  }
  __syncthreads();
  if (tid < G) {
#pragma clang fp contract(off)
    const int h = tid;
    double bh = 0.0;
    if (b0 > 0) {
      const double fb = s_fb[h];
      const double mD = fb * s_sc[2 * splits + 1][h] * inv;
      const double varD = fb * fb * s_sc[2 * splits + 2][h] / (double)(b0 - 1);
      const double trN = fb * fb * s_sc[2 * splits + 3][h] / (double)(b0 - 1);
      const double normN = sqrt(s_hs[h][0] + s_hs[h][1]);
      const double Dhat = s_Df[h] + (double)n_s * mD;
      bh = p.nz > 0 ? budget_verified(p.zs, p.nz, p.eps, (double)n_s, varD, Dhat, trN, normN)
                    : budget_of(p.z, p.eps, (double)n_s, varD, Dhat, trN, normN);
    }
    s_bh[h] = bh;
    st[h] = s_M[h];
    st[G + h] = s_Df[h];
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
    if (p.b_out) p.b_out[u] = (int32_t)b;
    if (p.bstar_out) p.bstar_out[u] = bstar;
    if (p.samples_out && b > p.b_cap) flag_unit(p.flags, u, SDA_FLAG_SAMPLE_CAP);
    p.wb[u] = (int32_t)b;
  }
}

// the deterministic list as A[i] = I_f[i] - i (entries out of range count as
// position 0; the base-draw workgroup flags them)
__device__ __forceinline__ int list_len(const AttnParams& p, int u) {
  int mf = p.m;
  if (p.idx_len) {
    const int L = p.idx_len[u];
    mf = L < 0 ? 0 : (L > p.m ? p.m : L);
  }
  return mf;
}

// Exclusive prefix over the units of their work-item counts ceil(b_u / chunk)
// into pref[0..units] (pref[units] = total), by a workgroup of NT threads.
template <int NT>
__device__ void work_item_prefix(const int32_t* wb, int units, int* pref, int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (units + NT - 1) / NT;
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
  if (tid == NT - 1) pref[units] = base + v;
  __syncthreads();
}

template <typename T, int G>
__global__ __launch_bounds__(512, (sizeof(T) == 2 && G <= 4 ? 4 : 2)) void sampled_draws_kernel(const AttnParams p) {
  constexpr int W = 8;              // waves
  constexpr int NT = 64 * W;        // threads
  constexpr int NSB = 4;            // slots (of 4 rows) per wave per batch
  constexpr int STEP = 4 * W * NSB; // draws per batch
  const int units = p.B * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ int s_pref[kSampMaxUnits + 1];
  __shared__ int s_scan[W];
  __shared__ float s_m[W][G], s_l[W][G];
  // the list A[i] during a segment's draws, then the waves' partial sums:
  // one array for both keeps the workgroup within 40 KB of LDS (four per CU)
  constexpr int kBufBytes = kSampMaxList * 4 > W * G * kD * 4 ? kSampMaxList * 4 : W * G * kD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kBufBytes];
  int* const s_A = reinterpret_cast<int*>(s_buf);
  auto s_acc = reinterpret_cast<float (*)[G][kD]>(s_buf);

  work_item_prefix<NT>(p.wb, units, s_pref, s_scan);
  const int total = s_pref[units];
  if (blockIdx.x == 0)
    for (int i = tid; i <= units; i += NT) p.wsched[i] = s_pref[i];
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
    for (int i = tid; i < mf; i += NT) {
      int j = p.idx[lbase + i];
      if ((unsigned)j >= (unsigned)p.n) j = 0;
      s_A[i] = j - i;
    }
    const int64_t n_s = (int64_t)p.n - mf;
    const uint64_t key = splitmix_at(p.seed, (uint64_t)u);
    __syncthreads();

    // Batch tb's slot k of row group sub takes draw tb + 4*(k*W + w) + sub.
    // The positions of kPB batches are found at once, one draw per lane:
    // lane LPB*i + 4k + sub holds slot k, row group sub of batch i (a binary
    // search per draw, whose cost is per wave instruction, not per lane).
    constexpr int LPB = 4 * NSB, kPB = 64 / LPB;
    auto position = [&](int t) {
      const int64_t rank = (int64_t)__umul64hi(splitmix_at(key, (uint64_t)(p.b0 + t)), (uint64_t)n_s);
      const int j = tail_position(s_A, mf, rank);
      return j < p.n ? j : p.n - 1;
    };
    auto positions = [&](int tb) {  // of batches tb, tb + STEP, ...; the draws recorded here
      const int ll = lane % LPB;
      const int t = tb + (lane / LPB) * STEP + 4 * ((ll >> 2) * W + w) + (ll & 3);
      int j = 0;
      if (t < t1) {
        j = position(t);
        if (p.samples_out && t < p.b_cap) p.samples_out[(int64_t)u * p.b_cap + t] = j;
      }
      return j;
    };
    int pj = positions(t0);

    const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
    const rsrc_t rk = rsrc_of<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
    const rsrc_t rv = rsrc_of<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
    // the query: bf16 rows keep it as bf16 pairs for the two-wide bf16 dot
    // product (exact products, fp32 sums; the scale follows the sum), fp32
    // rows as fp32 with the scale folded in
    constexpr bool kBf = std::is_same<T, bf16_t>::value;
    float qf[G][8];
    uint32_t qw[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t qoff = ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16;
      if constexpr (kBf) {
        RowChunk<bf16_t> c;
        c.load_cached(reinterpret_cast<const bf16_t*>(p.q) + qoff);
        qw[h][0] = c.raw.x;
        qw[h][1] = c.raw.y;
        qw[h][2] = c.raw.z;
        qw[h][3] = c.raw.w;
      } else {
        load_q8<T>(p.q, qoff, qf[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[h][i] *= p.qscale;
      }
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }

    int bi = 0;  // this batch's place among the kPB whose positions pj holds
    for (int tb = t0; tb < t1; tb += STEP) {
      int off[NSB];
      bool ok[NSB];
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        ok[k] = tb + 4 * (k * W + w) + sub < t1;
        const int j = __shfl(pj, LPB * bi + 4 * k + sub, 64);
        off[k] = ok[k] ? off_of<T>(j, p.sn, r16) : kOOBs;
      }
      RowChunk<T> kc[NSB], vc[NSB];
#pragma unroll
      for (int k = 0; k < NSB; ++k) gather(kc[k], rk, off[k]);
#pragma unroll
      for (int k = 0; k < NSB; ++k) gather(vc[k], rv, off[k]);
      // the next kPB batches' positions while the rows are in flight
      if (++bi == kPB) {
        bi = 0;
        pj = positions(tb + STEP);
      }
      if constexpr (kBf && G == 4) {
        // the four heads' dot products reduce-scattered over the row group:
        // lane r16 holds head ho = r16 >> 2's logit of each slot and takes its
        // one exponential; the row group's lanes 4h hand head h's values on
        const int ho = r16 >> 2;
        float xo[NSB], bmo = kNegInf;
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
          const uint32_t kw[4] = {kc[k].raw.x, kc[k].raw.y, kc[k].raw.z, kc[k].raw.w};
          float a[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            a[h] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              a[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[h][i]),
                                                     __builtin_bit_cast(bf16x2_t, kw[i]), a[h], false);
          }
          xo[k] = ok[k] ? sum16_scatter4(a, r16) * p.qscale : kNegInf;
          bmo = fmaxf(bmo, xo[k]);
        }
        const float bm[4] = {bcast_f<0>(bmo), bcast_f<4>(bmo), bcast_f<8>(bmo), bcast_f<12>(bmo)};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (__ballot(bm[h] > m[h])) {  // some row group's maximum grows (elsewhere al = 1)
            const float mn = fmaxf(m[h], bm[h]);
            const float al = rescale(m[h], mn);
            m[h] = mn;
            l[h] *= al;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][i] *= al;
          }
        }
        const float mo = ho == 0 ? m[0] : ho == 1 ? m[1] : ho == 2 ? m[2] : m[3];
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
          float vf[8];
          vc[k].unpack(vf);
          const float eo = (mo == kNegInf) ? 0.f : fast_exp2(xo[k] - mo);
          const float e[4] = {bcast_f<0>(eo), bcast_f<4>(eo), bcast_f<8>(eo), bcast_f<12>(eo)};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            l[h] += e[h];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(e[h], vf[i], acc[h][i]);
          }
        }
      } else {
        float x[NSB][G], bm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) bm[h] = kNegInf;
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float a = 0.f;
            if constexpr (kBf) {
              const uint32_t kw[4] = {kc[k].raw.x, kc[k].raw.y, kc[k].raw.z, kc[k].raw.w};
#pragma unroll
              for (int i = 0; i < 4; ++i)
                a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[h][i]),
                                                    __builtin_bit_cast(bf16x2_t, kw[i]), a, false);
              a = sum16(a) * p.qscale;
            } else {
              float kf[8];
              kc[k].unpack(kf);
#pragma unroll
              for (int i = 0; i < 8; ++i) a = fmaf(qf[h][i], kf[i], a);
              a = sum16(a);
            }
            x[k][h] = ok[k] ? a : kNegInf;
            bm[h] = fmaxf(bm[h], x[k][h]);
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (__ballot(bm[h] > m[h])) {  // some row group's maximum grows (elsewhere al = 1)
            const float mn = fmaxf(m[h], bm[h]);
            const float al = rescale(m[h], mn);
            m[h] = mn;
            l[h] *= al;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][i] *= al;
          }
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
    }

    // ---- merge the four row groups, then the waves; one record per head ----
    __syncthreads();  // every wave is done with A[i]: its LDS takes the partial sums
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
    for (int e = tid; e < G * kD; e += NT) {
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
  constexpr int kBlk = 256;  // records staged per round
  constexpr int NE = (G * kD + 511) / 512;
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int units = p.B * p.Hkv;
  const int mf = list_len(p, u);
  const int64_t n_s = (int64_t)p.n - mf;
  const int b = p.wb[u];
  const int maxc = sampled_max_items(p.n);
  const int S = p.wsched[u], nc = p.wsched[u + 1] - S, total = p.wsched[units];
  const int grid = min(p.draw_grid, units * maxc);
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

  __shared__ float s_pm[8][G];     // per wave: partial maxima
  __shared__ float s_md[G];
  __shared__ int s_c[kBlk];
  __shared__ float s_rm[kBlk][G], s_rl[kBlk][G], s_f[kBlk][G];

  // the exact part's values for this thread's outputs, loaded up front
  double xM[NE], xD[NE], xN[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int e = tid + 512 * k;
    const int h = (e < G * kD ? e : 0) / kD;
    xM[k] = st[h];
    xD[k] = st[G + h];
    xN[k] = e < G * kD ? st[2 * G + e] : 0.0;
  }

  // maximum of the record maxima per head; the first round's (m, l) stay in LDS
  {
    float mx = kNegInf;
    for (int e = tid; e < nrec * G; e += 512) {
      const int r = e / G, h = e - r * G;
      const float* rh = rec + ((int64_t)rc(r) * G + h) * kDrawRec;
      const float m = rh[0];
      if (r < kBlk) {
        s_rm[r][h] = m;
        s_rl[r][h] = rh[1];
        if (h == 0) s_c[r] = rc(r);
      }
      mx = fmaxf(mx, m);
    }
    // 512 is a multiple of G: thread tid serves head tid % G throughout
    for (int d = G; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if (lane < G) s_pm[w][lane] = mx;
    __syncthreads();
    if (tid < G) {
      float m = kNegInf;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) m = fmaxf(m, s_pm[ww][tid]);
      s_md[tid] = m;
    }
    __syncthreads();
  }

  float a[NE], L[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) a[k] = L[k] = 0.f;
  for (int r0 = 0; r0 < nrec; r0 += kBlk) {
    const int nb = min(kBlk, nrec - r0);
    for (int e = tid; e < nb * G; e += 512) {
      const int r = e / G, h = e - r * G;
      float m, l;
      if (r0 == 0) {
        m = s_rm[r][h];
        l = s_rl[r][h];
      } else {
        const int c = rc(r0 + r);
        const float* rh = rec + ((int64_t)c * G + h) * kDrawRec;
        m = rh[0];
        l = rh[1];
        if (h == 0) s_c[r] = c;
      }
      s_f[r][h] = rescale(m, s_md[h]);
      if (r0 != 0) s_rl[r][h] = l;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NE; ++k) {
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
  for (int k = 0; k < NE; ++k) {
    const int e = tid + 512 * k;
    if (e < G * kD) {
      const int h = e / kD, dim = e - h * kD;
      // back to the fp64 shift M (natural units): exp(s - M) = 2^(x' - M log2 e)
      const double M = xM[k];
      const double sc = (L[k] > 0.f) ? exp2((double)s_md[h] - M * 1.4426950408889634) : 0.0;
      const double num = xN[k] + fw * (double)a[k] * sc;
      const double den = xD[k] + fw * (double)L[k] * sc;
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      p.out[qh * kD + dim] = den > 0.0 ? (float)(num / den) : 0.f;
      if (dim == 0 && p.lse) p.lse[qh] = den > 0.0 ? (float)(M + log(den)) : kNegInf;
    }
  }
}

template <typename T, int G>
static hipError_t launch_sampled_g(const AttnParams& p, hipStream_t st) {
  const int units = p.B * p.Hkv;
  hipLaunchKernelGGL((sampled_exact_kernel<T, G>), dim3(units * (1 + p.splits)), dim3(512), 0, st, p);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL((sampled_budget_kernel<G>), dim3(units), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one round of draw workgroups: as many as the chip holds at once
  static const int resident = [] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sampled_draws_kernel<T, G>, 512, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return per_cu * cus;
  }();
  if (resident <= 0) return hipErrorInvalidDeviceFunction;
  AttnParams q = p;
  q.draw_grid = std::min(kDrawGrid, resident);
  const int grid = std::min(q.draw_grid, units * sampled_max_items(p.n));
  hipLaunchKernelGGL((sampled_draws_kernel<T, G>), dim3(grid), dim3(512), 0, st, q);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sampled_merge_kernel<G>), dim3(units), dim3(512), 0, st, q);
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
