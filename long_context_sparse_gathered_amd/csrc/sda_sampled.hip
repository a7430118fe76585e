// sda_sampled.hip -- sparse decode attention with a sampled tail
// ("vAttention: Verified Sparse Attention via Sampling", method sections
// 1-3): the deterministic set I_f is read exactly, the unread rows are
// sampled uniformly with replacement, each sample weighted n_s / b (eq. 3),
// and the budget b comes from the CLT sample-size lemma applied to the
// numerator and the denominator (b = max(b_N, b_D), Lemma 4.2), with the
// statistics estimated from b0 base draws.
//
// One workgroup (8 waves) per (sequence, KV head).  Everything the budget
// depends on -- logits, weights, sums, variances -- is fp64, so the integer
// budget matches an fp64 reference up to the summation order.  The b fresh
// draws feed only the output and are accumulated in fp32.
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

__device__ __forceinline__ double shfl_xor_d(double v, int mask) { return __shfl_xor(v, mask, 64); }

// sum over the 16 lanes of a row group, identical bits on every lane
__device__ __forceinline__ double sum16_d(double v) {
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) v += shfl_xor_d(v, msk);
  return v;
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

template <typename T, int G>
__global__ __launch_bounds__(512) void sampled_kernel(const AttnParams p) {
  constexpr int NSB = 4;  // slots (of 4 rows) per wave per batch
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ int s_A[kSampMaxList];
  __shared__ int s_bj[kSampMaxB0];
  __shared__ double s_red[kW][kD];       // fp64 scratch for cross-wave sums
  __shared__ double s_M[G], s_Df[G];
  __shared__ double s_Nf[G][kD];
  __shared__ double s_mx[kW][G];
  __shared__ double s_hs[G][4];          // per head: trN, |Nhat|^2 (two waves each)
  __shared__ double s_bh[G];
  __shared__ int s_b;
  __shared__ float s_dm[kW][G], s_dl[kW][G];
  __shared__ float s_dacc[kW][kD];

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

  // ---- base draws -------------------------------------------------------------
  for (int k = tid; k < b0; k += 512) {
    const int64_t rank = (int64_t)__umul64hi(splitmix_at(key, (uint64_t)k), (uint64_t)n_s);
    int pos = tail_position(s_A, mf, rank);
    s_bj[k] = pos < p.n ? pos : p.n - 1;  // in range whenever the list is valid
  }
  __syncthreads();

  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = rsrc_of<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = rsrc_of<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
  const T* Vrow0 = reinterpret_cast<const T*>(p.V) + kvoff;
  const int R1 = mf + b0;
  double* wl = p.wlog + (int64_t)u * (p.m + p.b0) * G;
  const double scale = (double)p.scale;

  // query chunk (bf16/fp32 values are exact in fp32 and in fp64)
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load_q8<T>(p.q, ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16, qr[h]);
  auto row_of = [&](int r) { return r < mf ? s_A[r] + r : s_bj[r - mf]; };

  // ---- pass 1: fp64 logits of I_f and the base draws ------------------------
  double mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = -__builtin_huge_val();
  for (int rb = 0; rb < R1; rb += 4 * kW * NSB) {
    int off[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      off[k] = r < R1 ? off_of<T>(row_of(r), p.sn, r16) : kOOBs;
    }
    RowChunk<T> kc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) gather(kc[k], rk, off[k]);
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      double kd[8];
      widen8(kc[k], kd);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        double a = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fma((double)qr[h][i], kd[i], a);
        const double sv = scale * sum16_d(a);
        if (r < R1) {
          mx[h] = fmax(mx[h], sv);
          if (r16 == h) wl[(int64_t)r * G + h] = sv;
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    double v = mx[h];
    v = fmax(v, shfl_xor_d(v, 16));
    v = fmax(v, shfl_xor_d(v, 32));
    if (lane == 0) s_mx[w][h] = v;
  }
  __threadfence_block();
  __syncthreads();
  if (tid < G) {
    double v = s_mx[0][tid];
#pragma unroll
    for (int ww = 1; ww < kW; ++ww) v = fmax(v, s_mx[ww][tid]);
    s_M[tid] = v;
  }
  __syncthreads();

  // ---- weights exp(s - M), once per (row, head) -------------------------------
  for (int e = tid; e < R1 * G; e += 512) {
    const int h = e % G;
    wl[e] = exp(wl[e] - s_M[h]);
  }
  __threadfence_block();
  __syncthreads();

  // ---- pass 2: D_f and N_f over I_f (fp64) -----------------------------------
  double Df[G], Nf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Df[h] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) Nf[h][i] = 0.0;
  }
  for (int rb = 0; rb < mf; rb += 4 * kW * NSB) {
    int off[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      off[k] = r < mf ? off_of<T>(row_of(r), p.sn, r16) : kOOBs;
    }
    RowChunk<T> vc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) gather(vc[k], rv, off[k]);
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      if (r < mf) {
        double vd[8];
        widen8(vc[k], vd);
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma clang fp contract(off)
          const double e = wl[(int64_t)r * G + h];
          Df[h] += e;
#pragma unroll
          for (int i = 0; i < 8; ++i) Nf[h][i] += e * vd[i];
        }
      }
    }
  }
  // reduce the four row groups, then the waves (fixed order), head by head
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double v = Nf[h][i];
      v += shfl_xor_d(v, 16);
      v += shfl_xor_d(v, 32);
      Nf[h][i] = v;
    }
    double d = Df[h];
    d += shfl_xor_d(d, 16);
    d += shfl_xor_d(d, 32);
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_red[w][8 * r16 + i] = Nf[h][i];
    }
    if (lane == 0) s_mx[w][h] = d;
    __syncthreads();
    if (tid < kD) {
      double a = 0.0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) a += s_red[ww][tid];
      s_Nf[h][tid] = a;
    }
    if (tid == kD) {
      double a = 0.0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) a += s_mx[ww][h];
      s_Df[h] = a;
    }
    __syncthreads();
  }

  // ---- budget from the base draws ---------------------------------------------
  for (int e = tid; e < G * kD; e += 512) {
#pragma clang fp contract(off)
    const int h = e / kD, i = e - h * kD;
    double trN = 0.0, nn = 0.0;
    if (b0 > 0) {
      double mN = 0.0;
      for (int k = 0; k < b0; ++k) {
        float f;
        if constexpr (sizeof(T) == 2) {
          f = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Vrow0)[(int64_t)s_bj[k] * p.sn + i] << 16);
        } else {
          f = reinterpret_cast<const float*>(Vrow0)[(int64_t)s_bj[k] * p.sn + i];
        }
        mN += wl[(int64_t)(mf + k) * G + h] * (double)f;
      }
      mN /= (double)b0;
      for (int k = 0; k < b0; ++k) {
        float f;
        if constexpr (sizeof(T) == 2) {
          f = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Vrow0)[(int64_t)s_bj[k] * p.sn + i] << 16);
        } else {
          f = reinterpret_cast<const float*>(Vrow0)[(int64_t)s_bj[k] * p.sn + i];
        }
        const double dv = wl[(int64_t)(mf + k) * G + h] * (double)f - mN;
        trN += dv * dv;
      }
      const double nh = s_Nf[h][i] + (double)n_s * mN;
      nn = nh * nh;
    }
    // sums over the 128 dims of head h: 64 lanes, then the head's two waves
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      trN += shfl_xor_d(trN, msk);
      nn += shfl_xor_d(nn, msk);
    }
    if (lane == 0) {
      s_hs[h][(i >> 6) * 2 + 0] = trN;
      s_hs[h][(i >> 6) * 2 + 1] = nn;
    }
  }
  __syncthreads();
  if (tid < G) {
#pragma clang fp contract(off)
    const int h = tid;
    double bh = 0.0;
    if (b0 > 0) {
      double mD = 0.0;
      for (int k = 0; k < b0; ++k) mD += wl[(int64_t)(mf + k) * G + h];
      mD /= (double)b0;
      double varD = 0.0;
      for (int k = 0; k < b0; ++k) {
        const double dv = wl[(int64_t)(mf + k) * G + h] - mD;
        varD += dv * dv;
      }
      varD /= (double)(b0 - 1);
      const double trN = (s_hs[h][0] + s_hs[h][2]) / (double)(b0 - 1);
      const double normN = sqrt(s_hs[h][1] + s_hs[h][3]);
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
  const int b = s_b;

  // ---- positions of the b fresh draws ------------------------------------------
  int32_t* pos = p.wpos + (int64_t)u * p.n;
  for (int k = tid; k < b; k += 512) {
    const int64_t rank = (int64_t)__umul64hi(splitmix_at(key, (uint64_t)(b0 + k)), (uint64_t)n_s);
    int j = tail_position(s_A, mf, rank);
    j = j < p.n ? j : p.n - 1;
    pos[k] = j;
    if (p.samples_out && k < p.b_cap) p.samples_out[(int64_t)u * p.b_cap + k] = j;
  }
  __threadfence_block();
  __syncthreads();

  // ---- the sampled rows: fp32 online softmax per row group ------------------
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[h][i] = qr[h][i] * p.qscale;
  float dm[G], dl[G], dacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    dm[h] = kNegInf;
    dl[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dacc[h][i] = 0.f;
  }
  for (int rb = 0; rb < b; rb += 4 * kW * NSB) {
    int off[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      off[k] = r < b ? off_of<T>(pos[r], p.sn, r16) : kOOBs;
    }
    RowChunk<T> kc[NSB], vc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) gather(kc[k], rk, off[k]);
#pragma unroll
    for (int k = 0; k < NSB; ++k) gather(vc[k], rv, off[k]);
    float x[NSB][G], bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) bm[h] = kNegInf;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int r = rb + 4 * (k * kW + w) + sub;
      float kf[8];
      kc[k].unpack(kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qf[h][i], kf[i], a);
        a = sum16(a);
        x[k][h] = r < b ? a : kNegInf;
        bm[h] = fmaxf(bm[h], x[k][h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(dm[h], bm[h]);
      const float al = rescale(dm[h], mn);
      dm[h] = mn;
      dl[h] *= al;
#pragma unroll
      for (int i = 0; i < 8; ++i) dacc[h][i] *= al;
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      float vf[8];
      vc[k].unpack(vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float e = (dm[h] == kNegInf) ? 0.f : fast_exp2(x[k][h] - dm[h]);
        dl[h] += e;
#pragma unroll
        for (int i = 0; i < 8; ++i) dacc[h][i] = fmaf(e, vf[i], dacc[h][i]);
      }
    }
  }

  // ---- combine and write, head by head ----------------------------------------
  const double fw = b > 0 ? (double)n_s / (double)b : 0.0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // merge the four row groups (log-sum-exp)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const RowPair mm = pass ? swap32(dm[h]) : swap16(dm[h]);
      const float M = fmaxf(mm.even, mm.odd);
      const float fa = rescale(mm.even, M), fb = rescale(mm.odd, M);
      const RowPair ll = pass ? swap32(dl[h]) : swap16(dl[h]);
      dl[h] = ll.even * fa + ll.odd * fb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const RowPair aa = pass ? swap32(dacc[h][i]) : swap16(dacc[h][i]);
        dacc[h][i] = aa.even * fa + aa.odd * fb;
      }
      dm[h] = M;
    }
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_dacc[w][8 * r16 + i] = dacc[h][i];
      if (r16 == 0) {
        s_dm[w][h] = dm[h];
        s_dl[w][h] = dl[h];
      }
    }
    __syncthreads();
    if (tid < kD) {
      float Md = kNegInf;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) Md = fmaxf(Md, s_dm[ww][h]);
      float a = 0.f, L = 0.f;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) {
        const float f = rescale(s_dm[ww][h], Md);
        a = fmaf(s_dacc[ww][tid], f, a);
        L = fmaf(s_dl[ww][h], f, L);
      }
      // back to the fp64 shift M (natural units): exp(s - M) = 2^(x' - M log2 e)
      const double M = s_M[h];
      const double sc = (L > 0.f) ? exp2((double)Md - M * 1.4426950408889634) : 0.0;
      const double num = s_Nf[h][tid] + fw * (double)a * sc;
      const double den = s_Df[h] + fw * (double)L * sc;
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      p.out[qh * kD + tid] = den > 0.0 ? (float)(num / den) : 0.f;
      if (tid == 0 && p.lse) p.lse[qh] = den > 0.0 ? (float)(M + log(den)) : kNegInf;
    }
    __syncthreads();
  }
}

template <typename T>
static hipError_t launch_sampled_t(const AttnParams& p, int G, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  switch (G) {
    case 1: hipLaunchKernelGGL((sampled_kernel<T, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((sampled_kernel<T, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((sampled_kernel<T, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((sampled_kernel<T, 8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sampled(const AttnParams& p, int dtype, int G, hipStream_t st) {
  return dtype == SDA_BF16 ? launch_sampled_t<bf16_t>(p, G, st) : launch_sampled_t<float>(p, G, st);
}

}  // namespace sda
