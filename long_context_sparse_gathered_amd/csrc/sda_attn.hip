// sda_attn.hip -- decode-attention kernels for gfx950.
//
//  sparse_unit_kernel   one 512-thread workgroup per (sequence, KV head):
//                       gathers every listed K and V row at once, two-pass
//                       softmax with an exact unit maximum, optional
//                       count-aware mean proxies ("OpenAttention", method
//                       stages 04-05: exact rows and proxies share one
//                       softmax).
//  stream_kernel        split-K streaming kernel with a per-row-group online
//                       softmax; serves plain sparse lists, the rank-1 prior
//                       ("RESA", Online Aggregator), dense decode and the
//                       prior build ("RESA", Prior Estimator: one extra query
//                       over the whole cache).
//  merge_kernel         log-sum-exp merge of split partials + the prior's
//                       delta merge.
#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

constexpr int kRsrcFlags = 0x00020000;
constexpr int kOOB = 0x7fffffff;   // byte offset outside every resource range

using rsrc_t = __amdgpu_buffer_rsrc_t;

template <typename T>
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t n, int64_t sn) {
  const int64_t bytes = ((int64_t)(n - 1) * sn + kD) * (int64_t)sizeof(T);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// Gather one row chunk through a range-checked buffer resource: an offset
// outside the resource returns zeros and touches no memory.
__device__ __forceinline__ void buf_load(RowChunk<bf16_t>& c, rsrc_t r, int off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  c.raw = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buf_load(RowChunk<float>& c, rsrc_t r, int off) {
  auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off == kOOB ? kOOB : off + 16, 0, 0);
  c.a = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
  c.b = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
}

template <typename T>
__device__ __forceinline__ int row_off(int64_t j, int64_t sn, int r16) {
  return (int)((j * sn + 8 * r16) * (int64_t)sizeof(T));
}

// Load the G query heads of KV head g (dims 8*r16..) scaled to log2 units.
template <int G>
__device__ __forceinline__ void load_query(const void* q, bool is_f32, int64_t row0, int r16, float qscale,
                                           float (&qf)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load_q8(q, (row0 + h) * kD + 8 * r16, is_f32, qf[h]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[h][i] *= qscale;
  }
}

template <int G>
__device__ __forceinline__ void dot_heads(const float (&qf)[G][8], const float (&kf)[8], float (&a)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(qf[h][i], kf[i], acc);
    a[h] = sum16(acc);
  }
}

// ---------------------------------------------------------------------------
// One workgroup per unit.  Slot k of wave w holds entries
// t = 4*(k*W + w) + (lane >> 4): every load instruction fetches four
// consecutive list entries.
template <typename T, int G, bool PROXY, int NS>
__global__ __launch_bounds__(512) void sparse_unit_kernel(const AttnParams p) {
  constexpr int W = kUnitWaves;
  constexpr int PC = PROXY ? kCmax : 1;
  constexpr int PW = PROXY ? W : 1;
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ float s_wmax[W][G];
  __shared__ float s_M[G];
  __shared__ float s_pl[G];
  __shared__ float s_l[W][G];
  __shared__ __attribute__((aligned(16))) float s_red[W][G][kD];
  __shared__ float s_csum[PW][PC][G];
  __shared__ int s_ccnt[PW][PC];
  __shared__ float s_qk[PC][G];
  __shared__ float s_cw[PC][G];
  __shared__ __attribute__((aligned(16))) float s_sv[PC][PROXY ? kD : 1];

  int len = p.m;
  if (p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    len = L;
  }
  if constexpr (PROXY) {
    // each wave clears its own slice, so program order alone orders the
    // clears before that wave's accumulations
#pragma unroll
    for (int i = lane; i < PC * G; i += 64) (&s_csum[w][0][0])[i] = 0.f;
    for (int i = lane; i < PC; i += 64) s_ccnt[w][i] = 0;
  }

  float qf[G][8];
  load_query<G>(p.q, p.q_f32, (int64_t)s * p.Hq + (int64_t)g * G, r16, p.qscale, qf);

  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);

  // ---- list entries -------------------------------------------------------
  int off[NS];
  float lw[NS];
  int cl[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int t = 4 * (k * W + w) + sub;
    int o = kOOB, c = -1;
    float lwk = kNegInf;
    if (t < len) {
      const int j = p.idx[lbase + t];
      if ((unsigned)j < (unsigned)p.n) {
        o = row_off<T>(j, p.sn, r16);
        lwk = p.logw ? p.logw[lbase + t] * kLog2e : 0.f;
        if constexpr (PROXY) {
          c = p.idx_cluster ? p.idx_cluster[lbase + t] : p.cluster_id[(int64_t)u * p.n + j];
          if (c < -1 || c >= p.C) {
            if (r16 == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
            c = -1;
          }
          if (t > 0 && r16 == 0 && p.idx[lbase + t - 1] >= j) flag_unit(p.flags, u, SDA_FLAG_IDX_ORDER);
        }
      } else if (r16 == 0) {
        flag_unit(p.flags, u, SDA_FLAG_IDX_RANGE);
      }
    }
    off[k] = o;
    lw[k] = lwk;
    cl[k] = c;
  }

  // ---- proxy state: q . sumK per cluster, sumV staged in LDS ---------------
  if constexpr (PROXY) {
#pragma unroll
    for (int cp = 0; cp < kCmax / (4 * W); ++cp) {
      const int b = 4 * (cp * W + w) + sub;
      if (b < p.C) {
        const int64_t rb = ((int64_t)u * p.C + b) * kD + 8 * r16;
        float skf[8], svf[8];
        load8f(p.sumK + rb, skf);
        load8f(p.sumV + rb, svf);
        float a[G];
        dot_heads<G>(qf, skf, a);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (r16 == h) s_qk[b][h] = a[h];
        *reinterpret_cast<float4*>(&s_sv[b][8 * r16]) = make_float4(svf[0], svf[1], svf[2], svf[3]);
        *reinterpret_cast<float4*>(&s_sv[b][8 * r16 + 4]) = make_float4(svf[4], svf[5], svf[6], svf[7]);
      }
    }
  }

  // ---- gather every listed row --------------------------------------------
  RowChunk<T> kc[NS], vc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) buf_load(kc[k], rk, off[k]);
#pragma unroll
  for (int k = 0; k < NS; ++k) buf_load(vc[k], rv, off[k]);

  // ---- logits ---------------------------------------------------------------
  float x[NS][G];
  float mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = kNegInf;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    float kf[8];
    kc[k].unpack(kf);
    float a[G];
    dot_heads<G>(qf, kf, a);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      x[k][h] = a[h] + lw[k];
      mx[h] = fmaxf(mx[h], x[k][h]);
    }
    if constexpr (PROXY) {
      if (cl[k] >= 0) {
        float mine = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (r16 == h) mine = a[h];
        if (r16 < G) atomicAdd(&s_csum[w][cl[k]][r16], mine);
        if (r16 == 0) atomicAdd(&s_ccnt[w][cl[k]], 1);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = max_rowgroups(mx[h]);
    if (lane == 0) s_wmax[w][h] = v;
  }
  __syncthreads();

  // ---- tail preparation (wave 0): unit maximum, proxy logits ---------------
  if (w == 0) {
    if constexpr (PROXY) {
      // lane handles (cluster, head) pairs e = lane + 64 r: head = lane % G
      constexpr int R = (kCmax * G + 63) / 64;
      const int h = lane % G;
      float pi[R], nbf[R];
      float hm = kNegInf;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = lane + 64 * r;
        const int b = e / G;
        pi[r] = kNegInf;
        nbf[r] = 0.f;
        if (b < p.C) {
          float ssum = 0.f;
          int rc = 0;
#pragma unroll
          for (int ww = 0; ww < W; ++ww) {
            ssum += s_csum[ww][b][h];
            rc += s_ccnt[ww][b];
          }
          const int nb = p.count[(int64_t)u * p.C + b] - rc;
          if (nb < 0 && h == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
          if (nb > 0) {
            nbf[r] = (float)nb;
            pi[r] = (s_qk[b][h] - ssum) / nbf[r] + __builtin_amdgcn_logf(nbf[r]);
          }
        }
        hm = fmaxf(hm, pi[r]);
      }
      // max over lanes with the same head (lane bits above log2 G)
#pragma unroll
      for (int msk = G; msk < 64; msk <<= 1) hm = fmaxf(hm, shfl_xor(hm, msk));
#pragma unroll
      for (int ww = 0; ww < W; ++ww) hm = fmaxf(hm, s_wmax[ww][h]);
      const float M = (hm == kNegInf) ? 0.f : hm;
      float pe = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = lane + 64 * r;
        const int b = e / G;
        const float ev = (pi[r] == kNegInf) ? 0.f : fast_exp2(pi[r] - M);
        pe += ev;
        if (b < p.C) s_cw[b][h] = (nbf[r] > 0.f) ? ev / nbf[r] : 0.f;
      }
#pragma unroll
      for (int msk = G; msk < 64; msk <<= 1) pe += shfl_xor(pe, msk);
      if (lane < G) {
        s_M[lane] = M;
        s_pl[lane] = pe;
      }
    } else {
      if (lane < G) {
        float hm = kNegInf;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) hm = fmaxf(hm, s_wmax[ww][lane]);
        s_M[lane] = (hm == kNegInf) ? 0.f : hm;
        s_pl[lane] = 0.f;
      }
    }
  }
  __syncthreads();

  // ---- weighted values --------------------------------------------------------
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) M[h] = s_M[h];
  float acc[G][8], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    float wt[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float e = fast_exp2(x[k][h] - M[h]);
      l[h] += e;
      wt[h] = e;
    }
    if constexpr (PROXY) {
      // a read member leaves its cluster's proxy: subtract its share of the
      // proxy value term (the proxy adds cw * sum of all member values)
      if (cl[k] >= 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) wt[h] -= s_cw[cl[k]][h];
      }
    }
    float vf[8];
    vc[k].unpack(vf);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(wt[h], vf[i], acc[h][i]);
  }

  // ---- reduce row groups, then waves ---------------------------------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = sum_rowgroups(acc[h][i]);
    l[h] = sum_rowgroups(l[h]);
  }
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&s_red[w][h][8 * r16]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(&s_red[w][h][8 * r16 + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      if (r16 == 0) s_l[w][h] = l[h];
    }
  }
  __syncthreads();

  for (int e = tid; e < G * kD; e += 512) {
    const int h = e / kD, dim = e - h * kD;
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      a += s_red[ww][h][dim];
      L += s_l[ww][h];
    }
    if constexpr (PROXY) {
      for (int b = 0; b < p.C; ++b) a = fmaf(s_cw[b][h], s_sv[b][dim], a);
      L += s_pl[h];
    }
    const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
    p.out[qh * kD + dim] = (L > 0.f) ? a / L : 0.f;
    if (dim == 0 && p.lse) p.lse[qh] = (L > 0.f) ? (s_M[h] + log2f(L)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Final value of one (head, dim) output from the merged sums.
//   M, L, a : the exact part (log2-unit max, denominator, numerator)
//   prior   : c (log2 bias shift), mP (log2 maxP), zP (sumP), oe (O_est[dim]),
//             SP, SPV (sums over the listed rows of exp2(P - mP) and its
//             value product)
struct Fin {
  float out, lse;
};

__device__ __forceinline__ Fin finalize_plain(float M, float L, float a) {
  Fin f;
  f.out = (L > 0.f) ? a / L : 0.f;
  f.lse = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
  return f;
}

__device__ __forceinline__ Fin finalize_prior(float M, float L, float a, float c, float mP, float zP, float oe,
                                              float SP, float SPV, float lambda) {
  // prior mass of the whole cache, log2 units: log2(lambda) + c + mP + log2(zP)
  float lp = kNegInf;
  if (lambda > 0.f && zP > 0.f) lp = log2f(lambda) + c + mP;
  const float Lexact = (L > 0.f) ? M + log2f(L) : kNegInf;
  const float lpt = (lp == kNegInf) ? kNegInf : lp + log2f(zP);
  float Ms = fmaxf(Lexact, lpt);
  if (Ms == kNegInf) Ms = 0.f;
  const float E = (lp == kNegInf) ? 0.f : fast_exp2(lp - Ms);
  float Bt = E * (zP - SP);
  float A = 0.f;
  if (Bt > 0.f) {
    A = E * (zP * oe - SPV);
  } else {
    Bt = 0.f;
  }
  const float fs = (L > 0.f) ? fast_exp2(M - Ms) : 0.f;
  const float num = A + a * fs;
  const float den = Bt + L * fs;
  Fin f;
  f.out = (den > 0.f) ? num / den : 0.f;
  f.lse = (den > 0.f) ? (Ms + log2f(den)) * kLn2 : kNegInf;
  return f;
}

// c_h in log2 units: <q'_h - muQ'_h, mu_K>, q' = q*scale*log2e.
template <int G>
__device__ __forceinline__ void bias_shift(const AttnParams& p, int s, int g, int r16, const float (&qf)[G][8],
                                           float (&c)[G]) {
  float mk[8];
  load8f(p.mu_K + ((int64_t)s * p.Hkv + g) * kD + 8 * r16, mk);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mq[8];
    load8f(p.mu_Q + ((int64_t)s * p.Hq + (int64_t)g * G + h) * kD + 8 * r16, mq);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaf(qf[h][i] - mq[i] * p.qscale, mk[i], a);
    c[h] = sum16(a);
  }
}

// ---------------------------------------------------------------------------
// Split-K streaming kernel.  Workgroup (u, split) covers list entries (or
// rows, for the dense modes) [split*chunk, min(len, (split+1)*chunk)).  Each
// 16-lane row group keeps its own online-softmax state; groups and waves are
// merged at the end.
template <typename T, int G, int MODE, int NSB>
__global__ __launch_bounds__(256) void stream_kernel(const AttnParams p) {
  constexpr int W = 4;
  constexpr bool DENSE = (MODE == kModeDense || MODE == kModeBuildPrior);
  constexpr bool PRIOR = (MODE == kModePrior);
  constexpr bool BUILD = (MODE == kModeBuildPrior);
  const int u = blockIdx.x / p.splits;
  const int split = blockIdx.x - u * p.splits;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;

  __shared__ float s_m[W][G], s_l[W][G], s_sp[W][G];
  __shared__ __attribute__((aligned(16))) float s_acc[W][G][kD];
  __shared__ __attribute__((aligned(16))) float s_spv[PRIOR ? W : 1][G][PRIOR ? kD : 1];
  __shared__ __attribute__((aligned(16))) float s_ks[BUILD ? W : 1][BUILD ? kD : 1];
  __shared__ float s_c[G];

  int len = DENSE ? p.n : p.m;
  if (!DENSE && p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0 && split == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    len = L;
  }
  const int t0 = split * p.chunk;
  const int t1 = min(len, t0 + p.chunk);

  float qf[G][8];
  load_query<G>(p.q, p.q_f32, (int64_t)s * p.Hq + (int64_t)g * G, r16, p.qscale, qf);
  float qp[PRIOR ? G : 1][8];
  float mP[G];
  if constexpr (PRIOR) {
    // prior logits use the mean query; shifted by the stored maxP
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      load8f(p.mu_Q + qh * kD + 8 * r16, qp[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qp[h][i] *= p.qscale;
      mP[h] = p.maxP[qh] * kLog2e;
    }
  }

  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);

  float m[G], l[G], acc[G][8];
  float sp[PRIOR ? G : 1], spv[PRIOR ? G : 1][8];
  float ks[8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }
  if constexpr (PRIOR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sp[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) spv[h][i] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ks[i] = 0.f;

  for (int tb = t0; tb < t1; tb += 4 * W * NSB) {
    int off[NSB];
    float lw[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      const int t = tb + 4 * (k * W + w) + sub;
      int o = kOOB;
      float lwk = kNegInf;
      if (t < t1) {
        if constexpr (DENSE) {
          o = row_off<T>(t, p.sn, r16);
          lwk = 0.f;
        } else {
          const int j = p.idx[lbase + t];
          if ((unsigned)j < (unsigned)p.n) {
            o = row_off<T>(j, p.sn, r16);
            lwk = p.logw ? p.logw[lbase + t] * kLog2e : 0.f;
            if (PRIOR && t > 0 && r16 == 0 && p.idx[lbase + t - 1] >= j) flag_unit(p.flags, u, SDA_FLAG_IDX_ORDER);
          } else if (r16 == 0) {
            flag_unit(p.flags, u, SDA_FLAG_IDX_RANGE);
          }
        }
      }
      off[k] = o;
      lw[k] = lwk;
    }
    RowChunk<T> kc[NSB], vc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) buf_load(kc[k], rk, off[k]);
#pragma unroll
    for (int k = 0; k < NSB; ++k) buf_load(vc[k], rv, off[k]);

    float x[NSB][G];
    float pl[PRIOR ? NSB : 1][G];
    float bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) bm[h] = kNegInf;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      float kf[8];
      kc[k].unpack(kf);
      if constexpr (BUILD) {
        if (off[k] != kOOB) {
#pragma unroll
          for (int i = 0; i < 8; ++i) ks[i] += kf[i];
        }
      }
      float a[G];
      dot_heads<G>(qf, kf, a);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        x[k][h] = a[h] + lw[k];
        bm[h] = fmaxf(bm[h], x[k][h]);
      }
      if constexpr (PRIOR) {
        float ap[G];
        dot_heads<G>(qp, kf, ap);
#pragma unroll
        for (int h = 0; h < G; ++h) pl[k][h] = (off[k] == kOOB) ? kNegInf : ap[h] - mP[h];
      }
    }
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], bm[h]);
      alpha[h] = rescale(m[h], mn);
      m[h] = mn;
      l[h] *= alpha[h];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= alpha[h];
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
        if constexpr (PRIOR) {
          const float ep = fast_exp2(pl[k][h]);
          sp[h] += ep;
#pragma unroll
          for (int i = 0; i < 8; ++i) spv[h][i] = fmaf(ep, vf[i], spv[h][i]);
        }
      }
    }
  }

  // ---- merge the four row groups of the wave ----------------------------
#pragma unroll
  for (int msk = 16; msk <= 32; msk <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor(m[h], msk);
      const float mn = fmaxf(m[h], mo);
      const float fa = rescale(m[h], mn), fb = rescale(mo, mn);
      l[h] = l[h] * fa + shfl_xor(l[h], msk) * fb;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * fa + shfl_xor(acc[h][i], msk) * fb;
      m[h] = mn;
      if constexpr (PRIOR) {
        sp[h] += shfl_xor(sp[h], msk);
#pragma unroll
        for (int i = 0; i < 8; ++i) spv[h][i] += shfl_xor(spv[h][i], msk);
      }
    }
    if constexpr (BUILD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ks[i] += shfl_xor(ks[i], msk);
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&s_acc[w][h][8 * r16]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(&s_acc[w][h][8 * r16 + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      if (r16 == 0) {
        s_m[w][h] = m[h];
        s_l[w][h] = l[h];
      }
      if constexpr (PRIOR) {
        *reinterpret_cast<float4*>(&s_spv[w][h][8 * r16]) = make_float4(spv[h][0], spv[h][1], spv[h][2], spv[h][3]);
        *reinterpret_cast<float4*>(&s_spv[w][h][8 * r16 + 4]) = make_float4(spv[h][4], spv[h][5], spv[h][6], spv[h][7]);
        if (r16 == 0) s_sp[w][h] = sp[h];
      }
    }
    if constexpr (BUILD) {
      *reinterpret_cast<float4*>(&s_ks[w][8 * r16]) = make_float4(ks[0], ks[1], ks[2], ks[3]);
      *reinterpret_cast<float4*>(&s_ks[w][8 * r16 + 4]) = make_float4(ks[4], ks[5], ks[6], ks[7]);
    }
  }
  if constexpr (PRIOR) {
    if (p.splits == 1 && w == 0) {
      float c[G];
      bias_shift<G>(p, s, g, r16, qf, c);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_c[h] = c[h];
      }
    }
  }
  __syncthreads();

  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, dim = e - h * kD;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) M = fmaxf(M, s_m[ww][h]);
    float a = 0.f, L = 0.f, SP = 0.f, SPV = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float f = rescale(s_m[ww][h], M);
      a = fmaf(s_acc[ww][h][dim], f, a);
      L = fmaf(s_l[ww][h], f, L);
      if constexpr (PRIOR) {
        SP += s_sp[ww][h];
        SPV += s_spv[ww][h][dim];
      }
    }
    const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
    if (p.splits > 1) {
      float* rec = p.part + (((int64_t)u * p.splits + split) * G + h) * kPartStride;
      if (dim == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = SP;
      }
      rec[4 + dim] = a;
      if constexpr (PRIOR) rec[4 + kD + dim] = SPV;
    } else if constexpr (PRIOR) {
      const Fin f = finalize_prior(M, L, a, s_c[h], mP[h], p.sumP[qh], p.O_est[qh * kD + dim], SP, SPV, p.lambda);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    } else if constexpr (BUILD) {
      // sumP is made relative to the maxP value that decode will read back
      const float maxP = M * kLn2;
      const float corr = fast_exp2(M - maxP * kLog2e);
      p.out[qh * kD + dim] = (L > 0.f) ? a / L : 0.f;
      if (dim == 0) {
        p.lse[qh] = maxP;
        p.aux[qh] = L * corr;
      }
    } else {
      const Fin f = finalize_plain(M, L, a);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    }
  }
  if constexpr (BUILD) {
    for (int dim = tid; dim < kD; dim += 256) {
      float a = 0.f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) a += s_ks[ww][dim];
      if (p.splits > 1) {
        p.ksum[((int64_t)u * p.splits + split) * kD + dim] = a;
      } else {
        p.aux2[(int64_t)u * kD + dim] = a / (float)p.n;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of split partials: one workgroup per unit, fixed split order.
template <int G, int MODE>
__global__ __launch_bounds__(256) void merge_kernel(const AttnParams p) {
  constexpr bool PRIOR = (MODE == kModePrior);
  constexpr bool BUILD = (MODE == kModeBuildPrior);
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float s_c[G];

  if constexpr (PRIOR) {
    if (w == 0) {
      float qf[G][8];
      const int r16 = lane & 15;
      load_query<G>(p.q, p.q_f32, (int64_t)s * p.Hq + (int64_t)g * G, r16, p.qscale, qf);
      float c[G];
      bias_shift<G>(p, s, g, r16, qf, c);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_c[h] = c[h];
      }
    }
    __syncthreads();
  }

  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, dim = e - h * kD;
    const float* base = p.part + ((int64_t)u * p.splits * G + h) * kPartStride;
    const int64_t stride = (int64_t)G * kPartStride;
    float M = kNegInf;
    for (int sp = 0; sp < p.splits; ++sp) M = fmaxf(M, base[sp * stride]);
    float a = 0.f, L = 0.f, SP = 0.f, SPV = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      const float* rec = base + sp * stride;
      const float f = rescale(rec[0], M);
      a = fmaf(rec[4 + dim], f, a);
      L = fmaf(rec[1], f, L);
      if constexpr (PRIOR) {
        SP += rec[2];
        SPV += rec[4 + kD + dim];
      }
    }
    const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
    if constexpr (PRIOR) {
      const float mP = p.maxP[qh] * kLog2e;
      const Fin f = finalize_prior(M, L, a, s_c[h], mP, p.sumP[qh], p.O_est[qh * kD + dim], SP, SPV, p.lambda);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    } else if constexpr (BUILD) {
      const float maxP = M * kLn2;
      const float corr = fast_exp2(M - maxP * kLog2e);
      p.out[qh * kD + dim] = (L > 0.f) ? a / L : 0.f;
      if (dim == 0) {
        p.lse[qh] = maxP;
        p.aux[qh] = L * corr;
      }
    } else {
      const Fin f = finalize_plain(M, L, a);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    }
  }
  if constexpr (BUILD) {
    for (int dim = tid; dim < kD; dim += 256) {
      float a = 0.f;
      for (int sp = 0; sp < p.splits; ++sp) a += p.ksum[((int64_t)u * p.splits + sp) * kD + dim];
      p.aux2[(int64_t)u * kD + dim] = a / (float)p.n;
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers

template <typename T, int G, bool PROXY>
static hipError_t launch_unit_ns(const AttnParams& p, int ns, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  switch (ns) {
    case 4: hipLaunchKernelGGL((sparse_unit_kernel<T, G, PROXY, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((sparse_unit_kernel<T, G, PROXY, 8>), grid, block, 0, st, p); break;
    case 12: hipLaunchKernelGGL((sparse_unit_kernel<T, G, PROXY, 12>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((sparse_unit_kernel<T, G, PROXY, 16>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_unit_g(const AttnParams& p, bool proxy, int ns, hipStream_t st) {
  return proxy ? launch_unit_ns<T, G, true>(p, ns, st) : launch_unit_ns<T, G, false>(p, ns, st);
}

template <typename T>
static hipError_t launch_unit_t(const AttnParams& p, int G, bool proxy, int ns, hipStream_t st) {
  switch (G) {
    case 1: return launch_unit_g<T, 1>(p, proxy, ns, st);
    case 2: return launch_unit_g<T, 2>(p, proxy, ns, st);
    case 4: return launch_unit_g<T, 4>(p, proxy, ns, st);
    case 8: return launch_unit_g<T, 8>(p, proxy, ns, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_unit(const AttnParams& p, int dtype, int G, bool proxy, int ns, hipStream_t st) {
  return dtype == SDA_BF16 ? launch_unit_t<bf16_t>(p, G, proxy, ns, st) : launch_unit_t<float>(p, G, proxy, ns, st);
}

constexpr int kStreamSlots = 4;

template <typename T, int G>
static hipError_t launch_stream_g(const AttnParams& p, int mode, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv * p.splits), block(256);
  switch (mode) {
    case kModeSparse: hipLaunchKernelGGL((stream_kernel<T, G, kModeSparse, kStreamSlots>), grid, block, 0, st, p); break;
    case kModePrior: hipLaunchKernelGGL((stream_kernel<T, G, kModePrior, kStreamSlots>), grid, block, 0, st, p); break;
    case kModeDense: hipLaunchKernelGGL((stream_kernel<T, G, kModeDense, kStreamSlots>), grid, block, 0, st, p); break;
    case kModeBuildPrior:
      hipLaunchKernelGGL((stream_kernel<T, G, kModeBuildPrior, kStreamSlots>), grid, block, 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_stream_t(const AttnParams& p, int G, int mode, hipStream_t st) {
  switch (G) {
    case 1: return launch_stream_g<T, 1>(p, mode, st);
    case 2: return launch_stream_g<T, 2>(p, mode, st);
    case 4: return launch_stream_g<T, 4>(p, mode, st);
    case 8: return launch_stream_g<T, 8>(p, mode, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const AttnParams& p, int dtype, int G, int mode, hipStream_t st) {
  return dtype == SDA_BF16 ? launch_stream_t<bf16_t>(p, G, mode, st) : launch_stream_t<float>(p, G, mode, st);
}

template <int G>
static hipError_t launch_merge_g(const AttnParams& p, int mode, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(256);
  switch (mode) {
    case kModeSparse:
    case kModeDense: hipLaunchKernelGGL((merge_kernel<G, kModeSparse>), grid, block, 0, st, p); break;
    case kModePrior: hipLaunchKernelGGL((merge_kernel<G, kModePrior>), grid, block, 0, st, p); break;
    case kModeBuildPrior: hipLaunchKernelGGL((merge_kernel<G, kModeBuildPrior>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnParams& p, int G, int mode, hipStream_t st) {
  switch (G) {
    case 1: return launch_merge_g<1>(p, mode, st);
    case 2: return launch_merge_g<2>(p, mode, st);
    case 4: return launch_merge_g<4>(p, mode, st);
    case 8: return launch_merge_g<8>(p, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sda
