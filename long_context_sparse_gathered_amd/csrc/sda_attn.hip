// sda_attn.hip -- decode-attention kernels for gfx950.
//
//  sparse_unit_kernel      one 512-thread workgroup per (sequence, KV head),
//                          fp32 rows: gathers every listed K and V row at
//                          once, two-pass softmax with an exact unit maximum,
//                          optional count-aware mean proxies
//                          ("OpenAttention", method stages 04-05: exact rows
//                          and proxies share one softmax).
//  sparse_unit_vt_kernel   the same for bf16 rows with up to four query heads
//                          per KV head: logits and weighted values on the
//                          matrix cores, value rows in registers.
//  sparse_unit_mfma_kernel the same for bf16 rows with eight query heads per
//                          KV head: value tiles staged in LDS.
//  stream_kernel,          split-K streaming kernels with an online softmax;
//  stream_dma_kernel,      they serve plain sparse lists, the rank-1 prior
//  stream_mfma_kernel      ("RESA", Online Aggregator), dense decode and the
//                          prior build ("RESA", Prior Estimator: one extra
//                          query over the whole cache). stream_kernel: fp32
//                          rows and the build; stream_dma_kernel: bf16 plain
//                          lists, prior and dense on the matrix cores, values
//                          staged by direct-to-LDS loads, two batches in
//                          flight per wave; stream_mfma_kernel: bf16
//                          proxy-tail lists longer than one workgroup holds,
//                          each split keeping per-cluster listed counts,
//                          logit sums and value sums.
//  merge_kernel            log-sum-exp merge of split partials + the prior's
//                          delta merge.
//  merge_proxy_kernel      merge of proxy-mode splits: adds the per-cluster
//                          records across splits, forms the proxy entries
//                          and finishes the softmax.
#include "sda_device.hpp"
#include "sda_kernels.hpp"

#include <type_traits>

namespace sda {

constexpr int kRsrcFlags = 0x00020000;
constexpr int kOOB = kMaxUnitBytes;  // byte offset past every unit's rows (loads return 0)

using rsrc_t = __amdgpu_buffer_rsrc_t;

template <typename T>
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t n, int64_t sn) {
  const int64_t bytes = ((int64_t)(n - 1) * sn + kD) * (int64_t)sizeof(T);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// Streaming cache policy for rows read once per step (the non-temporal bit
// of the buffer load): measured about 10% faster than the default policy for
// gathers of random 256-byte rows.
constexpr int kLoadNT = 2;

// Gather one row chunk through a range-checked buffer resource: an offset
// outside the resource returns zeros and touches no memory.
__device__ __forceinline__ void buf_load(RowChunk<bf16_t>& c, rsrc_t r, int off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNT);
  c.raw = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buf_load(RowChunk<float>& c, rsrc_t r, int off) {
  auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNT);
  auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kLoadNT);
  c.a = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
  c.b = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
}

template <typename T>
__device__ __forceinline__ int row_off(int64_t j, int64_t sn, int r16) {
  return (int)((j * sn + 8 * r16) * (int64_t)sizeof(T));
}

// Load the G query heads of KV head g (dims 8*r16..) scaled to log2 units.
template <typename QT, int G>
__device__ __forceinline__ void load_query(const void* q, int64_t row0, int r16, float qscale, float (&qf)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load_q8<QT>(q, (row0 + h) * kD + 8 * r16, qf[h]);
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

__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, 64); }
// DPP move within 16-lane rows; lanes whose source lies outside the row
// receive zero.
template <int CTRL>
__device__ __forceinline__ float dppz(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// 4 x 4 transpose of (row group, register): out[j] of row group r is in[r]
// of row group j. v_permlane32_swap exchanges row groups 2-3 of its first
// operand with 0-1 of its second, v_permlane16_swap the odd row groups of
// the first with the even ones of the second.
__device__ __forceinline__ void transpose_rows(const float (&in)[4], float (&out)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(in[0]), __float_as_uint(in[2]), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(in[1]), __float_as_uint(in[3]), false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  out[0] = __uint_as_float(c[0]);
  out[1] = __uint_as_float(c[1]);
  out[2] = __uint_as_float(d[0]);
  out[3] = __uint_as_float(d[1]);
}
// Integer DPP move within 16-lane rows; lanes whose source lies outside the
// row receive `edge`.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v, int edge) {
  return __builtin_amdgcn_update_dpp(edge, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float shfl_f(float v, int src) { return __shfl(v, src, 64); }

// ---------------------------------------------------------------------------
// One workgroup per unit.  Wave w owns list entries [w*CH, (w+1)*CH): lane l
// loads entry w*CH + l, and slot k of the wave's row group `sub` takes entry
// 4k + sub by a lane shuffle.  Every load that does not depend on another
// load is issued in the prologue, the row gathers right after the list
// arrives, and all checks run while the rows are in flight.
template <typename T, int G, bool PROXY, int NS>
__global__ __launch_bounds__(512) void sparse_unit_kernel(const AttnParams p) {
  constexpr int W = kUnitWaves;
  constexpr int PC = PROXY ? kCmax : 1;
  constexpr int PW = PROXY ? W : 1;
  constexpr int R = PROXY ? (kCmax * G + 63) / 64 : 1;  // (cluster, head) pairs per lane in wave 0
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int CH = p.chunk;

  __shared__ float s_wmax[W][G];
  __shared__ float s_M[G];
  __shared__ float s_pl[G];
  __shared__ float s_l[W][G];
  __shared__ __attribute__((aligned(16))) float s_red[W][G][kD];
  __shared__ float s_csum[PW][PC][G];
  __shared__ int s_ccnt[PW][PC];
  __shared__ float s_qk[PC][G];
  __shared__ float s_cw[PC][G];

  // ---- prologue ------------------------------------------------------------
  float qf[G][8];
  load_query<T, G>(p.q, (int64_t)s * p.Hq + (int64_t)g * G, r16, p.qscale, qf);

  const int64_t lbase = (int64_t)u * p.m;
  const int e = w * CH + lane;
  const bool in_list = (lane < CH) && (e < p.m);
  int li = -1, lp = -1, lc = -1;
  float lwv = 0.f;
  if (p.m > 0) {
    const int64_t ea = lbase + (in_list ? e : 0);
    li = p.idx[ea];
    if constexpr (PROXY) {
      lp = p.idx[lbase + ((in_list && e > 0) ? e - 1 : 0)];
      if (p.idx_cluster) lc = p.idx_cluster[ea];
    }
    if (p.logw) lwv = p.logw[ea];
  }

  float skf[8], svf[8];
  int cnt[R];
  const int b0 = 4 * w + sub;  // this row group's first cluster slot
  if constexpr (PROXY) {
    const int64_t rb = ((int64_t)u * p.C + (b0 < p.C ? b0 : 0)) * kD + 8 * r16;
    load8f(p.sumK + rb, skf);
    load8f(p.sumV + rb, svf);
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int b = (lane + 64 * r) / G;
        cnt[r] = p.count[(int64_t)u * p.C + (b < p.C ? b : 0)];
      }
    }
  }

  int len = p.m;
  if (p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    len = L;
  }

  // ---- row addresses from the list ----------------------------------------
  const bool live = in_list && e < len;
  const bool in_range = (unsigned)li < (unsigned)p.n;
  const bool valid = live && in_range;
  const bool bad_cluster = PROXY && p.idx_cluster && valid && (lc < -1 || lc >= p.C);
  if (bad_cluster) lc = -1;

  int off[NS];
  float lw[NS];
  int cl[NS];
  const bool lookup = PROXY && !p.idx_cluster;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int src = 4 * k + sub;
    const int j = shfl_i(li, src);
    const bool ok = shfl_i(valid ? 1 : 0, src) != 0;
    off[k] = ok ? row_off<T>(j, p.sn, r16) : kOOB;
    lw[k] = ok ? shfl_f(lwv, src) * kLog2e : kNegInf;
    if constexpr (PROXY) cl[k] = ok ? (lookup ? j : shfl_i(lc, src)) : -1;
  }
  if constexpr (PROXY) {
    if (lookup) {
      const int32_t* crow = p.cluster_id + (int64_t)u * p.n;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int c = crow[cl[k] >= 0 ? cl[k] : 0];   // unconditional load, selected after
        cl[k] = (off[k] != kOOB) ? c : -1;
      }
    }
  }

  // ---- gather every listed row ----------------------------------------------
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);
  RowChunk<T> kc[NS], vc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) buf_load(kc[k], rk, off[k]);
#pragma unroll
  for (int k = 0; k < NS; ++k) buf_load(vc[k], rv, off[k]);

  // ---- checks and proxy preparation while the rows are in flight ----------
  {
    int bad = 0;
    if (live && !in_range) bad |= SDA_FLAG_IDX_RANGE;
    if (PROXY && live && e > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
    if (bad_cluster) bad |= SDA_FLAG_CLUSTER;
    if (bad) flag_unit(p.flags, u, bad);
  }
  if constexpr (PROXY) {
#pragma unroll
    for (int i = lane; i < PC * G; i += 64) (&s_csum[w][0][0])[i] = 0.f;
    for (int i = lane; i < PC; i += 64) s_ccnt[w][i] = 0;
    float a[G];
    dot_heads<G>(qf, skf, a);
    if (b0 < p.C) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (r16 == h) s_qk[b0][h] = a[h];
    }
    if (p.C > 4 * W) {  // second cluster slot (C > 32)
      const int b1 = b0 + 4 * W;
      if (b1 < p.C) {
        float sk1[8];
        load8f(p.sumK + ((int64_t)u * p.C + b1) * kD + 8 * r16, sk1);
        dot_heads<G>(qf, sk1, a);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (r16 == h) s_qk[b1][h] = a[h];
      }
    }
  }

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
      if (cl[k] < -1 || cl[k] >= p.C) {
        if (r16 == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
        cl[k] = -1;
      }
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
      const int h = lane % G;
      float pi[R], nbf[R];
      float hm = kNegInf;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int b = (lane + 64 * r) / G;
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
          const int nb = cnt[r] - rc;
          if (nb < 0 && h == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
          if (nb > 0) {
            nbf[r] = (float)nb;
            pi[r] = (s_qk[b][h] - ssum) / nbf[r] + __builtin_amdgcn_logf(nbf[r]);
          }
        }
        hm = fmaxf(hm, pi[r]);
      }
#pragma unroll
      for (int msk = G; msk < 64; msk <<= 1) hm = fmaxf(hm, shfl_xor(hm, msk));
#pragma unroll
      for (int ww = 0; ww < W; ++ww) hm = fmaxf(hm, s_wmax[ww][h]);
      const float M = (hm == kNegInf) ? 0.f : hm;
      float pe = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int b = (lane + 64 * r) / G;
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
      const float ev = fast_exp2(x[k][h] - M[h]);
      l[h] += ev;
      wt[h] = ev;
    }
    if constexpr (PROXY) {
      // a read member leaves its cluster: subtract its share of the proxy's
      // value term (the proxy below adds cw * the sum of all member values)
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
  if constexpr (PROXY) {
    // proxy value terms: cw_b * (sum of the cluster's values)
    if (b0 < p.C) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float cw = s_cw[b0][h];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(cw, svf[i], acc[h][i]);
      }
    }
    if (p.C > 4 * W) {
      const int b1 = b0 + 4 * W;
      if (b1 < p.C) {
        float sv1[8];
        load8f(p.sumV + ((int64_t)u * p.C + b1) * kD + 8 * r16, sv1);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float cw = s_cw[b1][h];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(cw, sv1[i], acc[h][i]);
        }
      }
    }
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

  for (int ei = tid; ei < G * kD; ei += 512) {
    const int h = ei / kD, dim = ei - h * kD;
    float a = 0.f, L = s_pl[h];
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      a += s_red[ww][h][dim];
      L += s_l[ww][h];
    }
    const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
    p.out[qh * kD + dim] = (L > 0.f) ? a / L : 0.f;
    if (dim == 0 && p.lse) p.lse[qh] = (L > 0.f) ? (s_M[h] + log2f(L)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// bf16 variant of the one-workgroup-per-unit kernel, both products on the
// matrix cores.
//
// Logits: v_mfma_f32_16x16x32_bf16 multiplies the (zero-padded) 16 x 128
// query block of the KV group by 16 gathered keys.  The 128-long reduction is
// split into four steps; in step st, lane group qg = lane >> 4 supplies dims
// 32*st + 8*qg .. +8, so every load instruction reads 64 contiguous bytes of
// each of 16 keys.  Lane l then holds the logits of key l & 15 for heads
// 4*(l >> 4) + i (accumulator element i).
//
// Tail preparation is spread over the waves: wave w owns clusters 4w + qg and
// 4w + qg + 32 and computes their mean logits; the unit maximum comes from the
// per-wave maxima of the read logits and of the proxy logits.
//
// From the logits to the weights each (head, key) pair sits in one lane (the
// key layout); the weighted values take one v_mfma_f32_16x16x32_bf16 per two
// tiles of 16 keys and 16 dims (see the value phase below).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediate: vector memory count 0, the other counters unrestricted.
constexpr int kWaitVmem0 = 0x0F70;
// A value tile: 16 rows of 128 bf16 (256 bytes) in LDS.
constexpr int kVTile = 16 * 256;
// Position of 16-byte chunk c of tile row r: rows 4q..4q+3 spread a chunk pair
// over 4 x 32 bytes, and odd row quads use the other half of the banks.
__device__ __forceinline__ int vt_chunk(int r, int c) { return c ^ (2 * (r & 3)) ^ (8 * ((r >> 2) & 1)); }
// Workgroup barrier over LDS data only: each wave waits for its own LDS
// operations, while loads that write LDS directly stay in flight (the fence of
// __syncthreads would wait for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// LDS atomic adds without a return value. Written out so that the compiler
// does not order them behind the loads that fill the value tiles (it treats
// them as possibly overlapping those); the targets here never do.
__device__ __forceinline__ void lds_add(float* p, float v) {
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)p;
  asm volatile("ds_add_f32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add(int* p, int v) {
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// A 16-bit LDS store, written out for the same reason.
__device__ __forceinline__ void lds_store(unsigned char* p, __bf16 v) {
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)p;
  const unsigned x = __builtin_bit_cast(unsigned short, v);
  asm volatile("ds_write_b16 %0, %1" ::"v"(a), "v"(x) : "memory");
}

template <int G, bool PROXY, int NT>
__global__ __launch_bounds__(512) void sparse_unit_mfma_kernel(const AttnParams p) {
  constexpr int W = kUnitWaves;
  constexpr int NS = 4 * NT;   // value slots per wave
  constexpr int KW = 16 * NT;  // list entries per wave
  constexpr int PC = PROXY ? kCmax : 1;
  constexpr int PW = PROXY ? W : 1;
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int CH = p.chunk;      // entries of this wave: [w*CH, (w+1)*CH), CH <= KW
  const int hr = r16 < G ? r16 : 0;  // head of this lane in the [head][..] layouts (clamped)

  constexpr int NV = G < 4 ? 1 : G / 4;  // heads per lane in the key layout
  constexpr int NP = (NT + 1) / 2;       // key tile pairs (the last may be single)
  constexpr int NBT = NT + (PROXY ? 1 : 0);  // value tiles per wave, the cluster-sum tile last
  constexpr int NPW = (NBT + 1) / 2;         // their pairs
  // Per-wave results, the wave index last so that a lane reads all waves'
  // values of one head or cluster with two 16-byte loads.
  static_assert(W % 4 == 0, "per-wave results are read four at a time");
  __shared__ __attribute__((aligned(16))) float s_wmax[G][W];
  __shared__ __attribute__((aligned(16))) float s_pmax[G][PW];
  __shared__ float s_M[G];
  __shared__ __attribute__((aligned(16))) float s_l[G][W];   // normaliser: the wave's keys
  __shared__ __attribute__((aligned(16))) float s_lp[G][PW]; // and its proxies
  __shared__ __attribute__((aligned(16))) float s_csum[PC][G][PW];
  __shared__ __attribute__((aligned(16))) int s_ccnt[PC][PW];
  // mean logit of a cluster's unread members (-inf if none), per head; entry
  // PC is a -inf sentinel for keys outside every cluster (rows padded to 16
  // bytes)
  __shared__ __attribute__((aligned(16))) float s_mu[G][PC + 4];
  // Weights handed from the key layout to the matrix-core layout: per wave,
  // bf16 high part (0) and remainder (1), per pair of key tiles, head and
  // group of four keys, 16 bytes: four keys of the even tile, then four of
  // the odd one.
  __shared__ __attribute__((aligned(16))) unsigned char s_wt[W][2][NPW][G][4][16];
  // The value loads' list entries, handed from the key loads' lanes: entry
  // 16t + 4kq + sub at [w][t][sub][kq].
  __shared__ __attribute__((aligned(16))) int s_jv[W][NT][4][4];
  // Value tiles, written by the row loads straight into LDS: per wave NT
  // tiles of 16 rows x 256 bytes, 16-byte chunks swizzled (vt_chunk) so that
  // the transposed reads are free of bank conflicts. After the products, tile
  // 0 of each wave holds the wave's partial sums (and, when the cluster-sum
  // tile has no buffer of its own, that tile before them).
  __shared__ __attribute__((aligned(16))) unsigned char s_vt[W][NT][kVTile];
  // The cluster-sum tile (below) gets a per-wave buffer of its own where it
  // fits next to the value tiles, so that it is written and read while the
  // rows are still in flight; otherwise it reuses tile 0 late.
  constexpr int kLdsOther =
      (2 * W * G + PW * G + G + PW * PC * G + PW * PC + (PC + 1) * G) * 4 + W * 2 * NPW * G * 64 + W * NT * 64 + 256;
  constexpr bool SEP = PROXY && (W * (NT + 1) * kVTile + kLdsOther <= 160 * 1024);
  __shared__ __attribute__((aligned(16))) unsigned char s_pt[SEP ? W : 1][SEP ? kVTile : 16];

  // ---- prologue ------------------------------------------------------------
  // Every load that does not depend on the list is issued before the first
  // use of any loaded value, in one branch-free block: the query, the list
  // entries and the cluster sums share a single memory round trip. (With no
  // list, and for absent optional arrays, the loads read a valid dummy
  // address and the values are discarded.)
  const int64_t lbase = (int64_t)u * p.m;
  const int e = w * CH + lane;
  const bool in_list = (lane < CH) && (e < p.m);
  const int32_t* lst = p.m > 0 ? p.idx : reinterpret_cast<const int32_t*>(p.q);
  const int64_t ea = lbase + (in_list ? e : 0);
  int li = lst[ea];
  int lp = -1, lc = -1;
  if constexpr (PROXY) {
    lp = lst[lbase + ((in_list && e > 0) ? e - 1 : 0)];
    lc = (p.idx_cluster ? p.idx_cluster : lst)[ea];
  }
  const float lwv = (p.logw ? p.logw : reinterpret_cast<const float*>(lst))[ea];
  // the key rows this lane fetches: entry 16t + r16 of tile t, read straight
  // from the list (no shuffle round trip)
  auto entry = [&](int pos) { return w * CH + pos; };
  auto listed = [&](int pos) { return pos < CH && entry(pos) < p.m; };
  int jk[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) jk[t] = lst[lbase + (listed(16 * t + r16) ? entry(16 * t + r16) : 0)];

  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;
  uint4 qa[4];  // MFMA A operand: head r16 (zero past G), dims 32*st + 8*sub
#pragma unroll
  for (int st = 0; st < 4; ++st)
    qa[st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + hr) * kD + 32 * st +
                                             8 * sub);
  float qf[PROXY ? G : 1][8];  // row-layout query for the cluster-sum logits
  if constexpr (PROXY) load_query<bf16_t, G>(p.q, qrow0, r16, p.qscale, qf);

  // cluster sums and counts of the two clusters this lane owns: b0 = 4w + sub
  // and b1 = b0 + 32 (dims 8*r16 .. +8 of the sums)
  const int b0 = 4 * w + sub, b1 = b0 + 4 * W;
  const bool has0 = PROXY && b0 < p.C, has1 = PROXY && b1 < p.C;
  float skf[8], svf[8], sk1[8], sv1[8];
  int cnt0 = 0, cnt1 = 0;
  if constexpr (PROXY) {
    const int64_t c0 = (int64_t)u * p.C + (has0 ? b0 : 0);
    load8f(p.sumK + c0 * kD + 8 * r16, skf);
    load8f(p.sumV + c0 * kD + 8 * r16, svf);
    cnt0 = p.count[c0];
    if (has1) {
      const int64_t c1 = (int64_t)u * p.C + b1;
      load8f(p.sumK + c1 * kD + 8 * r16, sk1);
      load8f(p.sumV + c1 * kD + 8 * r16, sv1);
      cnt1 = p.count[c1];
    }
  }

  int len = p.m;
  if (p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    len = L;
  }

  // ---- addresses ------------------------------------------------------------
  // The unit's rows span less than 2^31 bytes (checked on the host), so byte
  // offsets are 32-bit; an absent row reads past the resource and returns
  // zeros.
  const bool live = in_list && e < len;
  const bool in_range = (unsigned)li < (unsigned)p.n;
  const bool valid = live && in_range;
  const int rs = 2 * (int)p.sn;
  // (an unpredictable select keeps each product unconditional: left to
  // itself the compiler branches around it)
  auto row_byte = [&](int pos, int j, int c) {
    const bool ok = (pos < CH) & (entry(pos) < len) & ((unsigned)j < (unsigned)p.n);
    return __builtin_unpredictable(ok) ? j * rs + c : kOOB;
  };
  int koff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = row_byte(16 * t + r16, jk[t], 16 * sub);
  // value slot k = 4t + kq (entry 16t + 4kq + sub) fills tile t, rows
  // 4kq .. 4kq+3: lane (sub, r16) lands at row 4kq + sub, chunk position r16,
  // so it fetches the chunk that the swizzle puts there. The entries come
  // from the key lanes through LDS (the value loads are issued late, so the
  // round trip hides behind the key loads).
  if (sub == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) s_jv[w][t][r16 & 3][r16 >> 2] = jk[t];
  }
  wave_lds_sync();
  int voff[NS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int4 j4 = *reinterpret_cast<const int4*>(&s_jv[w][t][sub][0]);
    const int jv[4] = {j4.x, j4.y, j4.z, j4.w};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const int k = 4 * t + kq;
      voff[k] = row_byte(4 * k + sub, jv[kq], 16 * vt_chunk(4 * kq + sub, r16));
    }
  }

  // cluster of this lane's entry from the per-row ids when the list carries
  // none: issued ahead of the row loads, so that its use does not wait for
  // them (loads complete in issue order)
  if constexpr (PROXY) {
    if (!p.idx_cluster) lc = valid ? p.cluster_id[(int64_t)u * p.n + li] : -1;
  }

  // ---- row loads (streaming: read once) -------------------------------------
  // Keys first; the work below that needs no row runs while they are in
  // flight (the memory queues are full by then), and the value loads follow.
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);
  uint4 kt[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[t] + 64 * st, 0, kLoadNT);
      kt[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
  for (int st = 0; st < 4; ++st)
    if (r16 >= G) qa[st] = make_uint4(0, 0, 0, 0);

  // ---- checks and cluster lookups, behind the key loads ---------------------
  const float lw_own = valid ? (p.logw ? lwv * kLog2e : 0.f) : kNegInf;
  const bool bad_cluster = PROXY && p.idx_cluster && valid && (lc < -1 || lc >= p.C);
  if (bad_cluster) lc = -1;
  {
    int bad = 0;
    if (live && !in_range) bad |= SDA_FLAG_IDX_RANGE;
    if (PROXY && live && e > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
    if (bad_cluster) bad |= SDA_FLAG_CLUSTER;
    if (bad) flag_unit(p.flags, u, bad);
  }
  if constexpr (PROXY) {
    if (!has0) cnt0 = 0;
    if (!has1) {
      cnt1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sk1[i] = sv1[i] = 0.f;
    }
  }
  float qk0 = 0.f, qk1 = 0.f;  // q . (sum of keys) of clusters b0, b1 for head r16
  if constexpr (PROXY) {
#pragma unroll
    for (int i = lane; i < PC * G; i += 64) s_csum[i / G][i % G][w] = 0.f;
    for (int i = lane; i < PC; i += 64) s_ccnt[i][w] = 0;
    float a[G];
    dot_heads<G>(qf, skf, a);
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (r16 == h) qk0 = a[h];
    if (has1) {
      dot_heads<G>(qf, sk1, a);
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (r16 == h) qk1 = a[h];
    }
  }

  // Transposed tile reads (see the value phase) and the cluster-sum tile's
  // rows: row `row` of a tile holds the bf16 high part (lo = false) or
  // remainder of the eight sums of this lane's dims.
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const int tr_row = 4 * sub + (r16 >> 2);
  auto tile_read = [&](const unsigned char* tile, bf16x4_t (&b)[8]) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      auto src = (__attribute__((address_space(3))) bf16x4_t*)(tile + tr_row * 256 +
                                                               16 * vt_chunk(tr_row, 2 * nb + ((r16 & 3) >> 1)) +
                                                               8 * (r16 & 1));
      b[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src);
    }
  };
  auto put = [&](unsigned char* ct, int row, const float (&f)[8], bool lo) {
    bf16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 hi = (__bf16)f[i];
      v[i] = lo ? (__bf16)(f[i] - (float)hi) : hi;
    }
    *reinterpret_cast<bf16x8_t*>(ct + row * 256 + 16 * vt_chunk(row, r16)) = v;
  };
  auto put_cluster_tile = [&](unsigned char* ct) {
    put(ct, sub, svf, false);
    put(ct, 4 + sub, svf, true);
    put(ct, 8 + sub, sv1, false);
    put(ct, 12 + sub, sv1, true);
  };
  // the cluster-sum tile's B operand; with a buffer of its own it is built
  // now, while the rows are in flight
  bf16x4_t bc[8];
  if constexpr (SEP) {
    put_cluster_tile(&s_pt[w][0]);
    wave_lds_sync();  // the tile's rows, written by other lanes
    tile_read(&s_pt[w][0], bc);
  }

  // ---- per key tile: log-weight and cluster of this lane's key -------------
  // (key layout, below) and the controls of the segmented sums over runs of
  // keys with the same cluster (consecutive lanes of a row group). The read
  // members' counts per cluster are added here; their logit sums follow the
  // logits.
  float lwk[NT];
  int cmr[NT];  // cluster of the key, -1 if none
  float sf[NT][4];
  bool run_end[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int kk = 16 * t + r16;  // this lane's key within the wave's entries
    lwk[t] = shfl_f(lw_own, kk);
    cmr[t] = -1;
    run_end[t] = false;
    if constexpr (PROXY) {
      const int ck = shfl_i(lc, kk);
      const int cm = (lwk[t] != kNegInf && ck >= 0 && ck < p.C) ? ck : -1;
      cmr[t] = cm;
      // run start: the first lane of the row group, or a change of cluster
      // from the lane before; then a max-scan gives each lane its run's start
      const int cprev = dpp_i<0x111>(cm, -2), cnext = dpp_i<0x101>(cm, -2);  // row_shr:1, row_shl:1
      int start = cprev != cm ? r16 : 0;
      start = max(start, dpp_i<0x111>(start, 0));
      start = max(start, dpp_i<0x112>(start, 0));
      start = max(start, dpp_i<0x114>(start, 0));
      start = max(start, dpp_i<0x118>(start, 0));
      // 0/1 factors of the Hillis-Steele steps: a step takes the partial of
      // the lane s back only while that lane is in the same run
      sf[t][0] = r16 - 1 >= start ? 1.f : 0.f;
      sf[t][1] = r16 - 2 >= start ? 1.f : 0.f;
      sf[t][2] = r16 - 4 >= start ? 1.f : 0.f;
      sf[t][3] = r16 - 8 >= start ? 1.f : 0.f;
      run_end[t] = cm >= 0 && cnext != cm;  // last lane of a run
      if (run_end[t] && sub == 0) lds_add(&s_ccnt[cm][w], r16 - start + 1);
    }
  }

  // ---- value rows, straight into LDS ----------------------------------------
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int off = voff[k];  // (a plain local: the host pass mishandles an array element here)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)&s_vt[w][k >> 2][(k & 3) * 1024],
                                             16, off, 0, 0, kLoadNT);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- logits on the matrix cores ------------------------------------------
  // The MFMA leaves lane (key r16, group sub) the logits of heads 4*sub + i;
  // a 4 x 4 transpose of row groups turns that into the key layout used from
  // here to the weights: lane (sub, r16) holds heads 4j + sub (j < NV) of key
  // 16t + r16 of tile t, so each (head, key) pair sits in one lane only.
  float xr[NT][NV];  // logit plus log-weight (log2 units)
  float mxr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) mxr[j] = kNegInf;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                  __builtin_bit_cast(bf16x8_t, kt[t][st]), d, 0, 0, 0);
    float sv[4], hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = d[i] * p.qscale;
    transpose_rows(sv, hv);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      xr[t][j] = hv[j] + lwk[t];
      mxr[j] = fmaxf(mxr[j], xr[t][j]);
    }
    if constexpr (PROXY) {
      // read members' logit sums per cluster (this wave's slice): inclusive
      // sums within runs (every lane takes part in every move: a 0/1 factor,
      // not a branch, since a move must not read a lane that sits out; the
      // partials are finite); the last lane of each run adds the run total
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float x = hv[j];
        x = fmaf(sf[t][0], dppz<0x111>(x), x);
        x = fmaf(sf[t][1], dppz<0x112>(x), x);
        x = fmaf(sf[t][2], dppz<0x114>(x), x);
        x = fmaf(sf[t][3], dppz<0x118>(x), x);
        hv[j] = x;
      }
      if (run_end[t]) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (4 * j + sub < G) lds_add(&s_csum[cmr[t]][4 * j + sub][w], hv[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float v = max16(mxr[j]);
    if (r16 == 0 && 4 * j + sub < G) s_wmax[4 * j + sub][w] = v;
  }
  lds_barrier();

  // ---- rows of the value products ------------------------------------------
  // With at most four heads, rows 0 .. G-1 of the value products' A operand
  // take the weights' bf16 high parts and rows G .. 2G-1 their remainders (one
  // product covers both; the two row sets are added in the combine);
  // otherwise row h takes head h and the two parts take one product each.
  // This lane's row: head ah, part al (rows past those: any finite weights,
  // their outputs are dropped).
  constexpr bool HLR = G <= 4;
  const int ah = HLR ? (r16 < G ? r16 : (r16 < 2 * G ? r16 - G : 0)) : hr;
  const int al = HLR && r16 >= G && r16 < 2 * G ? 1 : 0;

  // ---- proxy logits of the clusters this wave owns ------------------------
  // Unread members of cluster b: n_b = count - (read members); their mean
  // logit mu_b = (q.sumK_b - sum of the read members' logits) / n_b; the
  // proxy logit is mu_b + log2(n_b). Every read of this phase is issued at
  // once (branch-free; both clusters' rows exist for every lane).
  float4 wm4[W / 4], a04[W / 4], a14[W / 4];
  int4 n04[W / 4], n14[W / 4];
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    wm4[q] = *reinterpret_cast<const float4*>(&s_wmax[ah][4 * q]);
    if constexpr (PROXY) {
      a04[q] = *reinterpret_cast<const float4*>(&s_csum[b0][hr][4 * q]);
      a14[q] = *reinterpret_cast<const float4*>(&s_csum[b1][hr][4 * q]);
      n04[q] = *reinterpret_cast<const int4*>(&s_ccnt[b0][4 * q]);
      n14[q] = *reinterpret_cast<const int4*>(&s_ccnt[b1][4 * q]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // (every read above in flight before the first use)
  float Mk = kNegInf;  // maximum of the read logits, head ah
#pragma unroll
  for (int q = 0; q < W / 4; ++q) Mk = fmaxf(Mk, fmaxf(fmaxf(wm4[q].x, wm4[q].y), fmaxf(wm4[q].z, wm4[q].w)));
  float pi0 = kNegInf, pi1 = kNegInf;
  bool neg_count = false;  // more read members than the cluster holds
  if constexpr (PROXY) {
    float cs0 = 0.f, cs1 = 0.f;
    int rc0 = 0, rc1 = 0;
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      cs0 += (a04[q].x + a04[q].y) + (a04[q].z + a04[q].w);
      cs1 += (a14[q].x + a14[q].y) + (a14[q].z + a14[q].w);
      rc0 += n04[q].x + n04[q].y + n04[q].z + n04[q].w;
      rc1 += n14[q].x + n14[q].y + n14[q].z + n14[q].w;
    }
    auto mean_logit = [&](int b, bool has, float qk, int cntb, float cs, int rc, float& pi) {
      const int nb = cntb - rc;
      neg_count |= has && nb < 0 && r16 == 0;
      const bool ok = has && nb > 0;
      const float nbf = (float)(ok ? nb : 1);
      const float mu = ok ? (qk - cs) * __builtin_amdgcn_rcpf(nbf) : kNegInf;  // (hardware reciprocal, ~1 ulp)
      pi = (ok && r16 < G) ? mu + __builtin_amdgcn_logf(nbf) : kNegInf;
      if (r16 < G) s_mu[r16][b] = mu;
    };
    mean_logit(b0, has0, qk0, cnt0, cs0, rc0, pi0);
    mean_logit(b1, has1, qk1, cnt1, cs1, rc1, pi1);
    if (w == 0 && sub == 0 && r16 < G) s_mu[r16][PC] = kNegInf;
    const float pm = max_rowgroups(fmaxf(pi0, pi1));
    if (sub == 0 && r16 < G) s_pmax[r16][w] = pm;
    lds_barrier();
    if (neg_count) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  }

  // ---- unit maximum (every wave, same value) --------------------------------
  // and the cluster means the weights need, in the same LDS round trip
  float mus[NT][NV], cmu[4];
  if constexpr (PROXY) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NV; ++j) mus[t][j] = s_mu[4 * j + sub < G ? 4 * j + sub : 0][cmr[t] >= 0 ? cmr[t] : PC];
    const float4 c4 = *reinterpret_cast<const float4*>(&s_mu[ah][4 * w + (sub >= 2 ? 4 * W : 0)]);
    cmu[0] = c4.x;
    cmu[1] = c4.y;
    cmu[2] = c4.z;
    cmu[3] = c4.w;
  }
  float Mh = Mk;  // head ah (= hr where r16 < G)
  if constexpr (PROXY) {
#pragma unroll
    for (int ww = 0; ww < W; ww += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(&s_pmax[ah][ww]);
      Mh = fmaxf(Mh, fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w)));
    }
  }
  if (Mh == kNegInf) Mh = 0.f;
  if (w == 0 && sub == 0 && r16 < G) s_M[r16] = Mh;
  float Mr[NV];  // the same in the key layout: head 4j + sub
#pragma unroll
  for (int j = 0; j < NV; ++j) Mr[j] = shfl_f(Mh, 4 * j + sub < G ? 4 * j + sub : 0);

  // ---- weights, in the key layout -------------------------------------------
  // w = exp2(x - M), minus exp2(mu_b - M) for a read member of cluster b
  // (whose value the proxy term counts in the cluster's sum), stored as a
  // bf16 high part and a bf16 remainder for the value products.
  float lsr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) lsr[j] = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int h = 4 * j + sub;
      const float ev = fast_exp2(xr[t][j] - Mr[j]);
      lsr[j] += ev;
      float wv = ev;
      if constexpr (PROXY) wv = ev - fast_exp2(mus[t][j] - Mr[j]);
      const __bf16 hi = (__bf16)wv;
      const __bf16 lo = (__bf16)(wv - (float)hi);
      if (h < G) {
        const int at = 8 * (t & 1) + 2 * (r16 & 3);
        lds_store(&s_wt[w][0][t >> 1][h][r16 >> 2][at], hi);
        lds_store(&s_wt[w][1][t >> 1][h][r16 >> 2][at], lo);
      }
    }
  }
  // the proxies' share of the normaliser (lanes of head r16, clusters b0, b1;
  // exp2(-inf) = 0 for the absent ones)
  float lsum = 0.f;
  float cws[4] = {0.f, 0.f, 0.f, 0.f};  // cluster-tile weights of the rows below
  const bool head_lane = r16 < (HLR ? 2 * G : G);
  if constexpr (PROXY) {
    lsum = fast_exp2(pi0 - Mh) + fast_exp2(pi1 - Mh);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 4 * w + j + (sub >= 2 ? 4 * W : 0);
      cws[j] = fast_exp2(((head_lane && b < p.C) ? cmu[j] : kNegInf) - Mh);
    }
  }

  // ---- weighted values on the matrix cores ---------------------------------
  // v_mfma_f32_16x16x32_bf16 with the values as B: ds_read_b64_tr_b16 gives
  // lane n of group sub the tile rows 4*sub .. 4*sub+3 at column 16*nb + n
  // when lane s of the group points at row 4*sub + s/4, column
  // 16*nb + 4*(s%4). Two tiles share a product: B holds the four rows of
  // tile a (elements 0-3) and of tile b (4-7), A (lane m = row, group sub)
  // the matching weights of the row's head and part (about 16 significant
  // bits of each weight, exact bf16 x bf16 products, fp32 accumulation). A
  // lone tile repeats its rows in both halves, with zero weights in the
  // second (with one row per head, its high parts and remainders go in the
  // two halves instead). The cluster-sum tile is the last tile: rows sub and
  // 4 + sub hold the high part and remainder of cluster b0's value sum, rows
  // 8 + sub and 12 + sub those of cluster b1 (zero when absent), weighted
  // exp2(mu_b - M).
  bf16x4_t chi, clo;  // cluster-tile weights, high parts and remainders
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    chi[j] = (__bf16)cws[j];
    clo[j] = (__bf16)(cws[j] - (float)chi[j]);
  }
  // With the cluster-sum tile in a buffer of its own (or none), each wave
  // computes 16 of the 128 output dims over the keys of every wave: the
  // products then sum across waves in the matrix cores, and no partials
  // pass through LDS. Otherwise each wave takes all dims of its own keys and
  // the waves' partials are added in a combine.
  constexpr bool DIMS = !PROXY || SEP;
  if constexpr (DIMS) {
    static_assert(W * 16 == kD, "one 16-dim block per wave");
    // ---- everything the other waves read: normalisers, cluster weights ----
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int h = 4 * j + sub;
      const float tot = sum16(lsr[j]);
      if (r16 == 0 && h < G) s_l[h][w] = tot;
    }
    if constexpr (PROXY) {
      lsum = sum_rowgroups(lsum);
      if (sub == 0 && r16 < G) s_lp[r16][w] = lsum;
      // the cluster-sum tile's weights go in the weight slots as tile NT
      unsigned char* cs = &s_wt[w][0][NT >> 1][0][sub][8 * (NT & 1)];
      constexpr int hstep = sizeof(s_wt[0][0][0][0]);
      constexpr int pstep = sizeof(s_wt[0][0]);
      if constexpr (HLR) {
        if (head_lane) *reinterpret_cast<bf16x4_t*>(cs + al * pstep + ah * hstep) = al ? clo : chi;
      } else if (r16 < G) {
        *reinterpret_cast<bf16x4_t*>(cs + r16 * hstep) = chi;
        *reinterpret_cast<bf16x4_t*>(cs + pstep + r16 * hstep) = clo;
      }
    }
    if constexpr (NBT % 2 == 1) {
      // a lone last tile: zero weights in the second half of its pair
      if (r16 < G) {
        const bf16x4_t z = {};
        *reinterpret_cast<bf16x4_t*>(&s_wt[w][0][NPW - 1][r16][sub][8]) = z;
        *reinterpret_cast<bf16x4_t*>(&s_wt[w][1][NPW - 1][r16][sub][8]) = z;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's value tiles have landed
    lds_barrier();                           // and every wave's, with the weights

    // ---- products: dims 16w .. 16w+15, every wave's tiles --------------------
    auto read1 = [&](const unsigned char* tile) {
      auto src = (__attribute__((address_space(3))) bf16x4_t*)(tile + tr_row * 256 +
                                                               16 * vt_chunk(tr_row, 2 * w + ((r16 & 3) >> 1)) +
                                                               8 * (r16 & 1));
      return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src);
    };
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sw = 0; sw < W; ++sw) {
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int ta = 2 * pp, tb = 2 * pp + 1 < NBT ? 2 * pp + 1 : 2 * pp;
        const unsigned char* pa = ta < NT ? &s_vt[sw][ta < NT ? ta : 0][0] : &s_pt[SEP ? sw : 0][0];
        const unsigned char* pb = tb < NT ? &s_vt[sw][tb < NT ? tb : 0][0] : &s_pt[SEP ? sw : 0][0];
        const bf16x8_t b = __builtin_shufflevector(read1(pa), read1(pb), 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (HLR) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<const bf16x8_t*>(&s_wt[sw][al][pp][ah][sub][0]), b, acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<const bf16x8_t*>(&s_wt[sw][0][pp][ah][sub][0]), b, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<const bf16x8_t*>(&s_wt[sw][1][pp][ah][sub][0]), b, acc, 0, 0, 0);
        }
      }
    }

    // ---- outputs ----------------------------------------------------------
    // normaliser of head hr (all waves' keys and proxies), then per head in
    // scalar registers
    float LA = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ww += 4) {
      const float4 l4 = *reinterpret_cast<const float4*>(&s_l[hr][ww]);
      LA += (l4.x + l4.y) + (l4.z + l4.w);
      if constexpr (PROXY) {
        const float4 p4 = *reinterpret_cast<const float4*>(&s_lp[hr][ww]);
        LA += (p4.x + p4.y) + (p4.z + p4.w);
      }
    }
    // accumulator element i of lane (n, group sub): row 4*sub + i, dim
    // 16w + n; rows G .. 2G-1 hold the remainders' share when HLR
    float tot[4];
    int hb = 0;          // first head of this lane's totals
    bool store = false;  // lanes whose totals are complete
    if constexpr (HLR && G == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const RowPair r = swap16(acc[i]);
        tot[i] = r.even + r.odd;
      }
      store = sub == 0;
    } else if constexpr (HLR && G == 2) {
      tot[0] = acc[0] + acc[2];
      tot[1] = acc[1] + acc[3];
      store = sub == 0;
    } else if constexpr (HLR) {
      tot[0] = acc[0] + acc[1];
      store = sub == 0;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] = acc[i];
      hb = 4 * sub;
      store = 4 * sub < G;
    }
    constexpr int NH = G < 4 ? G : 4;  // heads per storing lane
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int h = hb + i;
      // (a uniform lane index when G <= 4; per row group otherwise)
      const float L = (G <= 4) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(LA), i))
                               : shfl_f(LA, h < G ? h : 0);
      if (store) p.out[(qrow0 + h) * kD + 16 * w + r16] = (L > 0.f) ? tot[i] * __builtin_amdgcn_rcpf(L) : 0.f;
    }
    if (w == 0 && sub == 0 && r16 < G && p.lse)
      p.lse[qrow0 + r16] = (LA > 0.f) ? (Mh + __builtin_amdgcn_logf(LA)) * kLn2 : kNegInf;
  } else {
    floatx4_t oacc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) oacc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    auto product = [&](const bf16x8_t a, const bf16x4_t (&ba)[8], const bf16x4_t (&bb)[8]) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8_t b = __builtin_shufflevector(ba[nb], bb[nb], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[nb], 0, 0, 0);
      }
    };
    wave_lds_sync();  // the weights, written by other lanes
    auto wt8 = [&](int hl, int t) {  // 4 keys of tile t (pair half t & 1)
      return *reinterpret_cast<const bf16x4_t*>(&s_wt[w][hl][t >> 1][ah][sub][8 * (t & 1)]);
    };
    auto wt16 = [&](int hl, int pr) {  // 4 keys of both tiles of pair pr
      return *reinterpret_cast<const bf16x8_t*>(&s_wt[w][hl][pr][ah][sub][0]);
    };
    const bf16x4_t zero4 = {};
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // the value tiles have landed
    bf16x4_t bv[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) tile_read(&s_vt[w][t][0], bv[t]);
    if constexpr (PROXY && !SEP) {
      // no buffer of its own: the tile goes into the consumed tile 0 (the
      // writes follow this wave's reads of tile 0)
      unsigned char* ct = &s_vt[w][0][0];
      put_cluster_tile(ct);
      wave_lds_sync();  // the tile's rows, written by other lanes
      tile_read(ct, bc);
    }
    if constexpr (HLR) {
      const bf16x4_t cw = al ? clo : chi;
#pragma unroll
      for (int pr = 0; pr < NT / 2; ++pr) product(wt16(al, pr), bv[2 * pr], bv[2 * pr + 1]);
      if constexpr (NT % 2 == 1) {
        constexpr int t = NT - 1;
        if constexpr (PROXY)
          product(__builtin_shufflevector(wt8(al, t), cw, 0, 1, 2, 3, 4, 5, 6, 7), bv[t], bc);
        else
          product(__builtin_shufflevector(wt8(al, t), zero4, 0, 1, 2, 3, 4, 5, 6, 7), bv[t], bv[t]);
      } else if constexpr (PROXY) {
        product(__builtin_shufflevector(cw, zero4, 0, 1, 2, 3, 4, 5, 6, 7), bc, bc);
      }
    } else {
#pragma unroll
      for (int pr = 0; pr < NT / 2; ++pr) {
        product(wt16(0, pr), bv[2 * pr], bv[2 * pr + 1]);
        product(wt16(1, pr), bv[2 * pr], bv[2 * pr + 1]);
      }
      if constexpr (NT % 2 == 1) {
        constexpr int t = NT - 1;
        if constexpr (PROXY) {
          product(__builtin_shufflevector(wt8(0, t), chi, 0, 1, 2, 3, 4, 5, 6, 7), bv[t], bc);
          product(__builtin_shufflevector(wt8(1, t), clo, 0, 1, 2, 3, 4, 5, 6, 7), bv[t], bc);
        } else {
          product(__builtin_shufflevector(wt8(0, t), wt8(1, t), 0, 1, 2, 3, 4, 5, 6, 7), bv[t], bv[t]);
        }
      } else if constexpr (PROXY) {
        product(__builtin_shufflevector(chi, clo, 0, 1, 2, 3, 4, 5, 6, 7), bc, bc);
      }
    }

    // ---- per-wave partials, then the unit's combine ---------------------------
    // Accumulator element i of lane (n, group sub): row 4*sub + i, dim
    // 16*nb + n. The partials are stored dim-major, [dim][row] with NR4 rows
    // per dim, so that a lane writes each accumulator as one 16-byte store.
    constexpr int NR = HLR ? 2 * G : G;  // rows kept
    constexpr int NR4 = NR < 4 ? 4 : NR;
    static_assert(kD * NR4 * 4 <= kVTile, "partials must fit a tile");
    float* red = reinterpret_cast<float*>(&s_vt[w][0][0]);
    if (4 * sub < NR) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        *reinterpret_cast<floatx4_t*>(red + (16 * nb + r16) * NR4 + 4 * sub) = oacc[nb];
    }
    // normaliser of the wave: its keys (key layout, head 4j + sub) and its
    // proxies (head r16)
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int h = 4 * j + sub;
      const float tot = sum16(lsr[j]);
      if (r16 == 0 && h < G) s_l[h][w] = tot;
    }
    if constexpr (PROXY) {
      lsum = sum_rowgroups(lsum);
      if (sub == 0 && r16 < G) s_lp[r16][w] = lsum;
    }
    __syncthreads();

    for (int ei = tid; ei < G * kD; ei += 512) {
      const int dim = ei / G, h = ei - dim * G;
      float a = 0.f, L = 0.f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const float* rw = reinterpret_cast<const float*>(&s_vt[ww][0][0]) + dim * NR4 + h;
        a += HLR ? rw[0] + rw[G] : rw[0];
      }
#pragma unroll
      for (int ww = 0; ww < W; ww += 4) {
        const float4 l4 = *reinterpret_cast<const float4*>(&s_l[h][ww]);
        L += (l4.x + l4.y) + (l4.z + l4.w);
        if constexpr (PROXY) {
          const float4 p4 = *reinterpret_cast<const float4*>(&s_lp[h][ww]);
          L += (p4.x + p4.y) + (p4.z + p4.w);
        }
      }
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      // (hardware reciprocal and logarithm, ~1 ulp)
      p.out[qh * kD + dim] = (L > 0.f) ? a * __builtin_amdgcn_rcpf(L) : 0.f;
      if (dim == 0 && p.lse) p.lse[qh] = (L > 0.f) ? (s_M[h] + __builtin_amdgcn_logf(L)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 one-workgroup-per-unit kernel, value rows in registers (G <= 4).
//
// The logits run on the matrix cores as in sparse_unit_mfma_kernel (keys
// fetched in the MFMA operand layout, 16 keys x 64 bytes per load).  The
// value rows go to registers in the row layout: row group `sub` of wave w
// takes value slot k = list entry 16t + 4kq + sub (k = 4t + kq) of the wave's
// run, lane r16 holding dims 8*r16 .. +8 (one 16-byte load per slot, four
// whole rows per instruction).  The weighted values then run on the matrix
// cores with no LDS staging: for a block of eight slots the B operand of
// v_mfma_f32_16x16x32_bf16 for dim offset i is built with byte permutes from
// the eight slot registers (K index 8*sub + j = key 32*kb + 4j + sub, column
// r16 = dim 8*r16 + i), so a block is multiplied as soon as its rows land.
//
// The A operand holds each weight as three bf16 parts (rows h, 4 + h and
// 8 + h: high part, middle part and remainder, together exact to fp32), so
// the products carry the fp32 weights.  The weight of a read member of
// cluster b is e^{s - M} - e^{mu_b - M}; the cluster term e^{mu_b - M} sumV_b
// is added in fp32 on the vector units by the lanes that hold cluster b's
// sums, so the read members' share of sumV_b cancels at fp32 accuracy.
template <int G, bool PROXY, int NT>
__global__ __launch_bounds__(512) void sparse_unit_vt_kernel(const AttnParams p) {
  constexpr int W = kUnitWaves;
  constexpr int NS = 4 * NT;   // value slots per row group
  constexpr int PC = PROXY ? kCmax : 1;
  constexpr int PW = PROXY ? W : 1;
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int CH = p.chunk;      // entries of this wave: [w*CH, (w+1)*CH), CH <= 16*NT
  const int hr = r16 < G ? r16 : 0;  // head of this lane in the [head][..] layouts (clamped)

  constexpr int NV = G < 4 ? 1 : G / 4;  // heads per lane in the key layout
  static_assert(W % 4 == 0, "per-wave results are read four at a time");
  __shared__ __attribute__((aligned(16))) float s_wmax[G][W];
  __shared__ __attribute__((aligned(16))) float s_pmax[G][PW];
  __shared__ float s_M[G];
  __shared__ __attribute__((aligned(16))) float s_l[G][W];   // normaliser: the wave's keys
  __shared__ __attribute__((aligned(16))) float s_lp[G][PW]; // and its proxies
  __shared__ __attribute__((aligned(16))) float s_csum[PC][G][PW];
  __shared__ __attribute__((aligned(16))) int s_ccnt[PC][PW];
  // mean logit of a cluster's unread members (-inf if none), per head; entry
  // PC is a -inf sentinel for keys outside every cluster
  __shared__ __attribute__((aligned(16))) float s_mu[G][PC + 4];
  // list entries of the value slots, handed from the key loads' lanes
  __shared__ __attribute__((aligned(16))) int s_jv[W][NT][4][4];
  static_assert(G <= 4, "three weight parts per head fill at most 12 operand rows");
  constexpr int KB = (NT + 1) / 2;   // blocks of 32 keys (8 slots per row group)
  // weights as the value products' A operand: per wave, block kb, operand row
  // m (head m & 3, part m >> 2), key group kg and j: key 32kb + 4j + kg
  __shared__ __attribute__((aligned(16))) __bf16 s_wa[W][KB][16][4][8];
  // the waves' output partials, [wave][head][dim]
  __shared__ __attribute__((aligned(16))) float s_red[W][G][kD];

  // ---- prologue ------------------------------------------------------------
  // Every load that does not depend on the list is issued before the first
  // use of any loaded value: the query, the list entries and the cluster sums
  // share one memory round trip.  (With no list, and for absent optional
  // arrays, the loads read a valid dummy address and the values are
  // discarded.)
  const int64_t lbase = (int64_t)u * p.m;
  const int e = w * CH + lane;
  const bool in_list = (lane < CH) && (e < p.m);
  const int32_t* lst = p.m > 0 ? p.idx : reinterpret_cast<const int32_t*>(p.q);
  const int64_t ea = lbase + (in_list ? e : 0);
  int li = lst[ea];
  int lp = -1, lc = -1;
  if constexpr (PROXY) {
    lp = lst[lbase + ((in_list && e > 0) ? e - 1 : 0)];
    lc = (p.idx_cluster ? p.idx_cluster : lst)[ea];
  }
  const float lwv = (p.logw ? p.logw : reinterpret_cast<const float*>(lst))[ea];
  auto entry = [&](int pos) { return w * CH + pos; };
  auto listed = [&](int pos) { return pos < CH && entry(pos) < p.m; };
  int jk[NT];  // key rows of this lane: entry 16t + r16 of tile t
#pragma unroll
  for (int t = 0; t < NT; ++t) jk[t] = lst[lbase + (listed(16 * t + r16) ? entry(16 * t + r16) : 0)];

  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;
  uint4 qa[4];  // MFMA A operand: head r16 (zero past G), dims 32*st + 8*sub
#pragma unroll
  for (int st = 0; st < 4; ++st)
    qa[st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + hr) * kD + 32 * st +
                                             8 * sub);
  float qf[PROXY ? G : 1][8];  // row-layout query for the cluster-sum logits
  if constexpr (PROXY) load_query<bf16_t, G>(p.q, qrow0, r16, p.qscale, qf);

  // cluster sums and counts of the two clusters this lane owns: b0 = 4w + sub
  // and b1 = b0 + 32 (dims 8*r16 .. +8 of the sums); with C <= 32 there is no
  // b1 and its loads are skipped (a uniform branch)
  const int b0 = 4 * w + sub, b1 = b0 + 4 * W;
  const bool has0 = PROXY && b0 < p.C, has1 = PROXY && b1 < p.C;
  const bool two = PROXY && p.C > 4 * W;
  float skf[8], svf[8], sk1[8], sv1[8];
  int cnt0 = 0, cnt1 = 0;
  if constexpr (PROXY) {
    const int64_t c0 = (int64_t)u * p.C + (has0 ? b0 : 0);
    load8f(p.sumK + c0 * kD + 8 * r16, skf);
    load8f(p.sumV + c0 * kD + 8 * r16, svf);
    cnt0 = p.count[c0];
    if (two) {
      const int64_t c1 = (int64_t)u * p.C + (has1 ? b1 : 0);
      load8f(p.sumK + c1 * kD + 8 * r16, sk1);
      load8f(p.sumV + c1 * kD + 8 * r16, sv1);
      cnt1 = p.count[c1];
    }
  }

  int len = p.m;
  if (p.idx_len) {
    int L = p.idx_len[u];
    if (L < 0 || L > p.m) {
      if (tid == 0) flag_unit(p.flags, u, SDA_FLAG_LEN);
      L = L < 0 ? 0 : p.m;
    }
    len = L;
  }

  // ---- addresses ------------------------------------------------------------
  // The unit's rows span less than 2^31 bytes (checked on the host), so byte
  // offsets are 32-bit; an absent row reads past the resource and returns
  // zeros.
  const bool live = in_list && e < len;
  const bool in_range = (unsigned)li < (unsigned)p.n;
  const bool valid = live && in_range;
  const int rs = 2 * (int)p.sn;
  auto row_byte = [&](int pos, int j, int c) {
    const bool ok = (pos < CH) & (entry(pos) < len) & ((unsigned)j < (unsigned)p.n);
    return __builtin_unpredictable(ok) ? j * rs + c : kOOB;
  };
  int koff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = row_byte(16 * t + r16, jk[t], 16 * sub);
  // value slot k = 4t + kq is entry 16t + 4kq + sub: its list entry comes
  // from the key lanes through LDS
  if (sub == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) s_jv[w][t][r16 & 3][r16 >> 2] = jk[t];
  }
  wave_lds_sync();
  int voff[NS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int4 j4 = *reinterpret_cast<const int4*>(&s_jv[w][t][sub][0]);
    const int jv[4] = {j4.x, j4.y, j4.z, j4.w};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) voff[4 * t + kq] = row_byte(16 * t + 4 * kq + sub, jv[kq], 16 * r16);
  }

  // cluster of this lane's entry from the per-row ids when the list carries
  // none: issued ahead of the row loads (loads complete in issue order)
  if constexpr (PROXY) {
    if (!p.idx_cluster) lc = valid ? p.cluster_id[(int64_t)u * p.n + li] : -1;
  }

  // ---- row loads (streaming: read once) -------------------------------------
  // Keys first (MFMA layout); the work below that needs no row runs while they
  // are in flight (the memory queues are full by then), then the values (row
  // layout, to registers).
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);
  uint4 kt[NT][4];
  uint4 vt[NS];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[t] + 64 * st, 0, kLoadNT);
      kt[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < 4; ++st)
    if (r16 >= G) qa[st] = make_uint4(0, 0, 0, 0);

  // ---- checks and cluster lookups, behind the key loads ---------------------
  const float lw_own = valid ? (p.logw ? lwv * kLog2e : 0.f) : kNegInf;
  const bool bad_cluster = PROXY && p.idx_cluster && valid && (lc < -1 || lc >= p.C);
  if (bad_cluster) lc = -1;
  {
    int bad = 0;
    if (live && !in_range) bad |= SDA_FLAG_IDX_RANGE;
    if (PROXY && live && e > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
    if (bad_cluster) bad |= SDA_FLAG_CLUSTER;
    if (bad) flag_unit(p.flags, u, bad);
  }
  float qk0 = 0.f, qk1 = 0.f;  // q . (sum of keys) of clusters b0, b1 for head r16
  if constexpr (PROXY) {
    if (!has0) cnt0 = 0;
    if (!has1) cnt1 = 0;
#pragma unroll
    for (int i = lane; i < PC * G; i += 64) s_csum[i / G][i % G][w] = 0.f;
    for (int i = lane; i < PC; i += 64) s_ccnt[i][w] = 0;
    float a[G];
    dot_heads<G>(qf, skf, a);
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (r16 == h) qk0 = a[h];
    if (two) {
      dot_heads<G>(qf, sk1, a);
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (r16 == h) qk1 = a[h];
    }
  }

  // ---- per key tile: log-weight and cluster of this lane's key -------------
  // (key layout, below) and the controls of the segmented sums over runs of
  // keys with the same cluster (consecutive lanes of a row group). The read
  // members' counts per cluster are added here; their logit sums follow the
  // logits.
  float lwk[NT];
  int cmr[NT];  // cluster of the key, -1 if none
  float sf[NT][4];
  bool run_end[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int kk = 16 * t + r16;  // this lane's key within the wave's entries
    lwk[t] = shfl_f(lw_own, kk);
    cmr[t] = -1;
    run_end[t] = false;
    if constexpr (PROXY) {
      const int ck = shfl_i(lc, kk);
      const int cm = (lwk[t] != kNegInf && ck >= 0 && ck < p.C) ? ck : -1;
      cmr[t] = cm;
      const int cprev = dpp_i<0x111>(cm, -2), cnext = dpp_i<0x101>(cm, -2);  // row_shr:1, row_shl:1
      int start = cprev != cm ? r16 : 0;
      start = max(start, dpp_i<0x111>(start, 0));
      start = max(start, dpp_i<0x112>(start, 0));
      start = max(start, dpp_i<0x114>(start, 0));
      start = max(start, dpp_i<0x118>(start, 0));
      sf[t][0] = r16 - 1 >= start ? 1.f : 0.f;
      sf[t][1] = r16 - 2 >= start ? 1.f : 0.f;
      sf[t][2] = r16 - 4 >= start ? 1.f : 0.f;
      sf[t][3] = r16 - 8 >= start ? 1.f : 0.f;
      run_end[t] = cm >= 0 && cnext != cm;  // last lane of a run
      if (run_end[t] && sub == 0) lds_add(&s_ccnt[cm][w], r16 - start + 1);
    }
  }

  // ---- value rows, to registers -----------------------------------------------
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    auto v = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[k], 0, kLoadNT);
    vt[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- logits on the matrix cores ------------------------------------------
  // The MFMA leaves lane (key r16, group sub) the logits of heads 4*sub + i;
  // a 4 x 4 transpose of row groups turns that into the key layout: lane
  // (sub, r16) holds heads 4j + sub (j < NV) of key 16t + r16 of tile t.
  float xr[NT][NV];  // logit plus log-weight (log2 units)
  float mxr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) mxr[j] = kNegInf;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                  __builtin_bit_cast(bf16x8_t, kt[t][st]), d, 0, 0, 0);
    float sv[4], hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = d[i] * p.qscale;
    transpose_rows(sv, hv);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      xr[t][j] = hv[j] + lwk[t];
      mxr[j] = fmaxf(mxr[j], xr[t][j]);
    }
    if constexpr (PROXY) {
      // read members' logit sums per cluster (this wave's slice): inclusive
      // sums within runs by 0/1-weighted DPP steps (no branches: a move must
      // not read a lane that sits out); the last lane of each run adds the
      // run total
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float x = hv[j];
        x = fmaf(sf[t][0], dppz<0x111>(x), x);
        x = fmaf(sf[t][1], dppz<0x112>(x), x);
        x = fmaf(sf[t][2], dppz<0x114>(x), x);
        x = fmaf(sf[t][3], dppz<0x118>(x), x);
        hv[j] = x;
      }
      if (run_end[t]) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (4 * j + sub < G) lds_add(&s_csum[cmr[t]][4 * j + sub][w], hv[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float v = max16(mxr[j]);
    if (r16 == 0 && 4 * j + sub < G) s_wmax[4 * j + sub][w] = v;
  }
  lds_barrier();

  // ---- proxy logits of the clusters this wave owns ------------------------
  // Unread members of cluster b: n_b = count - (read members); their mean
  // logit mu_b = (q.sumK_b - sum of the read members' logits) / n_b; the
  // proxy logit is mu_b + log2(n_b).
  float Mk = kNegInf;  // maximum of the read logits, head hr
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const float4 m4 = *reinterpret_cast<const float4*>(&s_wmax[hr][4 * q]);
    Mk = fmaxf(Mk, fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w)));
  }
  float pi0 = kNegInf, pi1 = kNegInf;
  if constexpr (PROXY) {
    float cs0 = 0.f, cs1 = 0.f;
    int rc0 = 0, rc1 = 0;
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const float4 a0 = *reinterpret_cast<const float4*>(&s_csum[b0][hr][4 * q]);
      const float4 a1 = *reinterpret_cast<const float4*>(&s_csum[b1][hr][4 * q]);
      const int4 n0 = *reinterpret_cast<const int4*>(&s_ccnt[b0][4 * q]);
      const int4 n1 = *reinterpret_cast<const int4*>(&s_ccnt[b1][4 * q]);
      cs0 += (a0.x + a0.y) + (a0.z + a0.w);
      cs1 += (a1.x + a1.y) + (a1.z + a1.w);
      rc0 += n0.x + n0.y + n0.z + n0.w;
      rc1 += n1.x + n1.y + n1.z + n1.w;
    }
    bool neg_count = false;  // more read members than the cluster holds
    auto mean_logit = [&](int b, bool has, float qk, int cntb, float cs, int rc, float& pi) {
      const int nb = cntb - rc;
      neg_count |= has && nb < 0 && r16 == 0;
      const bool ok = has && nb > 0;
      const float nbf = (float)(ok ? nb : 1);
      const float mu = ok ? (qk - cs) * __builtin_amdgcn_rcpf(nbf) : kNegInf;  // (hardware reciprocal, ~1 ulp)
      pi = (ok && r16 < G) ? mu + __builtin_amdgcn_logf(nbf) : kNegInf;
      if (r16 < G) s_mu[r16][b] = mu;
    };
    mean_logit(b0, has0, qk0, cnt0, cs0, rc0, pi0);
    mean_logit(b1, has1, qk1, cnt1, cs1, rc1, pi1);
    if (w == 0 && sub == 0 && r16 < G) s_mu[r16][PC] = kNegInf;
    const float pm = max_rowgroups(fmaxf(pi0, pi1));
    if (sub == 0 && r16 < G) s_pmax[r16][w] = pm;
    lds_barrier();
    if (neg_count) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  }

  // ---- unit maximum (every wave, same value) --------------------------------
  float Mh = Mk;  // head hr
  if constexpr (PROXY) {
#pragma unroll
    for (int ww = 0; ww < W; ww += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(&s_pmax[hr][ww]);
      Mh = fmaxf(Mh, fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w)));
    }
  }
  if (Mh == kNegInf) Mh = 0.f;
  if (w == 0 && sub == 0 && r16 < G) s_M[r16] = Mh;
  float Mu[G];   // every head's maximum, uniform (lane h computed head h)
#pragma unroll
  for (int h = 0; h < G; ++h) Mu[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Mh), h));
  float Mr[NV];  // the same in the key layout: head 4j + sub (a select, no lane shuffle)
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    Mr[j] = Mu[0];
#pragma unroll
    for (int h = 1; h < G; ++h)
      if (4 * j + sub == h) Mr[j] = Mu[h];
  }

  // ---- weights, in the key layout -------------------------------------------
  // w = exp2(x - M), minus exp2(mu_b - M) for a read member of cluster b
  // (whose value the cluster term counts in the cluster's sum), split into
  // three bf16 parts that sum to w exactly (each part takes 8 of w's 24
  // significant bits)
  float lsr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) lsr[j] = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int h = 4 * j + sub;
      const float ev = fast_exp2(xr[t][j] - Mr[j]);
      lsr[j] += ev;
      float wv = ev;
      if constexpr (PROXY) {
        const float mu = s_mu[h < G ? h : 0][cmr[t] >= 0 ? cmr[t] : PC];
        wv = ev - fast_exp2(mu - Mr[j]);
      }
      const __bf16 w0 = (__bf16)wv;
      const float r1 = wv - (float)w0;
      const __bf16 w1 = (__bf16)r1;
      const __bf16 w2 = (__bf16)(r1 - (float)w1);
      if (h < G) {
        const int kk = 16 * t + r16;  // key within the wave's entries
        __bf16* dst = &s_wa[w][kk >> 5][h][kk & 3][(kk >> 2) & 7];
        dst[0] = w0;
        dst[4 * 4 * 8] = w1;   // row h + 4
        dst[8 * 4 * 8] = w2;   // row h + 8
      }
    }
  }
  // the proxies' share of the normaliser (lanes of head r16, clusters b0, b1;
  // exp2(-inf) = 0 for the absent ones)
  float lsum = 0.f;
  if constexpr (PROXY) lsum = fast_exp2(pi0 - Mh) + fast_exp2(pi1 - Mh);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int h = 4 * j + sub;
    const float tot = sum16(lsr[j]);
    if (r16 == 0 && h < G) s_l[h][w] = tot;
  }
  if constexpr (PROXY) {
    lsum = sum_rowgroups(lsum);
    if (sub == 0 && r16 < G) s_lp[r16][w] = lsum;
  }

  // ---- lane swaps that sum over row groups ------------------------------------
  // v_permlane16_swap(a, b) leaves even rows (a_even, a_odd) and odd rows
  // (b_even, b_odd): with a = what even rows keep and b = what odd rows keep,
  // one add per value sums a pair of rows and halves what each lane holds
  // (permlane32_swap likewise for rows 0-1 against 2-3).
  auto swap_add16 = [](float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  auto swap_add32 = [](float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  // ---- weighted values on the matrix cores -----------------------------------
  // A (lane: operand row r16, key group sub): the three weight parts of head
  // r16 & 3 for keys 32kb + 4j + sub (j = 0..7); rows of absent heads and
  // the fourth part row set are zero, as are keys past the wave's 16*NT.
  // B for dim offset i (lane: key group sub, column r16): dim 8*r16 + i of
  // slots 8kb + j, two slots per 32-bit word by a byte permute.
  //
  // The accumulators start from the cluster terms of this lane's clusters:
  // acc[i][r] (head r, dim 8*r16 + i) = e^{mu_b0 - M_r} sumV_b0[8*r16 + i]
  // (+ the same for b1), fp32; the sum over the row groups below adds them up
  // with the products' parts.
  floatx4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (PROXY) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float c0 = fast_exp2(s_mu[h][has0 ? b0 : PC] - Mu[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][h] = c0 * svf[i];
    }
    if (two) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float c1 = fast_exp2(s_mu[h][has1 ? b1 : PC] - Mu[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][h] = fmaf(c1, sv1[i], acc[i][h]);
      }
    }
  }
  wave_lds_sync();  // the weights, written by other lanes of this wave
  const bool arow = (r16 & 3) < G && r16 < 12;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    uint4 a4 = *reinterpret_cast<const uint4*>(&s_wa[w][kb][r16][sub][0]);
    if (!arow) a4 = make_uint4(0, 0, 0, 0);
    if (8 * kb + 8 > NS) a4.z = a4.w = 0;  // slots past the wave's keys
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a4);
    uint32_t vw[8][4];  // [slot j][word]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 8 * kb + j;
      if (k < NS) {
        vw[j][0] = vt[k].x; vw[j][1] = vt[k].y; vw[j][2] = vt[k].z; vw[j][3] = vt[k].w;
      } else {
        vw[j][0] = vw[j][1] = vw[j][2] = vw[j][3] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each word
      uint4 b4;
      b4.x = __builtin_amdgcn_perm(vw[1][i >> 1], vw[0][i >> 1], sel);
      b4.y = __builtin_amdgcn_perm(vw[3][i >> 1], vw[2][i >> 1], sel);
      b4.z = __builtin_amdgcn_perm(vw[5][i >> 1], vw[4][i >> 1], sel);
      b4.w = __builtin_amdgcn_perm(vw[7][i >> 1], vw[6][i >> 1], sel);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, b4), acc[i], 0, 0, 0);
    }
  }

  // ---- sum of the parts and row groups, then over the waves ------------------
  // acc[i][r] of lane (r16, sub): part sub of head r at dim 8*r16 + i plus
  // the cluster terms of row group sub.  Two swap steps leave lane (r16, sub)
  // heads 2*(sub >> 1) + r' (r' < 2) at dims 8*r16 + 4*(sub & 1) + i'
  // (i' < 4), summed over the row groups.
  float x[4][4], y[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[i][r] = swap_add16(acc[i][r], acc[i + 4][r]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 2; ++r) y[i][r] = swap_add32(x[i][r], x[i][r + 2]);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int h = 2 * (sub >> 1) + r;
    if (h < G)
      *reinterpret_cast<float4*>(&s_red[w][h][8 * r16 + 4 * (sub & 1)]) = make_float4(y[0][r], y[1][r], y[2][r], y[3][r]);
  }
  lds_barrier();

  // ---- outputs: one (head, dim) per thread, waves summed in order ----------
  for (int ei = tid; ei < G * kD; ei += 512) {
    const int h = ei / kD, dim = ei - h * kD;
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ww += 2) a += s_red[ww][h][dim] + s_red[ww + 1][h][dim];
#pragma unroll
    for (int ww = 0; ww < W; ww += 4) {
      const float4 l4 = *reinterpret_cast<const float4*>(&s_l[h][ww]);
      L += (l4.x + l4.y) + (l4.z + l4.w);
      if constexpr (PROXY) {
        const float4 p4 = *reinterpret_cast<const float4*>(&s_lp[h][ww]);
        L += (p4.x + p4.y) + (p4.z + p4.w);
      }
    }
    // (hardware reciprocal and logarithm, ~1 ulp)
    p.out[(qrow0 + h) * kD + dim] = (L > 0.f) ? a * __builtin_amdgcn_rcpf(L) : 0.f;
    if (dim == 0 && p.lse) p.lse[qrow0 + h] = (L > 0.f) ? (s_M[h] + __builtin_amdgcn_logf(L)) * kLn2 : kNegInf;
  }
}

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

// Online-softmax combine of two partials (m, l, acc); both lanes of a row
// pair compute the same bits.
__device__ __forceinline__ void lse_factors(float ma, float mb, float& M, float& fa, float& fb) {
  M = fmaxf(ma, mb);
  fa = rescale(ma, M);
  fb = rescale(mb, M);
}

// ---------------------------------------------------------------------------
// Split-K streaming kernel.  Workgroup (u, split) covers list entries (or
// rows, for the dense modes) [split*chunk, min(len, (split+1)*chunk)).  Each
// 16-lane row group keeps its own online-softmax state; groups and waves are
// merged at the end.  A batch is NSB slots of 4 rows per wave; the list
// entries of the next batch are fetched while the current batch's rows are
// in flight.
template <typename T, int G, int MODE, int NSB>
__global__ __launch_bounds__(256) void stream_kernel(const AttnParams p) {
  constexpr int W = 4;
  constexpr int STEP = 4 * W * NSB;
  constexpr bool DENSE = (MODE == kModeDense || MODE == kModeBuildPrior);
  constexpr bool PRIOR = (MODE == kModePrior);
  constexpr bool BUILD = (MODE == kModeBuildPrior);
  using QT = typename std::conditional<BUILD, float, T>::type;
  static_assert(4 * NSB <= 64, "one list entry per lane");
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

  float qf[G][8];
  load_query<QT, G>(p.q, (int64_t)s * p.Hq + (int64_t)g * G, r16, p.qscale, qf);
  float qp[PRIOR ? G : 1][8];
  float mP[G];
  if constexpr (PRIOR) {
    // prior logits use the mean query, shifted by the stored maxP
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
      load8f(p.mu_Q + qh * kD + 8 * r16, qp[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qp[h][i] *= p.qscale;
      mP[h] = p.maxP[qh] * kLog2e;
    }
  }

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

  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<T>(reinterpret_cast<const T*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<T>(reinterpret_cast<const T*>(p.V) + kvoff, p.n, p.sn);

  // lane l < 4*NSB of wave w holds list entry tb + 4*((l>>2)*W + w) + (l&3)
  const int lk = lane >> 2, lsub = lane & 3;
  auto list_t = [&](int tb) { return tb + 4 * (lk * W + w) + lsub; };
  int li = -1, lp = -1;
  float lwv = 0.f;
  auto load_list = [&](int tb, int& vi, int& vp, float& vw) {
    const int t = list_t(tb);
    const bool in = lane < 4 * NSB && t < t1;
    const int64_t a = lbase + (in ? t : 0);
    vi = p.idx[a];
    if (PRIOR) vp = p.idx[lbase + ((in && t > 0) ? t - 1 : 0)];
    if (p.logw) vw = p.logw[a];
  };
  if (!DENSE && t0 < t1) load_list(t0, li, lp, lwv);

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

  for (int tb = t0; tb < t1; tb += STEP) {
    int off[NSB];
    float lw[NSB];
    bool cov[PRIOR ? NSB : 1];   // the prior covers the slot's row
    bool lane_ok = false;
    if constexpr (!DENSE) {
      const int t = list_t(tb);
      lane_ok = lane < 4 * NSB && t < t1 && (unsigned)li < (unsigned)p.n;
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      if constexpr (DENSE) {
        const int t = tb + 4 * (k * W + w) + sub;
        off[k] = t < t1 ? row_off<T>(t, p.sn, r16) : kOOB;
        lw[k] = t < t1 ? 0.f : kNegInf;
      } else {
        const int src = 4 * k + sub;
        const int j = shfl_i(li, src);
        const bool ok = shfl_i(lane_ok ? 1 : 0, src) != 0;
        off[k] = ok ? row_off<T>(j, p.sn, r16) : kOOB;
        lw[k] = ok ? shfl_f(lwv, src) * kLog2e : kNegInf;
        if constexpr (PRIOR) cov[k] = ok && j < p.prior_n;
      }
    }
    RowChunk<T> kc[NSB], vc[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) buf_load(kc[k], rk, off[k]);
#pragma unroll
    for (int k = 0; k < NSB; ++k) buf_load(vc[k], rv, off[k]);

    if constexpr (!DENSE) {
      // checks of this batch's entries, then the next batch's list
      const int t = list_t(tb);
      const bool live = lane < 4 * NSB && t < t1;
      int bad = 0;
      if (live && (unsigned)li >= (unsigned)p.n) bad |= SDA_FLAG_IDX_RANGE;
      if (PRIOR && live && t > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
      if (bad) flag_unit(p.flags, u, bad);
      if (tb + STEP < t1) load_list(tb + STEP, li, lp, lwv);
    }

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
#pragma unroll
        for (int i = 0; i < 8; ++i) ks[i] += kf[i];   // rows outside the range load as zeros
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
        for (int h = 0; h < G; ++h) pl[k][h] = cov[k] ? ap[h] - mP[h] : kNegInf;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], bm[h]);
      const float alpha = rescale(m[h], mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      float vf[8];
      vc[k].unpack(vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ev = (m[h] == kNegInf) ? 0.f : fast_exp2(x[k][h] - m[h]);
        l[h] += ev;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(ev, vf[i], acc[h][i]);
        if constexpr (PRIOR) {
          const float ep = fast_exp2(pl[k][h]);
          sp[h] += ep;
#pragma unroll
          for (int i = 0; i < 8; ++i) spv[h][i] = fmaf(ep, vf[i], spv[h][i]);
        }
      }
    }
  }

  // ---- merge the four row groups of the wave ------------------------------
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const RowPair mm = pass ? swap32(m[h]) : swap16(m[h]);
      float M, fa, fb;
      lse_factors(mm.even, mm.odd, M, fa, fb);
      const RowPair ll = pass ? swap32(l[h]) : swap16(l[h]);
      l[h] = ll.even * fa + ll.odd * fb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const RowPair aa = pass ? swap32(acc[h][i]) : swap16(acc[h][i]);
        acc[h][i] = aa.even * fa + aa.odd * fb;
      }
      m[h] = M;
      if constexpr (PRIOR) {
        const RowPair ss = pass ? swap32(sp[h]) : swap16(sp[h]);
        sp[h] = ss.even + ss.odd;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const RowPair vv = pass ? swap32(spv[h][i]) : swap16(spv[h][i]);
          spv[h][i] = vv.even + vv.odd;
        }
      }
    }
    if constexpr (BUILD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const RowPair kk = pass ? swap32(ks[i]) : swap16(ks[i]);
        ks[i] = kk.even + kk.odd;
      }
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
    if (split == 0 && w == 0) {
      float c[G];
      bias_shift<G>(p, s, g, r16, qf, c);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_c[h] = c[h];
      }
    }
  }
  __syncthreads();

  for (int ei = tid; ei < G * kD; ei += 256) {
    const int h = ei / kD, dim = ei - h * kD;
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
        rec[3] = (PRIOR && split == 0) ? s_c[h] : 0.f;
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
// bf16 split-K streaming kernel with both products on the matrix cores.
//
// A workgroup (4 waves) takes entries [t0, t1) of one unit; per batch each
// wave takes 16*NT consecutive entries.  The logits come from
// v_mfma_f32_16x16x32_bf16 with the A operand rows holding the G query heads
// and, for the prior, the G mean queries mu_Q split into a bf16 high part
// (rows G..2G-1) and remainder (rows 2G..3G-1), so that sigma mu_Q.k keeps
// fp32 accuracy.  An online softmax runs across batches: the batch maximum of
// each head goes through LDS, the accumulator rows are rescaled in the
// accumulator layout and the normaliser in the operand layout, from the same
// values.  The weighted values use the same transposed-LDS products as the
// one-workgroup-per-unit kernel, with the prior weights exp(P - maxP) as A
// rows G..2G-1 (fixed shift, no rescaling).  Partial records and the merge
// are those of stream_kernel.
//
// One batch is always in flight: once a batch's keys have gone through the
// logit products and its values into the wave's LDS tiles, the registers
// that held them take the next batch's row loads, which then overlap the
// softmax and the value products of the current batch.
template <int G, int MODE, int NT>
__global__ __launch_bounds__(256) void stream_mfma_kernel(const AttnParams p) {
  constexpr int W = 4;
  constexpr bool DENSE = (MODE == kModeDense);
  constexpr bool PRIOR = (MODE == kModePrior);
  constexpr bool PROXY = (MODE == kModeProxy);
  constexpr int CBX = PROXY ? kCmax / 16 : 1;  // blocks of 16 clusters (value sums)
  constexpr int RA = PRIOR ? 3 * G : G;  // A rows of the logits
  constexpr int RP = PRIOR ? 2 * G : G;  // A rows of the weighted values
  static_assert(RA <= 16, "the logit rows fit one 16-row block");
  constexpr int KB = 16 * NT;            // entries per wave per batch
  constexpr int STEP = W * KB;           // entries per workgroup per batch
  constexpr int NS = 4 * NT;             // value slots per wave per batch
  constexpr int kVRow = 144;             // bf16 elements per staged value row
  constexpr int kTile = 16 * kVRow * 2;
  constexpr int kWaveLds = NT * kTile > RP * kD * 4 ? NT * kTile : RP * kD * 4;  // the batch's value tiles
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const int u = blockIdx.x / p.splits;
  const int split = blockIdx.x - u * p.splits;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int hr = r16 < G ? r16 : 0;

  __shared__ __attribute__((aligned(16))) float s_x[W][RA][KB];
  __shared__ float s_bm[W][G];
  __shared__ float s_m[W][G], s_l[W][G], s_sp[W][G];
  __shared__ float s_c[G];
  // proxy mode: the split's listed rows per cluster (count over all waves),
  // their logit sums per wave, and the cluster of each entry of the batch
  __shared__ int s_pcn[PROXY ? kCmax : 1];
  __shared__ float s_pcs[PROXY ? W : 1][PROXY ? kCmax : 1][G];
  __shared__ __attribute__((aligned(16))) int s_cl[2][PROXY ? W : 1][KB];  // double-buffered: batch in flight
  __shared__ __attribute__((aligned(16))) unsigned char s_pool[W * kWaveLds];

  // ---- A operand: row r16, dims 32*st + 8*sub .. +8 ---------------------------
  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;
  uint4 qa[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qa[st] = make_uint4(0, 0, 0, 0);
    if (r16 < G) {
      qa[st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + r16) * kD + 32 * st +
                                                8 * sub);
    } else if (PRIOR && r16 < 3 * G) {
      const int h = (r16 - G) % G;
      float mq[8];
      load8f(p.mu_Q + (qrow0 + h) * kD + 32 * st + 8 * sub, mq);
      bf16x8_t v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 hi = (__bf16)mq[i];
        v[i] = r16 < 2 * G ? hi : (__bf16)(mq[i] - (float)hi);
      }
      qa[st] = __builtin_bit_cast(uint4, v);
    }
  }
  // prior shift maxP (log2 units) of the operand-layout head r16 - G
  float mPa = 0.f;
  if (PRIOR && r16 >= G && r16 < 2 * G) mPa = p.maxP[qrow0 + r16 - G] * kLog2e;

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
  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);

  // list entry of this lane for the batch at tb: tb + w*KB + lane (lane < KB)
  int li = -1, lp = -1, lc = -1;
  float lwv = 0.f;
  // Every load here is unconditional (entry 0 stands in past the end, the
  // list itself for an absent log-weight or cluster array): a value that only
  // some paths load would be merged by a register copy, and the wait for that
  // copy would also wait for the batch's row loads issued before it.
  const float* lw_src = p.logw ? p.logw : reinterpret_cast<const float*>(p.idx);
  const int* lc_src = (PROXY && p.idx_cluster) ? p.idx_cluster : p.idx;
  auto load_list = [&](int tb, int& vi, int& vp, float& vw, int& vc) {
    const int t = tb + w * KB + lane;
    const bool in = lane < KB && t < t1;
    const int64_t a = lbase + (in ? t : 0);
    vi = p.idx[a];
    if constexpr (PRIOR || PROXY) vp = p.idx[lbase + ((in && t > 0) ? t - 1 : 0)];
    if constexpr (PROXY) vc = lc_src[a];
    vw = lw_src[a];
  };
  if (!DENSE && t0 < t1) load_list(t0, li, lp, lwv, lc);
  if constexpr (PROXY) {
    for (int i = tid; i < kCmax; i += 256) s_pcn[i] = 0;
    for (int i = lane; i < kCmax * G; i += 64) (&s_pcs[w][0][0])[i] = 0.f;
    __syncthreads();
  }
  const int CB = PROXY ? (p.C + 15) / 16 : 0;
  floatx4_t racc[CBX][8];  // proxy mode: listed value sums, 16 clusters x 16 dims per accumulator
#pragma unroll
  for (int cb = 0; cb < CBX; ++cb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) racc[cb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  floatx4_t oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_a = kNegInf;                                     // running max of head r16
  float m_d[4] = {kNegInf, kNegInf, kNegInf, kNegInf};     // running max of rows 4*sub + i
  float lsum = 0.f, spsum = 0.f;
  bf16_t* vt = reinterpret_cast<bf16_t*>(s_pool + w * kWaveLds);

  // the batch in flight: the keys and values of its rows, and the state of
  // this lane's entry (tb + w*KB + lane, lane < KB)
  uint4 kt[NT][4];
  RowChunk<bf16_t> vc[NS];
  bool b_valid = false;
  float b_lw = kNegInf;  // log-weight of the entry (log2 units), -inf if absent
  bool b_cov = false;    // the prior covers the entry's row
  int b_cm = -1;         // proxy mode: cluster of the entry's row, -1 if none
  // The entry state of the batch at tb from the list registers (cluster ids
  // into s_cl[buf]), then its row loads and the next batch's list entries.
  auto issue = [&](int tb, int buf) {
    const int e = tb + w * KB + lane;
    int row;
    if constexpr (DENSE) {
      b_valid = lane < KB && e < t1;
      row = b_valid ? e : 0;
      b_lw = b_valid ? 0.f : kNegInf;
    } else {
      const bool live = lane < KB && e < t1;
      b_valid = live && (unsigned)li < (unsigned)p.n;
      row = li;
      b_lw = b_valid ? (p.logw ? lwv * kLog2e : 0.f) : kNegInf;
      if constexpr (PRIOR) b_cov = b_valid && li < p.prior_n;
      int bad = 0;
      if (live && (unsigned)li >= (unsigned)p.n) bad |= SDA_FLAG_IDX_RANGE;
      if ((PRIOR || PROXY) && live && e > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
      if constexpr (PROXY) {
        int c = -1;
        if (b_valid) c = p.idx_cluster ? lc : p.cluster_id[(int64_t)u * p.n + li];
        if (b_valid && p.idx_cluster && (c < -1 || c >= p.C)) bad |= SDA_FLAG_CLUSTER;
        b_cm = (b_valid && c >= 0 && c < p.C) ? c : -1;
        if (lane < KB) s_cl[buf][w][lane] = b_cm;
        if (b_cm >= 0) atomicAdd(&s_pcn[b_cm], 1);
      }
      if (bad) flag_unit(p.flags, u, bad);
    }
    int koff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int src = 16 * t + r16;
      const int j = shfl_i(row, src);
      const bool ok = shfl_i(b_valid ? 1 : 0, src) != 0;
      koff[t] = ok ? (int)(((int64_t)j * p.sn + 8 * sub) * 2) : kOOB;
    }
    int voff[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int src = 4 * k + sub;
      const int j = shfl_i(row, src);
      const bool ok = shfl_i(b_valid ? 1 : 0, src) != 0;
      voff[k] = ok ? row_off<bf16_t>(j, p.sn, r16) : kOOB;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[t] + 64 * st, 0, kLoadNT);
        kt[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
    for (int k = 0; k < NS; ++k) buf_load(vc[k], rv, voff[k]);
    if constexpr (!DENSE) load_list(tb + STEP, li, lp, lwv, lc);
  };

  if (t0 < t1) issue(t0, 0);
  int buf = 0;
  for (int tb = t0; tb < t1; tb += STEP, buf ^= 1) {
    // ---- logits ---------------------------------------------------------------
    float bmx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                    __builtin_bit_cast(bf16x8_t, kt[t][st]), d, 0, 0, 0);
      const int kk = 16 * t + r16;
      const float lwk = shfl_f(b_lw, kk);
      const bool cvk = PRIOR && shfl_i(b_cov ? 1 : 0, kk) != 0;   // the prior covers this key
      if constexpr (PROXY) {
        // the listed rows' logits per cluster (log2 units, no log-weight),
        // this wave's slots: one LDS add per (key, head)
        const int ck = shfl_i(b_cm, kk);
        if (ck >= 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * sub + i < G) lds_add(&s_pcs[w][ck][4 * sub + i], d[i] * p.qscale);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * sub + i;
        if (r < G) {
          const float xv = d[i] * p.qscale + lwk;
          s_x[w][r][kk] = xv;
          bmx[i] = fmaxf(bmx[i], xv);
        } else if (r < RA) {
          s_x[w][r][kk] = cvk ? d[i] : kNegInf;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = max16(bmx[i]);
      if (r16 == 0 && 4 * sub + i < G) s_bm[w][4 * sub + i] = v;
    }
    // ---- the batch's values into LDS, which frees the row registers -----------
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        *reinterpret_cast<uint4*>(vt + (16 * t + 4 * kq + sub) * kVRow + 8 * r16) = vc[4 * t + kq].raw;
    // ---- the next batch's rows go out while this one is finished -------------
    if (tb + STEP < t1) issue(tb + STEP, buf ^ 1);
    wave_lds_sync();  // logits, batch maxima and value tiles, written by other lanes of the wave
    // ---- online rescale (same values in both layouts) --------------------------
    {
      const float mn = fmaxf(m_a, s_bm[w][hr]);
      const float al = rescale(m_a, mn);
      lsum *= al;
      m_a = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * sub + i;
        if (r < G) {
          const float mnd = fmaxf(m_d[i], s_bm[w][r]);
          const float ad = rescale(m_d[i], mnd);
          m_d[i] = mnd;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) oacc[nb][i] *= ad;
        }
      }
    }
    // ---- weighted values ------------------------------------------------------
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 x4 = *reinterpret_cast<const float4*>(&s_x[w][r16 < RP ? r16 : 0][16 * t + 4 * sub]);
      float4 y4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (PRIOR) y4 = *reinterpret_cast<const float4*>(&s_x[w][r16 >= G && r16 < 2 * G ? r16 + G : 0][16 * t + 4 * sub]);
      const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
      // proxy mode: one-hot cluster rows (row r16 of block cb is cluster
      // 16cb + r16) for the keys of this lane's operand half, so that the
      // same B operand also sums the listed values per cluster
      bf16x8_t a1[CBX];
      if constexpr (PROXY) {
        const int4 c4 = *reinterpret_cast<const int4*>(&s_cl[buf][w][16 * t + 4 * sub]);
        const int cl4[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int cb = 0; cb < CBX; ++cb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a1[cb][j] = (__bf16)(cl4[j] == 16 * cb + r16 ? 1.f : 0.f);
            a1[cb][4 + j] = (__bf16)0.f;
          }
      }
      const float ys[4] = {y4.x, y4.y, y4.z, y4.w};
      bf16x8_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // one exp per lane: softmax rows (r16 < G) and prior rows (G <= r16 < 2G)
        float arg;
        if constexpr (PRIOR) {
          arg = r16 < G ? xs[j] - m_a : (xs[j] + ys[j]) * p.qscale - mPa;
        } else {
          arg = xs[j] - m_a;
        }
        float wv = fast_exp2(arg);  // exp2(-inf) = 0 for absent keys
        if (r16 >= RP || (r16 < G && m_a == kNegInf)) wv = 0.f;
        if (r16 < G) lsum += wv;
        if (PRIOR && r16 >= G) spsum += wv;
        const __bf16 hi = (__bf16)wv;
        a[j] = hi;
        a[4 + j] = (__bf16)(wv - (float)hi);
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        auto src = (__attribute__((address_space(3))) bf16x4_t*)(vt + (16 * t + 4 * sub + (r16 >> 2)) * kVRow +
                                                                 16 * nb + 4 * (r16 & 3));
        const bf16x4_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src);
        const bf16x8_t b = {b4[0], b4[1], b4[2], b4[3], b4[0], b4[1], b4[2], b4[3]};
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[nb], 0, 0, 0);
        if constexpr (PROXY) {
#pragma unroll
          for (int cb = 0; cb < CBX; ++cb)
            if (cb < CB) racc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[cb], b, racc[cb][nb], 0, 0, 0);
        }
      }
    }
  }
  // ---- wave results -------------------------------------------------------------
  float* red = reinterpret_cast<float*>(s_pool + w * kWaveLds);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * sub + i;
    if (r < RP) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) red[r * kD + 16 * nb + r16] = oacc[nb][i];
    }
  }
  lsum = sum_rowgroups(lsum);
  spsum = sum_rowgroups(spsum);
  if (sub == 0 && r16 < G) {
    s_l[w][r16] = lsum;
    s_m[w][r16] = m_a;
  }
  if (PRIOR && sub == 0 && r16 >= G && r16 < 2 * G) s_sp[w][r16 - G] = spsum;
  if constexpr (PRIOR) {
    if (split == 0 && w == 0) {
      float qf[G][8];
      load_query<bf16_t, G>(p.q, qrow0, r16, p.qscale, qf);
      float c[G];
      bias_shift<G>(p, s, g, r16, qf, c);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_c[h] = c[h];
      }
    }
  }
  __syncthreads();

  for (int ei = tid; ei < G * kD; ei += 256) {
    const int h = ei / kD, dim = ei - h * kD;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) M = fmaxf(M, s_m[ww][h]);
    float a = 0.f, L = 0.f, SP = 0.f, SPV = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float* rw = reinterpret_cast<const float*>(s_pool + ww * kWaveLds);
      const float f = rescale(s_m[ww][h], M);
      a = fmaf(rw[h * kD + dim], f, a);
      L = fmaf(s_l[ww][h], f, L);
      if constexpr (PRIOR) {
        SP += s_sp[ww][h];
        SPV += rw[(G + h) * kD + dim];
      }
    }
    const int64_t qh = qrow0 + h;
    if (PROXY || p.splits > 1) {
      float* rec = p.part + (((int64_t)u * p.splits + split) * G + h) * kPartStride;
      if (dim == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = SP;
        rec[3] = (PRIOR && split == 0) ? s_c[h] : 0.f;
      }
      rec[4 + dim] = a;
      if constexpr (PRIOR) rec[4 + kD + dim] = SPV;
    } else if constexpr (PRIOR) {
      const Fin f = finalize_prior(M, L, a, s_c[h], p.maxP[qh] * kLog2e, p.sumP[qh], p.O_est[qh * kD + dim],
                                   SP, SPV, p.lambda);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    } else {
      const Fin f = finalize_plain(M, L, a);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    }
  }
  if constexpr (PROXY) {
    // the split's per-cluster records: counts and logit sums of every
    // cluster (the merge reads them unconditionally), value sums of the
    // clusters it touched, the waves' accumulators added through LDS 16
    // clusters at a time
    float* cbase = p.cpart + ((int64_t)u * p.splits + split) * p.C * kClusterRec;
    for (int b = tid; b < p.C; b += 256) {
      float* rec = cbase + (int64_t)b * kClusterRec;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sh = 0.f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) sh += s_pcs[ww][b][h];
        rec[128 + h] = sh;
      }
      reinterpret_cast<int*>(rec)[136] = s_pcn[b];
    }
    // a wave's pool slice holds 8 cluster rows of fp32 sums: two halves per
    // block of 16 clusters (rows 8hf .. 8hf+7 come from lanes with sub >> 1 == hf)
    static_assert(8 * kD * 4 <= kWaveLds, "half a cluster block fits a wave's slice");
#pragma unroll
    for (int cb = 0; cb < CBX; ++cb) {
      if (cb >= CB) break;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        __syncthreads();  // the pool is free
        float* mine = reinterpret_cast<float*>(s_pool + w * kWaveLds);
        if ((sub >> 1) == hf) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) mine[(4 * (sub & 1) + i) * kD + 16 * nb + r16] = racc[cb][nb][i];
        }
        __syncthreads();
        for (int e2 = tid; e2 < 8 * kD; e2 += 256) {
          const int row = e2 / kD, dim = e2 - row * kD;
          const int b = 16 * cb + 8 * hf + row;
          if (b < p.C && s_pcn[b] > 0) {
            float a = 0.f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) a += reinterpret_cast<const float*>(s_pool + ww * kWaveLds)[row * kD + dim];
            cbase[(int64_t)b * kClusterRec + dim] = a;
          }
        }
      }
    }
  }
}
// LDS accesses of a wave whose direct-to-LDS loads stay in flight, written
// out: the compiler cannot tell the tiles those loads fill from the other LDS
// arrays, and would wait for every one of them before any LDS access. A
// wave's LDS operations execute in order, so these need no waits between
// them; each read waits for its own results inside its statement, and every
// output is early-clobber (the reads complete after later ones issue).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void lds_st_f32(float* p, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Sixteen bytes at ax (and at ay when TWO) and the eight transposed 64-bit
// reads of a value tile at at[0..7].
template <bool TWO>
__device__ __forceinline__ void lds_tile_reads(unsigned ax, unsigned ay, const unsigned (&at)[8], f32x4_t& x,
                                               f32x4_t& y, u32x2_t (&b)[8]) {
  if constexpr (TWO) {
    asm volatile(
        "ds_read_b128 %0, %10\n\tds_read_b128 %1, %11\n\t"
        "ds_read_b64_tr_b16 %2, %12\n\tds_read_b64_tr_b16 %3, %13\n\t"
        "ds_read_b64_tr_b16 %4, %14\n\tds_read_b64_tr_b16 %5, %15\n\t"
        "ds_read_b64_tr_b16 %6, %16\n\tds_read_b64_tr_b16 %7, %17\n\t"
        "ds_read_b64_tr_b16 %8, %18\n\tds_read_b64_tr_b16 %9, %19\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x), "=&v"(y), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]),
          "=&v"(b[6]), "=&v"(b[7])
        : "v"(ax), "v"(ay), "v"(at[0]), "v"(at[1]), "v"(at[2]), "v"(at[3]), "v"(at[4]), "v"(at[5]), "v"(at[6]),
          "v"(at[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b64_tr_b16 %1, %10\n\tds_read_b64_tr_b16 %2, %11\n\t"
        "ds_read_b64_tr_b16 %3, %12\n\tds_read_b64_tr_b16 %4, %13\n\t"
        "ds_read_b64_tr_b16 %5, %14\n\tds_read_b64_tr_b16 %6, %15\n\t"
        "ds_read_b64_tr_b16 %7, %16\n\tds_read_b64_tr_b16 %8, %17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]),
          "=&v"(b[7])
        : "v"(ax), "v"(at[0]), "v"(at[1]), "v"(at[2]), "v"(at[3]), "v"(at[4]), "v"(at[5]), "v"(at[6]), "v"(at[7])
        : "memory");
    y = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------------------
// bf16 split-K streaming kernel with the value rows staged straight from HBM
// into LDS: plain lists, dense rows and the rank-1 prior.
//
// The products are those of stream_mfma_kernel (logits with the G heads, and
// for the prior the mean-query rows, in one A operand; weighted values from
// transposed LDS reads), but each wave keeps two batches in flight instead of
// one. A batch's keys go to one of two register sets and its values, by
// direct-to-LDS buffer loads, to one of two sets of swizzled value tiles, so
// no register holds a value row. Once a batch's keys have gone through the
// logit products their registers take the keys of the batch two ahead; once
// its value products have read its tiles, the tiles take that batch's values.
// Every load is issued unconditionally (entries past the chunk get an offset
// outside the buffer, which returns zeros), so the number of loads issued
// after a batch's value tiles is fixed, and the wait for those tiles (an
// explicit vmcnt) leaves the later batches' loads in flight.
template <int G, int MODE, int NT>
__global__ __launch_bounds__(256, 2) void stream_dma_kernel(const AttnParams p) {
  constexpr int W = 4;
  constexpr bool DENSE = (MODE == kModeDense);
  constexpr bool PRIOR = (MODE == kModePrior);
  static_assert(MODE == kModeSparse || DENSE || PRIOR, "plain, dense and prior modes only");
  constexpr int RA = PRIOR ? 3 * G : G;  // A rows of the logits
  constexpr int RP = PRIOR ? 2 * G : G;  // A rows of the weighted values
  static_assert(RA <= 16, "the logit rows fit one 16-row block");
  constexpr int KB = 16 * NT;   // entries per wave per batch
  constexpr int STEP = W * KB;  // entries per workgroup per batch
  constexpr int NS = 4 * NT;    // value loads per wave per batch (four rows each)
  static_assert(RP * kD * 4 <= NT * kVTile, "a wave's partial sums fit its value tiles");
  // loads issued after a batch's value tiles until they are read: the next
  // batch's keys and values, then the keys of the batch two ahead
  constexpr int kAfterV = 2 * 4 * NT + NS;
  static_assert(kAfterV < 64, "the wait count fits vmcnt");
  constexpr int kWaitV = 0x0F70 | (kAfterV & 15) | ((kAfterV >> 4) << 14);
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const int u = blockIdx.x / p.splits;
  const int split = blockIdx.x - u * p.splits;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int hr = r16 < G ? r16 : 0;

  __shared__ __attribute__((aligned(16))) float s_x[W][RA][KB];
  __shared__ float s_m[W][G], s_l[W][G], s_sp[W][G];
  __shared__ float s_c[G];
  // value tiles of the two batches in flight: per wave NT tiles of 16 rows x
  // 256 bytes, 16-byte chunks swizzled (vt_chunk)
  __shared__ __attribute__((aligned(16))) unsigned char s_v0[W][NT][kVTile];
  __shared__ __attribute__((aligned(16))) unsigned char s_v1[W][NT][kVTile];

  // ---- A operand: row r16, dims 32*st + 8*sub .. +8 ---------------------------
  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;
  uint4 qa[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qa[st] = make_uint4(0, 0, 0, 0);
    if (r16 < G) {
      qa[st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + r16) * kD + 32 * st +
                                                8 * sub);
    } else if (PRIOR && r16 < 3 * G) {
      const int h = (r16 - G) % G;
      float mq[8];
      load8f(p.mu_Q + (qrow0 + h) * kD + 32 * st + 8 * sub, mq);
      bf16x8_t v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 hi = (__bf16)mq[i];
        v[i] = r16 < 2 * G ? hi : (__bf16)(mq[i] - (float)hi);
      }
      qa[st] = __builtin_bit_cast(uint4, v);
    }
  }
  // prior shift maxP (log2 units) of the operand-layout head r16 - G
  float mPa = 0.f;
  if (PRIOR && r16 >= G && r16 < 2 * G) mPa = p.maxP[qrow0 + r16 - G] * kLog2e;

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
  const int64_t lbase = (int64_t)u * p.m;
  const int64_t kvoff = (int64_t)s * p.sb + (int64_t)g * p.sh;
  const rsrc_t rk = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.K) + kvoff, p.n, p.sn);
  const rsrc_t rv = make_rsrc<bf16_t>(reinterpret_cast<const bf16_t*>(p.V) + kvoff, p.n, p.sn);

  // This wave's list entries of every batch of the chunk, staged in LDS before
  // any row load (a chunk holds at most kStreamDmaMaxChunk entries): row b
  // holds the entry before the wave's block of batch b (for the order check),
  // then the block's KB entries; the log-weights beside them. Read back
  // while row loads are in flight, so no loop-carried register waits on a
  // list load.
  constexpr int MB = kStreamDmaMaxChunk / STEP;  // batches per chunk, at most
  __shared__ int s_li[DENSE ? 1 : W][DENSE ? 1 : MB][KB + 1];
  __shared__ float s_lw[DENSE ? 1 : W][DENSE ? 1 : MB][KB];
  const int nbatch = t0 < t1 ? (t1 - t0 + STEP - 1) / STEP : 0;
  if constexpr (!DENSE) {
    for (int b = 0; b < nbatch; ++b) {
      const int e = t0 + b * STEP + w * KB - 1 + lane;  // entry of slot `lane`
      if (lane <= KB) s_li[w][b][lane] = (e >= 0 && e < t1) ? p.idx[lbase + e] : -1;
      if (lane >= 1 && lane <= KB) s_lw[w][b][lane - 1] = (p.logw && e < t1) ? p.logw[lbase + e] : 0.f;
    }
  }
  int bad = 0;  // list errors seen by this lane, flagged once at the end
  // (li, lp, log-weight) of this lane's entry of batch b from LDS
  auto read_list = [&](int b, int& li, int& lp, float& lw) {
    const int bb = b < nbatch ? b : 0;  // batches past the chunk: any row (not live)
    const int k = lane < KB ? lane : 0;
    asm volatile(
        "ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(li), "=&v"(lp), "=&v"(lw)
        : "v"(lds_addr(&s_li[0][0][0] + (w * MB + bb) * (KB + 1) + k + 1)),
          "v"(lds_addr(&s_li[0][0][0] + (w * MB + bb) * (KB + 1) + k)),
          "v"(lds_addr(&s_lw[0][0][0] + (w * MB + bb) * KB + k))
        : "memory");
  };

  floatx4_t oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_a = kNegInf;                                  // running max of head r16
  float m_d[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // running max of rows 4*sub + i
  float lsum = 0.f, spsum = 0.f;

  // the two batches in flight: keys in registers; this lane's entry row (-1 if
  // absent) until the batch's value loads go out; the entry state
  uint4 kt0[NT][4], kt1[NT][4];
  int vr0 = -1, vr1 = -1;
  float lw0 = kNegInf, lw1 = kNegInf;  // log-weight of the entry (log2 units), -inf if absent
  bool cv0 = false, cv1 = false;       // the prior covers the entry's row

  // Batch b: entry state from its list entries and its key loads.
  auto issue_keys = [&](int b, uint4 (&kt)[NT][4], int& vrow, float& b_lw, bool& b_cov) {
    const int e = t0 + b * STEP + w * KB + lane;
    int row;
    bool b_valid;
    if constexpr (DENSE) {
      b_valid = lane < KB && e < t1;
      row = b_valid ? e : 0;
      b_lw = b_valid ? 0.f : kNegInf;
    } else {
      int li, lp;
      float lwv;
      read_list(b, li, lp, lwv);
      const bool live = lane < KB && e < t1;
      b_valid = live && (unsigned)li < (unsigned)p.n;
      row = li;
      b_lw = b_valid ? lwv * kLog2e : kNegInf;
      if constexpr (PRIOR) b_cov = b_valid && li < p.prior_n;
      if (live && (unsigned)li >= (unsigned)p.n) bad |= SDA_FLAG_IDX_RANGE;
      if (PRIOR && live && e > 0 && lp >= li) bad |= SDA_FLAG_IDX_ORDER;
    }
    int koff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int src = 16 * t + r16;
      const int j = shfl_i(row, src);
      const bool ok = shfl_i(b_valid ? 1 : 0, src) != 0;
      koff[t] = ok ? (int)(((int64_t)j * p.sn + 8 * sub) * 2) : kOOB;
    }
    vrow = b_valid ? row : -1;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[t] + 64 * st, 0, kLoadNT);
        kt[t][st] = make_uint4(v[0], v[1], v[2], v[3]);
      }
  };
  // Its value loads: load k = 4t + kq fills rows 4kq .. 4kq+3 of tile t;
  // lane (sub, r16) lands at row 4kq + sub, chunk position r16, so it fetches
  // the chunk of entry 16t + 4kq + sub that the swizzle puts there.
  auto issue_values = [&](unsigned char (&tiles)[W][NT][kVTile], int vrow) {
    int vo[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int j = shfl_i(vrow, 4 * k + sub);
      vo[k] = j >= 0 ? (int)((int64_t)j * p.sn * 2) + 16 * vt_chunk(4 * (k & 3) + sub, r16) : kOOB;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int off = vo[k];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)&tiles[w][k >> 2][(k & 3) * 1024], 16, off, 0, 0, kLoadNT);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // this lane's transposed reads of a value tile: row tr = 4*sub + r16/4,
  // dims 16*nb + 4*(r16 & 3) .. +3, i.e. chunk 2*nb + q (q = (r16 & 3) / 2)
  // at position vt_chunk(tr, 2*nb + q) = 2*(nb ^ xh) + q with xh the odd
  // bits of the row's swizzle: byte tbase + 32*(nb ^ xh)
  const int tr_row = 4 * sub + (r16 >> 2);
  const unsigned tbase = tr_row * 256 + 16 * ((r16 & 3) >> 1) + 8 * (r16 & 1);
  const unsigned txh = (unsigned)(vt_chunk(tr_row, 0) >> 1);

  // One batch: logits from its key registers, which then take the keys of
  // the batch two ahead; online rescale; weighted values from its tiles, which
  // then take that batch's values.
  auto process = [&](int b, uint4 (&kt)[NT][4], int& vrow, float& b_lw, bool& b_cov,
                     unsigned char (&tiles)[W][NT][kVTile]) {
    // ---- logits ---------------------------------------------------------------
    float bmx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                    __builtin_bit_cast(bf16x8_t, kt[t][st]), d, 0, 0, 0);
      const int kk = 16 * t + r16;
      const float lwk = shfl_f(b_lw, kk);
      const bool cvk = PRIOR && shfl_i(b_cov ? 1 : 0, kk) != 0;  // the prior covers this key
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * sub + i;
        if (r < G) {
          const float xv = d[i] * p.qscale + lwk;
          lds_st_f32(&s_x[w][r][kk], xv);
          bmx[i] = fmaxf(bmx[i], xv);
        } else if (r < RA) {
          lds_st_f32(&s_x[w][r][kk], cvk ? d[i] : kNegInf);
        }
      }
    }
    // batch maxima: every lane of row group sub holds those of rows 4*sub + i
#pragma unroll
    for (int i = 0; i < 4; ++i) bmx[i] = max16(bmx[i]);
    // ---- the keys two batches ahead --------------------------------------------
    issue_keys(b + 2, kt, vrow, b_lw, b_cov);
    // ---- online rescale (same values in both layouts) --------------------------
    {
      // head hr's batch maximum from the row group that holds it
      float own = bmx[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) own = (hr & 3) == i ? bmx[i] : own;
      const float bm_h = shfl_f(own, 16 * (hr >> 2) + r16);
      const float mn = fmaxf(m_a, bm_h);
      const float al = rescale(m_a, mn);
      lsum *= al;
      m_a = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * sub + i;
        if (r < G) {
          const float mnd = fmaxf(m_d[i], bmx[i]);
          const float ad = rescale(m_d[i], mnd);
          m_d[i] = mnd;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) oacc[nb][i] *= ad;
        }
      }
    }
    // ---- weighted values ------------------------------------------------------
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitV);  // this batch's value tiles have landed
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      unsigned xh = txh;
      asm volatile("" : "+v"(xh));  // computed per tile, not held across the loop
      unsigned at[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) at[nb] = lds_addr(&tiles[w][t][0]) + tbase + 32 * (nb ^ xh);
      f32x4_t x4, y4;
      u32x2_t bt[8];
      lds_tile_reads<PRIOR>(lds_addr(&s_x[w][r16 < RP ? r16 : 0][16 * t + 4 * sub]),
                            lds_addr(&s_x[w][r16 >= G && r16 < 2 * G ? r16 + G : 0][16 * t + 4 * sub]), at, x4, y4,
                            bt);
      const float xs[4] = {x4[0], x4[1], x4[2], x4[3]};
      const float ys[4] = {y4[0], y4[1], y4[2], y4[3]};
      bf16x8_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // one exp per lane: softmax rows (r16 < G) and prior rows (G <= r16 < 2G)
        float arg;
        if constexpr (PRIOR) {
          arg = r16 < G ? xs[j] - m_a : (xs[j] + ys[j]) * p.qscale - mPa;
        } else {
          arg = xs[j] - m_a;
        }
        float wv = fast_exp2(arg);  // exp2(-inf) = 0 for absent keys
        if (r16 >= RP || (r16 < G && m_a == kNegInf)) wv = 0.f;
        if (r16 < G) lsum += wv;
        if (PRIOR && r16 >= G) spsum += wv;
        const __bf16 hi = (__bf16)wv;
        a[j] = hi;
        a[4 + j] = (__bf16)(wv - (float)hi);
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x4_t b4 = __builtin_bit_cast(bf16x4_t, bt[nb]);
        const bf16x8_t b = {b4[0], b4[1], b4[2], b4[3], b4[0], b4[1], b4[2], b4[3]};
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[nb], 0, 0, 0);
      }
    }
    // ---- the values two batches ahead, into the tiles just read ---------------
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every tile read has returned
    issue_values(tiles, vrow);
  };

  // two batches in flight from the start
  if (nbatch > 0) {
    issue_keys(0, kt0, vr0, lw0, cv0);
    issue_values(s_v0, vr0);
    issue_keys(1, kt1, vr1, lw1, cv1);
    issue_values(s_v1, vr1);
  }
  // batches in pairs (register sets and tiles alternate), then an odd last one
  int i = 0;
  for (; i + 1 < nbatch; i += 2) {
    process(i, kt0, vr0, lw0, cv0, s_v0);
    process(i + 1, kt1, vr1, lw1, cv1, s_v1);
  }
  if (i < nbatch) process(i, kt0, vr0, lw0, cv0, s_v0);
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // the loads past the end have landed too
  if (__ballot(bad != 0)) {
    int any = bad;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) any |= __shfl_xor(any, sh, 64);
    if (lane == 0) flag_unit(p.flags, u, any);
  }

  // ---- wave results -------------------------------------------------------------
  float* red = reinterpret_cast<float*>(&s_v0[w][0][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * sub + i;
    if (r < RP) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) red[r * kD + 16 * nb + r16] = oacc[nb][i];
    }
  }
  lsum = sum_rowgroups(lsum);
  spsum = sum_rowgroups(spsum);
  if (sub == 0 && r16 < G) {
    s_l[w][r16] = lsum;
    s_m[w][r16] = m_a;
  }
  if (PRIOR && sub == 0 && r16 >= G && r16 < 2 * G) s_sp[w][r16 - G] = spsum;
  if constexpr (PRIOR) {
    if (split == 0 && w == 0) {
      float qf[G][8];
      load_query<bf16_t, G>(p.q, qrow0, r16, p.qscale, qf);
      float c[G];
      bias_shift<G>(p, s, g, r16, qf, c);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_c[h] = c[h];
      }
    }
  }
  __syncthreads();

  for (int ei = tid; ei < G * kD; ei += 256) {
    const int h = ei / kD, dim = ei - h * kD;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) M = fmaxf(M, s_m[ww][h]);
    float a = 0.f, L = 0.f, SP = 0.f, SPV = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float* rw = reinterpret_cast<const float*>(&s_v0[ww][0][0]);
      const float f = rescale(s_m[ww][h], M);
      a = fmaf(rw[h * kD + dim], f, a);
      L = fmaf(s_l[ww][h], f, L);
      if constexpr (PRIOR) {
        SP += s_sp[ww][h];
        SPV += rw[(G + h) * kD + dim];
      }
    }
    const int64_t qh = qrow0 + h;
    if (p.splits > 1) {
      float* rec = p.part + (((int64_t)u * p.splits + split) * G + h) * kPartStride;
      if (dim == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = SP;
        rec[3] = (PRIOR && split == 0) ? s_c[h] : 0.f;
      }
      rec[4 + dim] = a;
      if constexpr (PRIOR) rec[4 + kD + dim] = SPV;
    } else if constexpr (PRIOR) {
      const Fin f = finalize_prior(M, L, a, s_c[h], p.maxP[qh] * kLog2e, p.sumP[qh], p.O_est[qh * kD + dim],
                                   SP, SPV, p.lambda);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    } else {
      const Fin f = finalize_plain(M, L, a);
      p.out[qh * kD + dim] = f.out;
      if (dim == 0 && p.lse) p.lse[qh] = f.lse;
    }
  }
}

// Merge of split partials: one workgroup per unit, fixed split order.
template <int G, int MODE>
__global__ __launch_bounds__(512) void merge_kernel(const AttnParams p) {
  constexpr bool PRIOR = (MODE == kModePrior);
  constexpr bool BUILD = (MODE == kModeBuildPrior);
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x;

  // one (head, dim) per thread; one pass over the splits with a running
  // maximum, so that every split's loads are independent of the others
  for (int ei = tid; ei < G * kD; ei += 512) {
    const int h = ei / kD, dim = ei - h * kD;
    const int64_t qh = (int64_t)s * p.Hq + (int64_t)g * G + h;
    float mP = 0.f, zP = 0.f, oe = 0.f;
    if constexpr (PRIOR) {
      mP = p.maxP[qh] * kLog2e;
      zP = p.sumP[qh];
      oe = p.O_est[qh * kD + dim];
    }
    const float* base = p.part + ((int64_t)u * p.splits * G + h) * kPartStride;
    const int64_t stride = (int64_t)G * kPartStride;
    float M = kNegInf, a = 0.f, L = 0.f, SP = 0.f, SPV = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < p.splits; ++sp) {
      const float* rec = base + sp * stride;
      const float ms = rec[0], ls = rec[1], as = rec[4 + dim];
      const float mn = fmaxf(M, ms);
      const float fo = rescale(M, mn), fs = rescale(ms, mn);
      a = a * fo + as * fs;
      L = L * fo + ls * fs;
      M = mn;
      if constexpr (PRIOR) {
        SP += rec[2];
        SPV += rec[4 + kD + dim];
      }
    }
    if constexpr (PRIOR) {
      const Fin f = finalize_prior(M, L, a, base[3], mP, zP, oe, SP, SPV, p.lambda);
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
    for (int dim = tid; dim < kD; dim += 512) {
      float a = 0.f;
      for (int sp = 0; sp < p.splits; ++sp) a += p.ksum[((int64_t)u * p.splits + sp) * kD + dim];
      p.aux2[(int64_t)u * kD + dim] = a / (float)p.n;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the split-K proxy decode, one workgroup per unit.  The splits'
// per-cluster listed counts, logit sums and value sums are added in split
// order; every cluster b with n_b = count_b - (listed rows) > 0 then enters
// the softmax as its proxy ("OpenAttention", method stage 04): mean logit
// mu_b = (scale <q, sumK_b> - listed logits) / n_b, weight n_b e^{mu_b - M}
// in the normaliser and e^{mu_b - M} (sumV_b - listed values) in the
// numerator, the difference formed in fp32.
template <int G>
__global__ __launch_bounds__(512) void merge_proxy_kernel(const AttnParams p) {
  const int u = blockIdx.x;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x;
  const int C = p.C;
  __shared__ float s_mu[kCmax][G];   // mean logit of the unread members (log2), -inf if none
  __shared__ float s_pi[kCmax][G];   // proxy logit mu_b + log2 n_b
  __shared__ float s_D[kCmax][kD];   // sumV_b minus the listed values
  const int64_t qrow0 = (int64_t)s * p.Hq + (int64_t)g * G;
  const float* cb0 = p.cpart + (int64_t)u * p.splits * C * kClusterRec;
  const int64_t sstride = (int64_t)C * kClusterRec;

  for (int t = tid; t < C * G; t += 512) {
    const int b = t / G, h = t - b * G;
    float S = 0.f;
    int cnt = 0;
    for (int sp = 0; sp < p.splits; ++sp) {
      const float* rec = cb0 + sp * sstride + (int64_t)b * kClusterRec;
      S += rec[128 + h];
      cnt += reinterpret_cast<const int*>(rec)[136];
    }
    const bf16_t* qh = reinterpret_cast<const bf16_t*>(p.q) + (qrow0 + h) * kD;
    const float* sk = p.sumK + ((int64_t)u * C + b) * kD;
    float qk = 0.f;
#pragma unroll 4
    for (int d0 = 0; d0 < kD; d0 += 8) {
      RowChunk<bf16_t> c;
      c.load_cached(qh + d0);
      float f[8], kf[8];
      c.unpack(f);
      load8f(sk + d0, kf);
#pragma unroll
      for (int i = 0; i < 8; ++i) qk = fmaf(f[i], kf[i], qk);
    }
    qk *= p.qscale;
    const int nb = p.count[(int64_t)u * C + b] - cnt;
    if (nb < 0 && h == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
    const bool ok = nb > 0;
    const float mu = ok ? (qk - S) / (float)nb : kNegInf;
    s_mu[b][h] = mu;
    s_pi[b][h] = ok ? mu + __builtin_amdgcn_logf((float)nb) : kNegInf;
  }
  for (int t = tid; t < C * kD; t += 512) {
    const int b = t / kD, dim = t - b * kD;
    float r = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      const float* rec = cb0 + sp * sstride + (int64_t)b * kClusterRec;
      if (reinterpret_cast<const int*>(rec)[136] > 0) r += rec[dim];
    }
    s_D[b][dim] = p.sumV[((int64_t)u * C + b) * kD + dim] - r;
  }
  __syncthreads();

  for (int ei = tid; ei < G * kD; ei += 512) {
    const int h = ei / kD, dim = ei - h * kD;
    const float* base = p.part + ((int64_t)u * p.splits * G + h) * kPartStride;
    const int64_t stride = (int64_t)G * kPartStride;
    float M = kNegInf;
    for (int sp = 0; sp < p.splits; ++sp) M = fmaxf(M, base[sp * stride]);
    for (int b = 0; b < C; ++b) M = fmaxf(M, s_pi[b][h]);
    float a = 0.f, L = 0.f;
    if (M != kNegInf) {
      for (int sp = 0; sp < p.splits; ++sp) {
        const float* rec = base + sp * stride;
        const float f = rescale(rec[0], M);
        a = fmaf(rec[4 + dim], f, a);
        L = fmaf(rec[1], f, L);
      }
      for (int b = 0; b < C; ++b) {
        a = fmaf(fast_exp2(s_mu[b][h] - M), s_D[b][dim], a);   // exp2(-inf) = 0: no unread member
        L += fast_exp2(s_pi[b][h] - M);
      }
    }
    const int64_t qh = qrow0 + h;
    p.out[qh * kD + dim] = (L > 0.f) ? a / L : 0.f;
    if (dim == 0 && p.lse) p.lse[qh] = (L > 0.f) ? (M + __builtin_amdgcn_logf(L)) * kLn2 : kNegInf;
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

template <int G, bool PROXY>
static hipError_t launch_mfma_nt(const AttnParams& p, int nt, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  switch (nt) {
    case 1: hipLaunchKernelGGL((sparse_unit_mfma_kernel<G, PROXY, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((sparse_unit_mfma_kernel<G, PROXY, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((sparse_unit_mfma_kernel<G, PROXY, 3>), grid, block, 0, st, p); break;
    case 4:
      if constexpr (G < 8) {  // LDS: the value tiles of 8 waves x 4 tiles leave no room for G = 8
        hipLaunchKernelGGL((sparse_unit_mfma_kernel<G, PROXY, 4>), grid, block, 0, st, p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G, bool PROXY>
static hipError_t launch_vt_nt(const AttnParams& p, int nt, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  switch (nt) {
    case 1: hipLaunchKernelGGL((sparse_unit_vt_kernel<G, PROXY, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((sparse_unit_vt_kernel<G, PROXY, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((sparse_unit_vt_kernel<G, PROXY, 3>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((sparse_unit_vt_kernel<G, PROXY, 4>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// bf16: value rows in registers for G <= 4 (three weight parts fit one
// operand's 16 rows), value tiles in LDS for G = 8
template <int G>
static hipError_t launch_mfma_g(const AttnParams& p, bool proxy, int nt, hipStream_t st) {
  if constexpr (G <= 4) return proxy ? launch_vt_nt<G, true>(p, nt, st) : launch_vt_nt<G, false>(p, nt, st);
  else return proxy ? launch_mfma_nt<G, true>(p, nt, st) : launch_mfma_nt<G, false>(p, nt, st);
}

hipError_t launch_sparse_unit(const AttnParams& p, int dtype, int G, bool proxy, int ns, hipStream_t st) {
  if (dtype == SDA_BF16) {
    // ns = 4 * tiles for the matrix-core kernel
    const int nt = ns / 4;
    switch (G) {
      case 1: return launch_mfma_g<1>(p, proxy, nt, st);
      case 2: return launch_mfma_g<2>(p, proxy, nt, st);
      case 4: return launch_mfma_g<4>(p, proxy, nt, st);
      case 8: return launch_mfma_g<8>(p, proxy, nt, st);
    }
    return hipErrorInvalidValue;
  }
  return launch_unit_t<float>(p, G, proxy, ns, st);
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

template <int G>
static hipError_t launch_stream_mfma_g(const AttnParams& p, int mode, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv * p.splits), block(256);
  // the list of a plain or prior chunk is staged in LDS
  if ((mode == kModeSparse || mode == kModePrior) && p.chunk > kStreamDmaMaxChunk) return hipErrorInvalidValue;
  switch (mode) {
    case kModeSparse: hipLaunchKernelGGL((stream_dma_kernel<G, kModeSparse, kStreamMfmaTiles>), grid, block, 0, st, p); break;
    case kModeDense: hipLaunchKernelGGL((stream_dma_kernel<G, kModeDense, kStreamMfmaTiles>), grid, block, 0, st, p); break;
    case kModePrior:
      if constexpr (3 * G <= 16) {
        hipLaunchKernelGGL((stream_dma_kernel<G, kModePrior, kStreamMfmaTiles>), grid, block, 0, st, p);
        break;
      }
      return hipErrorInvalidValue;
    case kModeProxy: hipLaunchKernelGGL((stream_mfma_kernel<G, kModeProxy, kStreamMfmaTiles>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_mfma(const AttnParams& p, int G, int mode, hipStream_t st) {
  switch (G) {
    case 1: return launch_stream_mfma_g<1>(p, mode, st);
    case 2: return launch_stream_mfma_g<2>(p, mode, st);
    case 4: return launch_stream_mfma_g<4>(p, mode, st);
    case 8: return launch_stream_mfma_g<8>(p, mode, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const AttnParams& p, int dtype, int G, int mode, hipStream_t st) {
  return dtype == SDA_BF16 ? launch_stream_t<bf16_t>(p, G, mode, st) : launch_stream_t<float>(p, G, mode, st);
}

template <int G>
static hipError_t launch_merge_g(const AttnParams& p, int mode, hipStream_t st) {
  const dim3 grid(p.B * p.Hkv), block(512);
  switch (mode) {
    case kModeSparse:
    case kModeDense: hipLaunchKernelGGL((merge_kernel<G, kModeSparse>), grid, block, 0, st, p); break;
    case kModePrior: hipLaunchKernelGGL((merge_kernel<G, kModePrior>), grid, block, 0, st, p); break;
    case kModeBuildPrior: hipLaunchKernelGGL((merge_kernel<G, kModeBuildPrior>), grid, block, 0, st, p); break;
    case kModeProxy: hipLaunchKernelGGL((merge_proxy_kernel<G>), grid, block, 0, st, p); break;
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
