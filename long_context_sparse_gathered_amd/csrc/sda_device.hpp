// sda_device.hpp -- device helpers shared by the libsda kernels (gfx950).
//
// Row layout used by every kernel: d = 128.  A 16-lane group of a wave owns
// one KV row; lane r16 = lane & 15 holds dims [8*r16, 8*r16 + 8).  A wave
// therefore covers 4 rows per load instruction (lane >> 4 picks the row);
// for bf16 that is one 16-byte load per lane (a 256-byte row per group), for
// fp32 two.  Logits are kept in log2 units (the query is pre-multiplied by
// scale * log2(e)) so every exponential is a single v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_kernels.hpp"

namespace sda {

constexpr int kRowLanes = 16;    // lanes per row
constexpr int kPerLane = 8;      // elements per lane
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

struct bf16_t {
  uint16_t bits;
};

// ---- loads -----------------------------------------------------------------

// 8 consecutive elements (dims 8*r16 ..) of a row, widened to fp32.
template <typename T>
struct RowChunk;

template <>
struct RowChunk<bf16_t> {
  uint4 raw;
  __device__ __forceinline__ void load_cached(const bf16_t* p) {
    raw = *reinterpret_cast<const uint4*>(p);
  }
  // read-once data (non-temporal: not kept in the caches)
  __device__ __forceinline__ void load_stream(const bf16_t* p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    raw = make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ void zero() { raw = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void unpack(float (&f)[8]) const {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct RowChunk<float> {
  float4 a, b;
  __device__ __forceinline__ void load_cached(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void load_stream(const float* p) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    const v4f y = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p) + 1);
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ void unpack(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// fp32 chunk of 8 (cluster sums, prior state).
__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Query chunk: 8 elements (dims 8*r16 ..) of a bf16 or fp32 query, as fp32.
template <typename QT>
__device__ __forceinline__ void load_q8(const void* q, int64_t off, float (&f)[8]) {
  RowChunk<QT> c;
  c.load_cached(reinterpret_cast<const QT*>(q) + off);
  c.unpack(f);
}

// ---- cross-lane --------------------------------------------------------------

// Hand-off of LDS data between lanes of one wave: the wave's LDS operations
// execute in order, and this wavefront-scope fence keeps the compiler from
// moving LDS accesses across the hand-off or forwarding a lane's own store to
// a load that another lane's store is meant to satisfy.
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row group; every lane receives the same bits
// (each step adds a pair in both orders, and fp addition is commutative).
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Max over the 16 lanes of a row group (same pattern as sum16).
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The four 16-lane row groups of a wave hold partial results for the same
// dims.  v_permlane16_swap / v_permlane32_swap exchange rows in one VALU op;
// each combine takes (even-row value, odd-row value) in the same order on
// both lanes, so every lane ends with bitwise-identical results.
struct RowPair {
  float even, odd;
};
__device__ __forceinline__ RowPair swap16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ RowPair swap32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float max_rowgroups(float v) {
  RowPair a = swap16(v);
  v = fmaxf(a.even, a.odd);
  RowPair b = swap32(v);
  return fmaxf(b.even, b.odd);
}

__device__ __forceinline__ float sum_rowgroups(float v) {
  RowPair a = swap16(v);
  v = a.even + a.odd;
  RowPair b = swap32(v);
  return b.even + b.odd;
}

// Scale factor exp2(m - M) that is 0 (not NaN) for an empty partial.
__device__ __forceinline__ float rescale(float m, float M) {
  return (m == kNegInf) ? 0.f : fast_exp2(m - M);
}

__device__ __forceinline__ void flag_unit(int32_t* flags, int u, int bits) {
  if (flags) atomicOr(flags + u, bits);
}

}  // namespace sda
