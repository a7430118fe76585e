// sda_build.hip -- per-cluster state for the count-aware mean proxies
// ("OpenAttention", method stage 01: per cluster, a count and a mean token
// cached once per request; stored here as count, key sum and value sum).
//
// Two deterministic passes: every workgroup owns (unit, row chunk) and each of
// its threads owns one 4-byte column word of K or V, walking the chunk's rows
// in order and keeping a running sum for the current cluster (a register run,
// flushed to its own LDS column on a cluster change).  A second kernel adds
// the chunk partials in chunk order.  No atomics, so repeated builds are
// bitwise identical.
#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

constexpr int kBuildUnroll = 8;

template <typename T>
struct Word;
template <>
struct Word<bf16_t> {
  static constexpr int E = 2;
  __device__ __forceinline__ static void get(uint32_t w, float (&f)[2]) {
    f[0] = __uint_as_float(w << 16);
    f[1] = __uint_as_float(w & 0xffff0000u);
  }
};
template <>
struct Word<float> {
  static constexpr int E = 1;
  __device__ __forceinline__ static void get(uint32_t w, float (&f)[1]) { f[0] = __uint_as_float(w); }
};

template <typename T>
__global__ __launch_bounds__(256) void proxy_partial_kernel(const ProxyBuildParams p) {
  constexpr int E = Word<T>::E;          // elements per 4-byte word
  constexpr int TPT = kD / E;            // threads per tensor
  extern __shared__ float s_dyn[];
  float* s_acc = s_dyn;                                  // [C][2*kD]
  int* s_cnt = reinterpret_cast<int*>(s_dyn + p.C * 2 * kD);  // [C]

  const int u = blockIdx.x / p.chunks;
  const int ch = blockIdx.x - u * p.chunks;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x;
  const int tensor = tid / TPT;          // 0 = K, 1 = V
  const int col0 = (tid - tensor * TPT) * E;

  for (int i = tid; i < p.C * 2 * kD; i += 2 * TPT) s_acc[i] = 0.f;
  for (int i = tid; i < p.C; i += 2 * TPT) s_cnt[i] = 0;
  __syncthreads();

  const int r0 = ch * p.rows_per_chunk;
  const int r1 = min(p.n, r0 + p.rows_per_chunk);
  const T* base = reinterpret_cast<const T*>(tensor ? p.V : p.K) + (int64_t)s * p.sb + (int64_t)g * p.sh + col0;
  const int32_t* cid = p.cid + (int64_t)u * p.n;

  int cur = -1;
  int run_cnt = 0;
  float run[E];
#pragma unroll
  for (int e = 0; e < E; ++e) run[e] = 0.f;
  bool bad = false;

  auto flush = [&]() {
    if (cur >= 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[cur * 2 * kD + tensor * kD + col0 + e] += run[e];
      if (tid == 0) s_cnt[cur] += run_cnt;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) run[e] = 0.f;
    run_cnt = 0;
  };
  auto take = [&](int c, uint32_t wv) {
    if (c < -1 || c >= p.C) {
      bad = true;
      c = -1;
    }
    if (c != cur) {
      flush();
      cur = c;
    }
    if (c >= 0) {
      float f[E];
      Word<T>::get(wv, f);
#pragma unroll
      for (int e = 0; e < E; ++e) run[e] += f[e];
      run_cnt += 1;
    }
  };

  int j = r0;
  for (; j + kBuildUnroll <= r1; j += kBuildUnroll) {
    uint32_t wv[kBuildUnroll];
    int cv[kBuildUnroll];
#pragma unroll
    for (int i = 0; i < kBuildUnroll; ++i) {
      wv[i] = *reinterpret_cast<const uint32_t*>(base + (int64_t)(j + i) * p.sn);
      cv[i] = cid[j + i];
    }
#pragma unroll
    for (int i = 0; i < kBuildUnroll; ++i) take(cv[i], wv[i]);
  }
  for (; j < r1; ++j) take(cid[j], *reinterpret_cast<const uint32_t*>(base + (int64_t)j * p.sn));
  flush();
  if (bad && tid == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  __syncthreads();

  float* dst = p.part + ((int64_t)u * p.chunks + ch) * p.C * 2 * kD;
  for (int i = tid; i < p.C * 2 * kD; i += 2 * TPT) dst[i] = s_acc[i];
  int* cdst = p.pcount + ((int64_t)u * p.chunks + ch) * p.C;
  for (int i = tid; i < p.C; i += 2 * TPT) cdst[i] = s_cnt[i];
}

__global__ __launch_bounds__(256) void proxy_reduce_kernel(const ProxyBuildParams p) {
  const int u = blockIdx.x / p.C;
  const int b = blockIdx.x - u * p.C;
  const int t = threadIdx.x;  // column of [K | V]
  float a = 0.f;
  int cnt = 0;
  for (int ch = 0; ch < p.chunks; ++ch) {
    const int64_t rec = (int64_t)u * p.chunks + ch;
    a += p.part[(rec * p.C + b) * 2 * kD + t];
    if (t == 0) cnt += p.pcount[rec * p.C + b];
  }
  const int64_t o = ((int64_t)u * p.C + b) * kD;
  if (t < kD) {
    p.sumK[o + t] = a;
  } else {
    p.sumV[o + t - kD] = a;
  }
  if (t == 0) p.count[(int64_t)u * p.C + b] = cnt;
}

hipError_t launch_proxy_build(const ProxyBuildParams& p, int dtype, int units, hipStream_t st) {
  const size_t lds = (size_t)p.C * 2 * kD * sizeof(float) + (size_t)p.C * sizeof(int);
  const dim3 grid(units * p.chunks);
  if (dtype == SDA_BF16) {
    hipLaunchKernelGGL(proxy_partial_kernel<bf16_t>, grid, dim3(2 * kD / 2), lds, st, p);
  } else {
    hipLaunchKernelGGL(proxy_partial_kernel<float>, grid, dim3(2 * kD), lds, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_reduce_kernel, dim3(units * p.C), dim3(2 * kD), 0, st, p);
  return hipGetLastError();
}

}  // namespace sda
