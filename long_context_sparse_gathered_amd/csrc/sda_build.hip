// sda_build.hip -- per-cluster state for the count-aware mean proxies
// ("OpenAttention", method stage 01: per cluster, a count and a mean token
// cached once per request; stored here as count, key sum and value sum).
//
// Two deterministic passes: every workgroup owns (unit, row chunk) and sums
// the chunk's rows per cluster in registers, in row order within each lane
// and in a fixed lane order across lanes; a second kernel adds the chunk
// partials in chunk order.  No atomics, so repeated builds are bitwise
// identical.  The pass streams K and V once (HBM-bound).
#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

constexpr int kBuildRows = 32;   // rows per group; two groups in flight per wave
constexpr int kBuildLoads = kBuildRows / 4;   // row loads per lane per group

// One workgroup = two waves, one for K and one for V, over one (unit, chunk).
// Row layout as in the attention kernels: a 16-lane quarter of the wave reads
// one row (lane r16 its dims [8*r16, 8*r16 + 8)), so one load instruction
// covers four rows.  Each lane keeps a running sum of its quarter's rows for
// the current cluster; on a cluster change the four quarters' runs are added
// in a fixed order and quarter 0 adds the result to this chunk's LDS column
// sums.  Cluster ids are contiguous runs in practice: a group of 32 rows that
// lies in one cluster is summed without per-row checks.  With SQ the K wave
// also sums the squared keys (the diagonal-variance token of stage 01).
template <typename T, bool SQ>
__global__ __launch_bounds__(128) void proxy_partial_kernel(const ProxyBuildParams p) {
  constexpr int NCOL = SQ ? 3 * kD : 2 * kD;   // [K | V | K^2] columns per cluster
  extern __shared__ float s_acc[];       // [C][NCOL] column sums of this chunk

  const int u = blockIdx.x / p.chunks;
  const int ch = blockIdx.x - u * p.chunks;
  const int s = u / p.Hkv;
  const int g = u - s * p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int tensor = tid >> 6;           // 0 = K, 1 = V
  const int r16 = lane & 15;
  const int rq = lane >> 4;              // row of the four a load covers

  for (int i = tid; i < p.C * NCOL; i += 128) s_acc[i] = 0.f;
  __syncthreads();

  const int r0 = ch * p.rows_per_chunk;
  const int r1 = min(p.n, r0 + p.rows_per_chunk);
  const T* base = reinterpret_cast<const T*>(tensor ? p.V : p.K) + (int64_t)s * p.sb + (int64_t)g * p.sh +
                  r16 * kPerLane;
  const int32_t* cid = p.cid + (int64_t)u * p.n;

  int cur = -1;
  int run_cnt = 0;
  int cnt_c = 0;   // K wave: lane c counts the rows of cluster c (C <= 64)
  float run[kPerLane], run2[kPerLane];
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) run[e] = run2[e] = 0.f;
  bool bad = false;

  auto flush = [&]() {
    if (cur >= 0) {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        const float v = sum_rowgroups(run[e]);
        if (rq == 0) s_acc[cur * NCOL + tensor * kD + r16 * kPerLane + e] += v;
      }
      if constexpr (SQ) {
        if (tensor == 0) {
#pragma unroll
          for (int e = 0; e < kPerLane; ++e) {
            const float v = sum_rowgroups(run2[e]);
            if (rq == 0) s_acc[cur * NCOL + 2 * kD + r16 * kPerLane + e] += v;
          }
        }
      }
      if (tensor == 0 && lane == cur) cnt_c += run_cnt;
    }
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) run[e] = run2[e] = 0.f;
    run_cnt = 0;
  };
  auto add_row = [&](const RowChunk<T>& w) {
    float f[kPerLane];
    w.unpack(f);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) run[e] += f[e];
    if constexpr (SQ) {
      if (tensor == 0) {
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) run2[e] = fmaf(f[e], f[e], run2[e]);
      }
    }
  };

  // Groups are double-buffered: the next group's rows are in flight while
  // this group's are summed.  One load brings a group's cluster ids (lane i
  // holds row i of the group, read back with readlane).  Loads past the chunk
  // end re-read its last row and are not summed, so every load is
  // unconditional and the waits count exactly.
  const int ngroups = (r1 - r0 + kBuildRows - 1) / kBuildRows;
  RowChunk<T> wa[kBuildLoads], wb[kBuildLoads];
  int ca, cb;
  auto load_group = [&](int gi, RowChunk<T> (&w)[kBuildLoads], int& cv) {
    const int j0 = r0 + gi * kBuildRows;
    cv = cid[min(j0 + (lane & (kBuildRows - 1)), r1 - 1)];
#pragma unroll
    for (int i = 0; i < kBuildLoads; ++i) w[i].load_stream(base + (int64_t)min(j0 + 4 * i + rq, r1 - 1) * p.sn);
  };
  auto sum_group = [&](int gi, const RowChunk<T> (&w)[kBuildLoads], int cv) {
    const int left = r1 - (r0 + gi * kBuildRows);
    if (left <= 0) return;
    const int c0 = __builtin_amdgcn_readfirstlane(cv);
    const bool valid = (lane & (kBuildRows - 1)) < left;
    const bool one = left >= kBuildRows && __ballot(valid && cv != c0) == 0 && c0 >= -1 && c0 < p.C;
    if (one) {
      if (c0 != cur) {
        flush();
        cur = c0;
      }
      if (c0 >= 0) {
#pragma unroll
        for (int i = 0; i < kBuildLoads; ++i) add_row(w[i]);
        run_cnt += kBuildRows;
      }
      return;
    }
    for (int i = 0; i < min(left, kBuildRows); ++i) {
      int c = __builtin_amdgcn_readlane(cv, i);
      if (c < -1 || c >= p.C) {
        bad = true;
        c = -1;
      }
      if (c != cur) {
        flush();
        cur = c;
      }
      if (c >= 0) {
        // row i sits in load i / 4 of quarter i % 4
#pragma unroll
        for (int k = 0; k < kBuildLoads; ++k)
          if (k == (i >> 2) && rq == (i & 3)) add_row(w[k]);
        run_cnt += 1;
      }
    }
  };
  load_group(0, wa, ca);
  for (int gi = 0; gi < ngroups; gi += 2) {
    load_group(gi + 1, wb, cb);
    sum_group(gi, wa, ca);
    load_group(gi + 2, wa, ca);
    sum_group(gi + 1, wb, cb);
  }
  flush();
  if (bad && tid == 0) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
  __syncthreads();

  float* dst = p.part + ((int64_t)u * p.chunks + ch) * p.C * NCOL;
  for (int i = tid; i < p.C * NCOL; i += 128) dst[i] = s_acc[i];
  if (tid < p.C) p.pcount[((int64_t)u * p.chunks + ch) * p.C + tid] = cnt_c;
}

__global__ __launch_bounds__(384) void proxy_reduce_kernel(const ProxyBuildParams p) {
  const int u = blockIdx.x / p.C;
  const int b = blockIdx.x - u * p.C;
  const int t = threadIdx.x;  // column of [K | V | K^2]
  const int ncol = p.sumK2 ? 3 * kD : 2 * kD;
  if (t >= ncol) return;
  float a = 0.f;
  int cnt = 0;
  for (int ch = 0; ch < p.chunks; ++ch) {
    const int64_t rec = (int64_t)u * p.chunks + ch;
    a += p.part[(rec * p.C + b) * ncol + t];
    if (t == 0) cnt += p.pcount[rec * p.C + b];
  }
  const int64_t o = ((int64_t)u * p.C + b) * kD;
  if (t < kD) {
    p.sumK[o + t] = a;
  } else if (t < 2 * kD) {
    p.sumV[o + t - kD] = a;
  } else {
    p.sumK2[o + t - 2 * kD] = a;
  }
  if (t == 0) p.count[(int64_t)u * p.C + b] = cnt;
}

hipError_t launch_proxy_build(const ProxyBuildParams& p, int dtype, int units, hipStream_t st) {
  const bool sq = p.sumK2 != nullptr;
  const size_t lds = (size_t)p.C * (sq ? 3 : 2) * kD * sizeof(float);
  const dim3 grid(units * p.chunks);
  if (dtype == SDA_BF16) {
    if (sq) hipLaunchKernelGGL((proxy_partial_kernel<bf16_t, true>), grid, dim3(128), lds, st, p);
    else hipLaunchKernelGGL((proxy_partial_kernel<bf16_t, false>), grid, dim3(128), lds, st, p);
  } else {
    if (sq) hipLaunchKernelGGL((proxy_partial_kernel<float, true>), grid, dim3(128), lds, st, p);
    else hipLaunchKernelGGL((proxy_partial_kernel<float, false>), grid, dim3(128), lds, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_reduce_kernel, dim3(units * p.C), dim3((sq ? 3 : 2) * kD), 0, st, p);
  return hipGetLastError();
}

}  // namespace sda
