// sda_cluster.hip -- clustering of the keys in the query geometry
// ("OpenAttention: One Percent Is Enough with Tail Proxies", stage 01 of the
// method list and the settings list: keys projected on the top 16 query
// eigenvectors are clustered with k-means, C = 64).
//
// Coordinates are fp64: z = V^T k, the projection summed over d in order
// (exact products), clamped to |z| <= 2048.  A squared distance adds its 16
// terms in coordinate order with no fused multiply-add, so it is the same
// fp64 number wherever it is computed.  A centroid is its rows' mean, formed
// from an exact 64-bit integer sum of the coordinates rounded to 2^-32
// (atomics in any order give the same bits), within 2^-33 of the plain mean.
// The k-means trajectory is therefore reproducible bit for bit.
#include <math.h>

#include "sda_device.hpp"
#include "sda_kernels.hpp"
#include "sda_cluster.hpp"

namespace sda {

// Projection: a lane owns 4 rows x 4 coordinates (lane & 3 picks the
// coordinates); keys pass through LDS 32 dimensions at a time.
template <typename T>
__global__ __launch_bounds__(256) void qgc_project_kernel(const QgcParams p) {
  __shared__ double s_v[kD * kQgcRank];
  __shared__ float s_k[kQgcRows][33];
  const int u = blockIdx.x / qgc_chunks(p.n);
  const int ch = blockIdx.x - u * qgc_chunks(p.n);
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x;
  const int cg = tid & 3, rg = tid >> 2;

  const float* Vu = p.V + (int64_t)u * kD * kQgcRank;
  for (int i = tid; i < kD * kQgcRank; i += 256) s_v[i] = (double)Vu[i];
  const int row0 = ch * kQgcRows;
  const T* kbase = reinterpret_cast<const T*>(p.K) + (int64_t)s * p.sb + (int64_t)g * p.sh;
  double acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0;
  for (int d0 = 0; d0 < kD; d0 += 32) {
    __syncthreads();
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
    for (int e = 0; e < 32; ++e) {
      double uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) uv[i] = s_v[(d0 + e) * kQgcRank + 4 * cg + i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double kd = (double)s_k[4 * rg + r][e];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[r][i] = fma(kd, uv[i], acc[r][i]);  // exact product: one rounding
      }
    }
  }
  bool bad = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = row0 + 4 * rg + r;
    if (j >= p.n) break;
    double zc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double x = acc[r][i];
      if (fabs(x) > kQgcZMax) {
        x = x > 0.0 ? kQgcZMax : -kQgcZMax;
        bad = true;
      }
      zc[i] = x;
    }
    double* dst = p.z + ((int64_t)u * p.n + j) * kQgcRank + 4 * cg;
    *reinterpret_cast<double2*>(dst) = make_double2(zc[0], zc[1]);
    *reinterpret_cast<double2*>(dst + 2) = make_double2(zc[2], zc[3]);
  }
  if (bad) flag_unit(p.flags, u, SDA_FLAG_CLUSTER);
}

// Start: centroid k is the point of row floor((2k + 1) n / (2C)); sums and
// counts cleared.
__global__ __launch_bounds__(256) void qgc_init_kernel(const QgcParams p) {
  const int u = blockIdx.x, C = p.C;
  for (int t = threadIdx.x; t < C * kQgcRank; t += 256) {
    const int k = t / kQgcRank, i = t - k * kQgcRank;
    const int row = (int)(((int64_t)(2 * k + 1) * p.n) / (2 * C));
    p.cent[(int64_t)u * C * kQgcRank + t] = p.z[((int64_t)u * p.n + row) * kQgcRank + i];
    p.sums[(int64_t)u * C * kQgcRank + t] = 0ull;
  }
  for (int k = threadIdx.x; k < C; k += 256) p.cnt[(int64_t)u * C + k] = 0;
}

// One assignment pass: each row to its nearest centroid (ties to the lower
// k), its coordinates added to that centroid's sums.  Two rows per thread
// share each centroid read.
__global__ __launch_bounds__(256) void qgc_assign_kernel(const QgcParams p) {
#pragma clang fp contract(off)  // distances: rounded products and sums, as in a plain loop
  __shared__ double s_c[kCmax * kQgcRank];
  __shared__ unsigned long long s_sum[kCmax * kQgcRank];
  __shared__ int s_cnt[kCmax];
  const int chunks = qgc_assign_chunks(p.n);
  const int u = blockIdx.x / chunks;
  const int ch = blockIdx.x - u * chunks;
  const int C = p.C, tid = threadIdx.x;
  for (int t = tid; t < C * kQgcRank; t += 256) {
    s_c[t] = p.cent[(int64_t)u * C * kQgcRank + t];
    s_sum[t] = 0ull;
  }
  for (int k = tid; k < C; k += 256) s_cnt[k] = 0;
  __syncthreads();

  constexpr int RW = 2;
  int jr[RW];
  double z[RW][kQgcRank];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    jr[r] = ch * kQgcAssignRows + r * 256 + tid;
    const int j = min(jr[r], p.n - 1);
    const double2* src = reinterpret_cast<const double2*>(p.z + ((int64_t)u * p.n + j) * kQgcRank);
#pragma unroll
    for (int q2 = 0; q2 < kQgcRank / 2; ++q2) {
      const double2 v = src[q2];
      z[r][2 * q2] = v.x;
      z[r][2 * q2 + 1] = v.y;
    }
  }
  double best[RW];
  int bk[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    best[r] = INFINITY;
    bk[r] = 0;
  }
  for (int k = 0; k < C; ++k) {
    double c[kQgcRank];
#pragma unroll
    for (int i = 0; i < kQgcRank; ++i) c[i] = s_c[k * kQgcRank + i];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      double d = 0.0;
#pragma unroll
      for (int i = 0; i < kQgcRank; ++i) {
        const double diff = z[r][i] - c[i];
        d = d + diff * diff;
      }
      if (d < best[r]) {
        best[r] = d;
        bk[r] = k;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if (jr[r] >= p.n) continue;
    p.cluster_id[(int64_t)u * p.n + jr[r]] = bk[r];
    atomicAdd(&s_cnt[bk[r]], 1);
#pragma unroll
    for (int i = 0; i < kQgcRank; ++i)  // |z| * 2^32 <= 2^43: rint is exact in fp64 and in int64
      atomicAdd(&s_sum[bk[r] * kQgcRank + i], (unsigned long long)(long long)rint(z[r][i] * kQgcSumScale));
  }
  __syncthreads();
  for (int t = tid; t < C * kQgcRank; t += 256)
    if (s_sum[t]) atomicAdd(&p.sums[(int64_t)u * C * kQgcRank + t], s_sum[t]);
  for (int k = tid; k < C; k += 256)
    if (s_cnt[k]) atomicAdd(&p.cnt[(int64_t)u * C + k], s_cnt[k]);
}

// Centroids = (sum / count) * 2^-32 in fp64 (the integer sum converted with
// one rounding, a correctly rounded division, an exact scaling); empty
// centroids stay; sums and counts cleared for the next pass.
__global__ __launch_bounds__(256) void qgc_update_kernel(const QgcParams p) {
  const int u = blockIdx.x, C = p.C;
  for (int t = threadIdx.x; t < C * kQgcRank; t += 256) {
    const int k = t / kQgcRank;
    const int N = p.cnt[(int64_t)u * C + k];
    const int64_t idx = (int64_t)u * C * kQgcRank + t;
    if (N > 0) p.cent[idx] = ((double)(long long)p.sums[idx] / (double)N) * (1.0 / kQgcSumScale);
    p.sums[idx] = 0ull;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < C; k += 256) p.cnt[(int64_t)u * C + k] = 0;
}

hipError_t launch_qgc(const QgcParams& p, int dtype, int units, int T, hipStream_t st) {
  if (dtype == SDA_BF16) {
    hipLaunchKernelGGL(qgc_project_kernel<bf16_t>, dim3(units * qgc_chunks(p.n)), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL(qgc_project_kernel<float>, dim3(units * qgc_chunks(p.n)), dim3(256), 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qgc_init_kernel, dim3(units), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int t = 1; t <= T; ++t) {
    hipLaunchKernelGGL(qgc_assign_kernel, dim3(units * qgc_assign_chunks(p.n)), dim3(256), 0, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (t < T) {
      hipLaunchKernelGGL(qgc_update_kernel, dim3(units), dim3(256), 0, st, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace sda
