// sda_cluster.hpp -- parameter block and launcher of the clustering kernels
// (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sda.h"

namespace sda {

constexpr int kQgcRank = 16;          // projection rank
constexpr int kQgcRows = 256;         // rows per workgroup of the projection
constexpr int kQgcAssignRows = 512;   // rows per workgroup of an assignment pass
constexpr double kQgcZMax = 2048.0;   // coordinate clamp: keeps the fixed-point sums within int64
constexpr double kQgcSumScale = 4294967296.0;  // 2^32: grid of the centroid sums
constexpr int kQgcMaxN = 1 << 20;     // rows per unit (sums below 2^63)

struct QgcParams {
  const void* K;
  const float* V;              // [units, d, 16]
  int64_t sb, sh, sn;
  int32_t Hkv, n, C;
  double* z;                   // workspace [units, n, 16] coordinates
  double* cent;                // workspace [units, C, 16] centroids
  unsigned long long* sums;    // workspace [units, C, 16] two's-complement sums of the coordinates x 2^32
  int32_t* cnt;                // workspace [units, C]
  int32_t* cluster_id;         // [units, n] output
  int32_t* flags;              // [units] or null
};

__host__ __device__ inline int qgc_chunks(int n) { return (n + kQgcRows - 1) / kQgcRows; }
__host__ __device__ inline int qgc_assign_chunks(int n) { return (n + kQgcAssignRows - 1) / kQgcAssignRows; }

hipError_t launch_qgc(const QgcParams& p, int dtype, int units, int T, hipStream_t st);

}  // namespace sda
