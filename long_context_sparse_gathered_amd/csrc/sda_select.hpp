// sda_select.hpp -- parameter blocks and launchers of the selector kernels
// (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sda.h"

namespace sda {

constexpr int kQgsRank = 32;        // subspace rank r
constexpr int kQgsRows = 256;       // rows per workgroup of the code builder
constexpr int kQgsMaxN = 1 << 20;   // row positions fit the 20-bit field of a selection key
constexpr int kQgsMaxG = 8;

// Selection key of one row, 64 bits:
//   [19:0]  2^20 - 1 - j           (lower position = larger key)
//   [39:20] S_j + 2^19             (the QGS score, |S_j| <= 32 * 127 * 127 < 2^19)
//   [46:40] cluster id, 127 = none
//   [47]    eligible (selectable by its cluster's budget)
constexpr int kKeyBits = 40;
constexpr uint64_t kKeyMask = (1ull << kKeyBits) - 1;
constexpr int kNoCluster = 127;

struct QgsBuildParams {
  const void* K;
  const float* U;              // [units, d, r]
  int64_t sb, sh, sn;
  int32_t Hkv, n;
  int32_t chunks;              // row chunks of kQgsRows per unit
  double* part;                // [units, chunks, r] chunk maxima of |y|
  double* y;                   // [units, n, r] projections kept by pass 1 for pass 2, or null (recomputed)
  int8_t* codes;               // [units, n, r]
  double* kmax;                // [units, r]
};

struct QgsSelectParams {
  const void* q;               // [B, Hq, d]
  const int32_t* cid;          // [units, n]
  const int32_t* count;        // [units, C]
  const float* sumK;           // [units, C, d]
  const float* sumK2;          // [units, C, d]
  const float* U;              // [units, d, r]
  const int8_t* codes;         // [units, n, r]
  const double* kmax;          // [units, r]
  int32_t B, Hq, Hkv, n, G, C;
  int32_t n_sink, n_local, E, m;
  float scale;
  // workspace
  uint64_t* keys;              // [units, n]
  uint32_t* wq;                // [units, G, r / 4] packed int8 query weights
  int32_t* wbudget;            // [units, C]
  int32_t* wavail;             // [units, C]
  // outputs
  int32_t* idx;                // [units, m]
  int32_t* idx_len;            // [units]
  int32_t* idx_cluster;        // [units, m]
  int32_t* budget;             // [units, C] or null
  int32_t* flags;              // [units] or null
};

inline int qgs_chunks(int n) { return (n + kQgsRows - 1) / kQgsRows; }

hipError_t launch_qgs_build(const QgsBuildParams& p, int dtype, int units, hipStream_t st);
hipError_t launch_qgs_select(const QgsSelectParams& p, int dtype, hipStream_t st);

}  // namespace sda
