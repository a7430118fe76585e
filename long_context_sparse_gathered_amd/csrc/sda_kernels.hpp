// sda_kernels.hpp -- kernel parameter blocks and host launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sda.h"

namespace sda {

constexpr int kD = 128;          // head dimension supported by the kernels
constexpr int kCmax = 64;        // clusters per unit supported by the kernels
constexpr int kPartStride = 264; // floats per (unit, split, head) partial
// Largest byte span of one unit's K (or V) rows: rows are addressed with
// 32-bit buffer offsets, and offsets from here up are the "absent row" marker.
constexpr int kMaxUnitBytes = 0x7ffffe00;

// One parameter block for the attention kernels (passed by value).
struct AttnParams {
  const void* q;               // [B,Hq,d] dims.dtype, or fp32 when q_f32
  const void* K;
  const void* V;
  const int32_t* idx;          // [B,Hkv,m]        (sparse modes)
  const int32_t* idx_len;      // [B,Hkv] or null
  const float* logw;           // [B,Hkv,m] or null
  int64_t sb, sh, sn;          // K/V element strides
  int32_t B, Hq, Hkv, n, m;
  float qscale;                // scale * log2(e)
  int32_t q_f32;

  // PROXY
  int32_t C;
  const int32_t* idx_cluster;
  const int32_t* cluster_id;
  const int32_t* count;
  const float* sumK;
  const float* sumV;

  // PRIOR
  const float* mu_Q;
  const float* mu_K;
  const float* O_est;
  const float* maxP;
  const float* sumP;
  float lambda;
  int32_t prior_n;             // rows [0, prior_n) covered by the prior

  // SAMPLED
  float scale;                 // logit scale (fp32 value, widened for fp64 statistics)
  double eps, z;
  int32_t b0;
  uint64_t seed;
  int32_t b_cap;
  int32_t* b_out;              // [B,Hkv] or null
  double* bstar_out;           // [B,Hkv] or null
  int32_t* samples_out;        // [B,Hkv,b_cap] or null
  int32_t nz;                  // verified budget: splits of delta (0 = the plain budget)
  double zs[2 * SDA_MAX_Z_SPLITS];  // per split (Phi^-1(1 - d_N/2), Phi^-1(1 - d_D/2))
  double* wstat;               // workspace: [units, G*(2 + d)] fp64 M, D_f, N_f of the exact part
  double* wexact;              // workspace: [units, splits, G*(2 + d)] fp64 records of the I_f shares
  double* wbase;               // workspace: [units, G*(4 + d)] fp64 moments of the base draws
  int32_t* wb;                 // workspace: [units] sample budget b
  int32_t* wsched;             // workspace: [units + 1] first draw work item of each unit
  int32_t draw_grid;           // draw workgroups of a full round (set by the launcher)

  // split-K
  int32_t splits;              // WGs per unit
  int32_t chunk;               // entries (rows) per split
  float* part;                 // [units, splits, G, kPartStride]
  float* cpart;                // [units, splits, C, kClusterRec] (split-K proxy decode)
  float* ksum;                 // [units, splits, d] (prior build)

  // outputs
  float* out;                  // [B,Hq,d]   (prior build: O_est)
  float* lse;                  // [B,Hq]     (prior build: maxP)
  float* aux;                  // prior build: sumP
  float* aux2;                 // prior build: mu_K
  int32_t* flags;              // [B,Hkv] or null
};

// Stream-kernel modes.
enum StreamMode { kModeSparse = 0, kModePrior = 1, kModeDense = 2, kModeBuildPrior = 3, kModeProxy = 4 };

// Per (unit, split, cluster) record of the split-K proxy decode: the listed
// rows' value sum [0, 128), logit sums per head (log2 units) [128, 136), and
// the listed-row count (int32 bits) at 136.
constexpr int kClusterRec = 144;

struct ProxyBuildParams {
  const void* K;
  const void* V;
  const int32_t* cid;          // [B,Hkv,n]
  int64_t sb, sh, sn;
  int32_t Hkv, n, C;
  int32_t rows_per_chunk;
  int32_t chunks;
  float* part;                 // [units, chunks, C, 2*d or 3*d]
  int32_t* pcount;             // [units, chunks, C]
  int32_t* count;              // outputs
  float* sumK;
  float* sumV;
  float* sumK2;                // or null
  int32_t* flags;
};

// Host launchers (return hipSuccess or the launch error).
hipError_t launch_sparse_unit(const AttnParams& p, int dtype, int G, bool proxy, int ns,
                              hipStream_t st);
hipError_t launch_stream(const AttnParams& p, int dtype, int G, int mode, hipStream_t st);
hipError_t launch_merge(const AttnParams& p, int G, int mode, hipStream_t st);
// bf16 split-K kernel on the matrix cores: entries per workgroup per batch
// are 64 * kStreamMfmaTiles; the prior needs 3G <= 16.
constexpr int kStreamMfmaTiles = 2;
constexpr int kStreamMfmaStep = 64 * kStreamMfmaTiles;
// entries of a chunk of the direct-to-LDS streaming kernel (plain lists and the
// prior), whose list is staged in LDS
constexpr int kStreamDmaMaxChunk = 1024;
hipError_t launch_stream_mfma(const AttnParams& p, int G, int mode, hipStream_t st);
hipError_t launch_sampled(const AttnParams& p, int dtype, int G, hipStream_t st);

// Sampled tail limits: the deterministic list and the base draws live in LDS.
constexpr int kSampMaxList = 4096;
constexpr int kSampMaxB0 = 256;
// The fresh draws are cut into work items of kDrawChunk draws, numbered unit
// by unit; each draw workgroup takes a contiguous range of work items.
constexpr int kDrawChunk = 256;
constexpr int kDrawRec = 4 + 128;        // floats per (work item, head) partial: m, l, -, -, acc[d]
constexpr int kSampMaxUnits = 4096;
constexpr int kDrawGrid = 1024;          // draw workgroups (upper bound); the launch takes one round
__host__ __device__ inline int sampled_max_items(int n) { return (n + kDrawChunk - 1) / kDrawChunk; }
// Workgroups per unit that share the exact pass over I_f: with the unit's
// base-draw workgroup, about 256 in all (the kernel holds one per CU).
constexpr int kSampMaxSplits = 8;  // exact-part workgroups per unit (at most)
inline int sampled_exact_splits(int units) {
  const int s = 256 / units - 1;
  return s < 1 ? 1 : (s > kSampMaxSplits ? kSampMaxSplits : s);
}
hipError_t launch_proxy_build(const ProxyBuildParams& p, int dtype, int units, hipStream_t st);
// Row chunks of the proxy builder: 4096 rows each (a workgroup holds C*2*kD
// fp32 column sums in LDS and writes them out once per chunk), shorter when
// there are too few (unit, chunk) workgroups to fill the chip, but at least
// 256 rows; always a multiple of 32 rows.
inline void proxy_build_shape(int units, int n, int C, int* chunks, int* rows) {
  (void)C;
  int ch = (n + 4095) / 4096;
  const int fill = (1280 + units - 1) / units;
  const int max_ch = (n + 255) / 256;
  const int want = fill < max_ch ? fill : max_ch;
  if (ch < want) ch = want;
  int r = (n + ch - 1) / ch;
  r = (r + 31) / 32 * 32;
  *rows = r;
  *chunks = (n + r - 1) / r;
}

// Row-gather measurement kernel (sda_gather.hip).
struct GatherParams {
  const void* K;
  const void* V;
  const int32_t* idx;        // [units, m]
  const void* state;         // [units, state_bytes] or null
  int64_t state_bytes;
  int64_t sb, sh, sn;        // element strides
  int32_t esize, row_bytes;  // element size, row stride in bytes
  int32_t Hkv, n, m, parts;
  uint32_t* checksum;        // [units * parts * waves]
};
int gather_rows_per_group(int m, int waves, int parts);
hipError_t launch_gather_rows(const GatherParams& p, int waves, int units, hipStream_t st);

// Largest slot count the one-workgroup-per-unit kernel is built for.
constexpr int kUnitWaves = 8;
// Tiles of 16 list entries per wave in the bf16 unit kernel (LDS-bound).
inline int unit_max_tiles(int G) { return G >= 8 ? 3 : 4; }
constexpr int kUnitMaxSlots = 16;
inline int unit_slots_for(int m) {
  const int need = (m + 4 * kUnitWaves - 1) / (4 * kUnitWaves);
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 12) return 12;
  if (need <= 16) return 16;
  return 0;
}

}  // namespace sda
