// sda_gather.hip -- a measurement aid, not part of the method: it reads the
// listed K and V rows of every (sequence, KV head) unit, and optionally a
// block of per-unit state, in a chosen launch shape, and folds every loaded
// word into one checksum per wave so that no load is dead.  Timing it beside
// the decode step gives the rate at which the memory system delivers the same
// random 256-byte rows with no arithmetic at all.
//
// Shape: `parts` workgroups of `waves` waves per unit.  Part p takes entries
// [p*EP, (p+1)*EP) of the unit's list (EP = ceil(m / parts)); its wave w takes
// a contiguous run of EW = ceil(EP / waves) of those; row group `sub` (16
// lanes) of the wave takes every fourth entry of the run, so one load
// instruction covers four rows of 256 bytes.  All row loads are issued before
// any is used, keys and values alternating.
#include "sda_device.hpp"
#include "sda_kernels.hpp"

namespace sda {

namespace {

using rsrc_g = __amdgpu_buffer_rsrc_t;
constexpr int kGatherNT = 2;  // streaming cache policy (read once)

template <int WAVES, int R>
__global__ __launch_bounds__(WAVES * 64) void gather_rows_kernel(const GatherParams p) {
  const int u = blockIdx.x / p.parts;
  const int part = blockIdx.x - u * p.parts;
  const int s = u / p.Hkv, g = u - s * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, sub = lane >> 4;
  const int EP = (p.m + p.parts - 1) / p.parts;
  const int e0 = part * EP;
  const int e1 = min(p.m, e0 + EP);
  const int EW = (EP + WAVES - 1) / WAVES;
  const int wb = e0 + w * EW;
  const int we = min(e1, wb + EW);
  const int64_t lbase = (int64_t)u * p.m;

  int off[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int e = wb + 4 * k + sub;
    const bool ok = e < we;
    const int j = p.idx[lbase + (ok ? e : 0)];
    off[k] = (ok && (unsigned)j < (unsigned)p.n) ? j * p.row_bytes + 16 * r16 : kMaxUnitBytes;
  }
  const int64_t kvoff = ((int64_t)s * p.sb + (int64_t)g * p.sh) * p.esize;
  const int span = (int)(((int64_t)(p.n - 1) * p.sn + kD) * p.esize);
  const rsrc_g rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(p.K) + kvoff), 0,
                                                      span, 0x00020000);
  const rsrc_g rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(p.V) + kvoff), 0,
                                                      span, 0x00020000);
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  v4u kr[R], vr[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    kr[k] = __builtin_amdgcn_raw_buffer_load_b128(rk, off[k], 0, kGatherNT);
    vr[k] = __builtin_amdgcn_raw_buffer_load_b128(rv, off[k], 0, kGatherNT);
  }
  // per-unit state: this part's share, 16 bytes per thread and step
  uint32_t x = 0;
  if (p.state_bytes > 0) {
    const int64_t sp = ((p.state_bytes + p.parts - 1) / p.parts + 15) / 16 * 16;  // 16-byte aligned shares
    const int64_t sb0 = part * sp, sb1 = min(p.state_bytes, sb0 + sp);
    const char* base = static_cast<const char*>(p.state) + (int64_t)u * p.state_bytes;
    for (int64_t b = sb0 + 16 * (int64_t)tid; b + 16 <= sb1; b += 16 * WAVES * 64) {
      const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base + b));
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k) x ^= kr[k][0] ^ kr[k][1] ^ kr[k][2] ^ kr[k][3] ^ vr[k][0] ^ vr[k][1] ^ vr[k][2] ^ vr[k][3];
  // fold the wave; one plain store per wave (no atomics: device-scope atomics
  // on a few shared words would add their own drain time to the launch)
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x ^= (uint32_t)__shfl_xor((int)x, sh, 64);
  if (lane == 0) p.checksum[(int64_t)blockIdx.x * WAVES + w] = x;
}

template <int WAVES>
hipError_t launch_w(const GatherParams& p, int R, int grid, hipStream_t st) {
  constexpr int kMaxR = WAVES >= 16 ? 12 : 24;  // the row registers fit without spilling
  const dim3 block(WAVES * 64);
#define SDA_GATHER_CASE(RR)                                                           \
  if (RR <= kMaxR && R <= RR) {                                                      \
    hipLaunchKernelGGL((gather_rows_kernel<WAVES, (RR <= kMaxR ? RR : kMaxR)>), dim3(grid), block, 0, st, p); \
    return hipGetLastError();                                                         \
  }
  SDA_GATHER_CASE(2)
  SDA_GATHER_CASE(4)
  SDA_GATHER_CASE(8)
  SDA_GATHER_CASE(12)
  SDA_GATHER_CASE(16)
  SDA_GATHER_CASE(24)
#undef SDA_GATHER_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int gather_rows_per_group(int m, int waves, int parts) {
  const int EP = (m + parts - 1) / parts;
  const int EW = (EP + waves - 1) / waves;
  return (EW + 3) / 4;
}

hipError_t launch_gather_rows(const GatherParams& p, int waves, int units, hipStream_t st) {
  const int R = gather_rows_per_group(p.m, waves, p.parts);
  const int grid = units * p.parts;
  if (waves == 4) return launch_w<4>(p, R, grid, st);
  if (waves == 8) return launch_w<8>(p, R, grid, st);
  if (waves == 16) return launch_w<16>(p, R, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace sda
