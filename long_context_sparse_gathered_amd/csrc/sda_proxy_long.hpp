// sda_proxy_long.hpp -- limits and launcher of the proxy decode for lists
// longer than the one-pass kernel holds (sda_proxy_long.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "sda_kernels.hpp"

namespace sda {

constexpr int kLongWaves = 8;                              // waves per workgroup
constexpr int kLongMaxPerWave = 128;                       // list entries per wave
constexpr int kLongMaxList = kLongWaves * kLongMaxPerWave;  // entries per unit

// Entries per wave for a list of m entries (a multiple of 16).
inline int long_chunk(int m) {
  const int per = (m + kLongWaves - 1) / kLongWaves;
  return (per + 15) / 16 * 16;
}

// One workgroup per unit and no workspace; p.chunk = long_chunk(p.m).
hipError_t launch_proxy_long(const AttnParams& p, int G, hipStream_t st);

}  // namespace sda
