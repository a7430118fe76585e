// sda_proxy_long.hpp -- limits and launcher of the two-launch proxy decode
// for lists longer than the one-pass kernel holds (sda_proxy_long.hip).
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

// Workspace floats per unit: the listed rows' weights [G][8 * chunk], then
// the cluster coefficients [C][G], the maxima [G] and the normalisers [G].
inline size_t long_weights_floats(int G, int m) { return (size_t)G * kLongWaves * long_chunk(m); }
inline size_t long_coef_floats(int G, int C) { return (size_t)C * G + 2 * (size_t)G; }

// p.part: weights of all units, p.cpart: coefficient blocks, p.chunk = long_chunk(m).
hipError_t launch_proxy_long(const AttnParams& p, int G, hipStream_t st);

}  // namespace sda
