// Shape of the wave-independent input-gate kernel's weight groups, shared by the host (which
// stores each group's weights as the kernel's LDS image) and the launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "launch.h"

namespace trimul {

constexpr int K1W_WAVES = 8;
constexpr int K1W_THREADS = 64 * K1W_WAVES;
constexpr int K1W_TP = 64;  // pairs per wave tile

// A group of ug units holds ug * 32 weight rows (gate and projection rows of each unit's
// 16 channels), each four chunk groups along c_z: 256 bytes in bf16 (128 values) and in
// fp32 (64 values). Its LDS image is the rows (chunk c of row r at position c ^ (r & 15))
// followed by the rows' fp32 start values.
constexpr size_t K1W_ROW_BYTES = 256;
__host__ __device__ inline size_t k1w_image_bytes(int ug) {
  return (size_t)ug * 32 * (K1W_ROW_BYTES + 4);
}
// LDS of one workgroup: the image, then each wave's tile masks
__host__ __device__ inline size_t k1w_lds_bytes(int ug) {
  return k1w_image_bytes(ug) + (size_t)K1W_WAVES * K1W_TP * sizeof(float);
}
// Units per group for c hidden channels (2 c / 16 units: a and b, 16 channels each): the
// largest even divisor of the unit count up to 16 whose LDS fits one workgroup; 0 if none.
inline int k1w_group_units(int c) {
  const int units = 2 * (c / 16);
  for (int g = units < 16 ? units : 16; g >= 2; g -= 2)
    if (units % g == 0 && k1w_lds_bytes(g) <= LDS_PER_CU) return g;
  return 0;
}

}  // namespace trimul
