// Launch interface of the pair-transition kernel (host code in pair_transition.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace trimul {

struct TransitionArgs {
  const void* z;      // [pairs][cz]
  const void* mask;   // [pairs], or the one-element `one` when there is no mask
  void* out;          // [pairs][cz] (may be z itself)
  const void* w1;     // [hp][cz]  W_1 diag(gamma), padded hidden rows zero
  const void* w2;     // [cz][hp]  W_2 with rows and columns in the kernel's order
  const float* b1;    // [hp]      W_1 beta + b_1
  const float* b2;    // [cz]      b_2 in the kernel's row order
  long long pairs;    // B * N * N
  int cz, hp, mask_all, num_cus;
};

// LDS of one workgroup: W_1 [hp][cz] and W_2 [cz][hp] with 16 bytes of padding per row,
// then the fp32 biases
inline size_t transition_lds_bytes(int cz, int hp, size_t esz) {
  return (size_t)hp * (cz * esz + 16) + (size_t)cz * (hp * esz + 16) + ((size_t)hp + cz) * 4;
}

// c_z chunk groups the kernel is compiled for (c_z = kz * 32 in bf16, kz * 16 in fp32);
// both layers' weights must fit one workgroup's LDS
inline bool transition_supported(bool bf16, int cz, int hp) {
  const int kg = bf16 ? 32 : 16;
  if (cz % kg || cz / kg < 1 || cz / kg > 4) return false;
  if (hp % kg || hp < kg) return false;
  return transition_lds_bytes(cz, hp, bf16 ? 2 : 4) <= 160 * 1024;
}

hipError_t launch_transition(bool bf16, const TransitionArgs& a, hipStream_t st);

}  // namespace trimul
