// Launch interface of the pair-transition kernel (host code in pair_transition.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace trimul {

struct TransitionArgs {
  const void* z;      // [pairs][cz]
  const void* mask;   // [pairs], or the one-element `one` when there is no mask
  void* out;          // [pairs][cz] (may be z itself)
  // the weights as the kernel's LDS image (transition_lds_bytes): W_1 diag(gamma)
  // [hp][cz + pad] (padded hidden rows zero), W_2 [cz][hp + pad] with rows and columns in
  // the kernel's order, then fp32 b_1' = W_1 beta + b_1 [hp] and b_2 [cz] (kernel order);
  // pad = 16 bytes of zeros per row
  const void* image;
  size_t image_bytes;
  long long pairs;    // B * N * N
  int cz, hp, mask_all, num_cus;
  int wide;           // the weights stream through LDS (pair_transition_wide_kernel)
  int czp;            // wide: c_z padded to the compiled width
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

// The wide form (bf16): c_z padded to 128, 256, 384 or 512; per hidden group of 32 units a
// block of 128 czp bytes (W_1 rows [32][czp], then W_2 columns [czp][32], both in the
// kernel's swizzled order), then fp32 b_1' [hp] and b_2 [czp]. LDS: two group buffers and
// the biases.
inline int transition_wide_czp(int cz) {
  const int czp = (cz + 127) / 128 * 128;
  return czp <= 512 ? czp : 0;
}
size_t transition_wide_lds_bytes(int czp, int hp);
inline bool transition_wide_supported(bool bf16, int cz, int hp) {
  if (!bf16 || cz % 32 || cz < 32) return false;
  const int czp = transition_wide_czp(cz);
  if (czp == 0 || hp % 32 || hp < 32) return false;
  return (size_t)2 * 128 * czp + ((size_t)hp + czp) * 4 <= 160 * 1024;
}

hipError_t launch_transition(bool bf16, const TransitionArgs& a, hipStream_t st);
hipError_t launch_transition_wide(const TransitionArgs& a, hipStream_t st);

}  // namespace trimul
