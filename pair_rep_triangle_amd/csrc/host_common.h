// Host-side helpers shared by the C-ABI entry points (tri_mul.cpp, pair_transition.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tri_mul.h"

namespace trimul_host {

// text of the last HIP failure on this thread (tri_mul_last_hip_error)
inline thread_local char g_hip_err[256] = "no HIP error recorded";

inline int hip_fail(hipError_t e, const char* what) {
  snprintf(g_hip_err, sizeof(g_hip_err), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return TRI_MUL_ERR_HIP;
}

// fp32 -> bf16, round to nearest even (NaN stays NaN)
inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// one value in the storage type at dst
inline void store_elem(unsigned char* dst, float v, bool bf16) {
  if (bf16) {
    const uint16_t h = f32_to_bf16_rne(v);
    memcpy(dst, &h, 2);
  } else {
    memcpy(dst, &v, 4);
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline bool overlaps(const void* p, size_t pn, const void* q, size_t qn) {
  if (!p || !q || pn == 0 || qn == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qn && b < a + pn;
}

// the current device, which must be gfx950, and its CU count
inline int check_device(int* dev_out, int* cus_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  *dev_out = dev;
  *cus_out = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  return TRI_MUL_OK;
}

// The device address of the static workspace of tri_mul_forward_static on device `dev`
// (the current device), looked up once per device (tri_mul_static.hip).
int static_workspace(int dev, void** ptr);

}  // namespace trimul_host
