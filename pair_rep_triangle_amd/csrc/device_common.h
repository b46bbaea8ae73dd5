// Device-side helpers shared by the three kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace trimul {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int chunk_t;  // 16 bytes
typedef __attribute__((ext_vector_type(2))) unsigned int half_t;   // 8 bytes

// E = elements of T per 16-byte chunk; KG = k covered by one 16x16 MFMA chunk group
// (4 lane groups x one chunk each).
template <class T> struct Traits;
template <> struct Traits<bf16> { static constexpr int E = 8; static constexpr int KG = 32; };
template <> struct Traits<float> { static constexpr int E = 4; static constexpr int KG = 16; };

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

__device__ __forceinline__ chunk_t ld16(const void* p) { return *(const chunk_t*)p; }
__device__ __forceinline__ void st16(void* p, chunk_t v) { *(chunk_t*)p = v; }
__device__ __forceinline__ f32x4 ld16f(const float* p) { return *(const f32x4*)p; }

// chunk <-> floats
__device__ __forceinline__ void unpack(chunk_t c, float* f, bf16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(c[i] << 16);
    f[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(chunk_t c, float* f, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
}
__device__ __forceinline__ chunk_t pack(const float* f, bf16) {
  chunk_t c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x2 h = {(bf16)f[2 * i], (bf16)f[2 * i + 1]};
    c[i] = __builtin_bit_cast(unsigned int, h);
  }
  return c;
}
__device__ __forceinline__ chunk_t pack(const float* f, float) {
  chunk_t c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(f[i]);
  return c;
}

// Four values -> one 8-byte (bf16) or 16-byte (fp32) store.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
  half_t v = {__builtin_bit_cast(unsigned int, lo), __builtin_bit_cast(unsigned int, hi)};
  *(half_t*)p = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(f32x4*)p = f32x4{a, b, c, d};
}

// 16x16 output tile: D[row][col] += sum_k A[row][k] B[col][k] over one chunk group. Lane l
// hands A row l%16 and B column l%16, each as one 16-byte chunk of consecutive k (the same
// lane -> k assignment for A and B, so every k of the group is summed exactly once).
__device__ __forceinline__ f32x4 mma16(f32x4 acc, chunk_t a, chunk_t b, bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, chunk_t a, chunk_t b, float) {
  f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
  return acc;
}
// 32x32 output tile over one chunk group (16 k for bf16, 8 k for fp32); lane l: row/col l%32.
__device__ __forceinline__ f32x16 mma32(f32x16 acc, chunk_t a, chunk_t b, bf16) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(f32x16 acc, chunk_t a, chunk_t b, float) {
  f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc, 0, 0, 0);
  return acc;
}

// Sum over the 8 consecutive lanes 8q .. 8q+7 (two quad permutes, then the half-row mirror),
// every lane of the group receives the total.
#define TRIMUL_DPP(v, ctrl) \
  __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true))
__device__ __forceinline__ float sum8(float v) {
  v += TRIMUL_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
  v += TRIMUL_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
  v += TRIMUL_DPP(v, 0x141);  // row_half_mirror
  return v;
}

// out = p * m * sigmoid(g) with the gate pre-activation given as g2 = -g * log2(e)
// (the host scales the gate rows by -log2 e): sigmoid(g) = 1 / (1 + 2^g2).
__device__ __forceinline__ float gate_mul(float p_times_m, float g2) {
  return p_times_m * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g2));
}

// LayerNorm of one row held by the 8 lanes of a pair: lane `part` holds chunks part,
// part+8, ... of the row in v[0..NCH); chunk indices >= nreal are padding (zero, and not
// counted). Normalises v in place to (x - mean) * rstd over the `width` real values
// (two passes in fp32); padding chunks stay zero.
template <class T, int NCH>
__device__ __forceinline__ void normalize_row(chunk_t (&v)[NCH], int part, int nreal, int width) {
  constexpr int E = Traits<T>::E;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    float f[E];
    unpack(v[i], f, T());
#pragma unroll
    for (int e = 0; e < E; ++e) s += f[e];
  }
  const float inv_w = 1.0f / (float)width;
  const float mean = sum8(s) * inv_w;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (part + 8 * i < nreal) {
      float f[E];
      unpack(v[i], f, T());
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = f[e] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = rsqrtf(sum8(q) * inv_w + TRI_MUL_LN_EPS_F);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (part + 8 * i < nreal) {
      float f[E];
      unpack(v[i], f, T());
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] = (f[e] - mean) * rstd;
      v[i] = pack(f, T());
    }
  }
}

}  // namespace trimul
