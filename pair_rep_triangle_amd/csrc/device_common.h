// Device-side helpers shared by the three kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace trimul {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int chunk_t;  // 16 bytes
typedef __attribute__((ext_vector_type(2))) unsigned int half_t;   // 8 bytes

// z and out are distinct buffers (restrict-qualified) unless the kernel adds the update
// to z, where out may be z itself.
template <class T, bool RESID>
using ZIn = std::conditional_t<RESID, const T*, const T* __restrict__>;
template <class T, bool RESID>
using ZOut = std::conditional_t<RESID, T*, T* __restrict__>;

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
// 16 bytes from an LDS address that is only 8-byte aligned (bf16 staging rows); fp32
// staging rows are 16-byte aligned.
__device__ __forceinline__ chunk_t ld16_lds8(const bf16* p) {
  const half_t lo = *(const half_t*)p, hi = *(const half_t*)(p + 4);
  return chunk_t{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ chunk_t ld16_lds8(const float* p) { return ld16(p); }

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane i
// of the wave writes lds_base + 16*i, where lds_base is wave-uniform. Completion is
// counted by vmcnt. (Wrapped in a plain device function so that kernel templates using
// it still get their host-side launch stubs.)
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
}

// Buffer resources for plain byte-addressed access: a read whose per-lane plus immediate
// offset is at or past `bytes` returns zero, a store there is dropped. The scalar offset
// of a load or store is NOT part of that check, so anything that must stay inside the
// extent goes in the per-lane or immediate offset, or moves the resource's base. Loads
// through them take a 32-bit per-lane offset, so per-lane offsets that stay the same from
// tile to tile never have to be recomputed into registers a load in flight still reads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}
// The same with an extent the caller already holds in 32 bits (scalar compares only; a
// 64-bit ordered compare has no scalar form and would take vector registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_u32(const void* base, unsigned int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
// Flat copy of `chunks` 16-byte chunks from device memory to LDS by a workgroup of NT
// threads: whole batches of 16 chunks per thread with all 16 loads in flight before the
// first store and no per-chunk predicate (which would put each load and store behind its
// own branch), then the remainder one chunk per thread at a time. `after_first_loads`
// runs once, right after the first batch's loads are issued (or before the remainder
// when there is no whole batch): the place for other loads that may wait behind them.
template <int NT, class F>
__device__ __forceinline__ void copy_image(const chunk_t* __restrict__ src, chunk_t* dst,
                                           int chunks, int tid, F after_first_loads) {
  const int whole = chunks / (16 * NT) * (16 * NT);
  chunk_t v[16];
  if (whole > 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = src[k * NT + tid];
  }
  after_first_loads();  // one call site: its code appears once
  if (whole > 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[k * NT + tid] = v[k];
  }
  for (int base = 16 * NT; base < whole; base += 16 * NT) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = src[base + k * NT + tid];
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[base + k * NT + tid] = v[k];
  }
  for (int idx = whole + tid; idx < chunks; idx += NT) dst[idx] = src[idx];
}

// Bytes left of an extent `bytes` after skipping `skip` (both below 2^31), at least 0. A
// signed max: the unsigned "a > b ? a - b : 0" becomes a saturating subtract, which has
// only a vector form, and a resource field in a vector register turns every load through
// it into a loop over lanes.
__device__ __forceinline__ unsigned int bytes_after(unsigned int bytes, unsigned int skip) {
  const int d = (int)bytes - (int)skip;
  return (unsigned int)(d > 0 ? d : 0);
}
__device__ __forceinline__ chunk_t load16(__amdgpu_buffer_rsrc_t r, unsigned int voff, int soff) {
  return __builtin_bit_cast(chunk_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}
// one element of the storage type
__device__ __forceinline__ bf16 load_elem(__amdgpu_buffer_rsrc_t r, unsigned int voff, int soff, bf16) {
  return __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, soff, 0));
}
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t r, unsigned int voff, int soff, float) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0));
}

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

// Element-wise a + b of two chunks, summed in fp32 and rounded once to the storage type.
__device__ __forceinline__ chunk_t add_chunks(chunk_t a, chunk_t b, bf16) {
  float fa[8], fb[8];
  unpack(a, fa, bf16());
  unpack(b, fb, bf16());
#pragma unroll
  for (int e = 0; e < 8; ++e) fa[e] += fb[e];
  return pack(fa, bf16());
}
__device__ __forceinline__ chunk_t add_chunks(chunk_t a, chunk_t b, float) {
  chunk_t c;
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = __float_as_uint(__uint_as_float(a[e]) + __uint_as_float(b[e]));
  return c;
}
// v[r] += p[r] for four consecutive elements at p (8-byte bf16 / 16-byte fp32 load).
__device__ __forceinline__ void add4(float (&v)[4], const bf16* p) {
  const half_t h = *(const half_t*)p;
  v[0] += __uint_as_float(h[0] << 16);
  v[1] += __uint_as_float(h[0] & 0xffff0000u);
  v[2] += __uint_as_float(h[1] << 16);
  v[3] += __uint_as_float(h[1] & 0xffff0000u);
}
__device__ __forceinline__ void add4(float (&v)[4], const float* p) {
  const f32x4 f = *(const f32x4*)p;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] += f[r];
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

// Sum over the G consecutive lanes G*q .. G*q+G-1 (G = 4, 8 or 16: quad permutes, then the
// half-row mirror for 8, then the row mirror for 16); every lane of the group receives the
// total.
#define TRIMUL_DPP(v, ctrl) \
  __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true))
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
  v += TRIMUL_DPP(v, 0xB1);  // quad_perm [1,0,3,2]
  v += TRIMUL_DPP(v, 0x4E);  // quad_perm [2,3,0,1]
  if (G >= 8) v += TRIMUL_DPP(v, 0x141);  // row_half_mirror
  if (G == 16) v += TRIMUL_DPP(v, 0x140);  // row_mirror
  return v;
}

// Maximum over the 64 lanes of a wave (every lane receives it).
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// The mask extent of batch item bb (the maximum of its TRI_MUL_EXTENT_PARTS = 64 partial
// extents, one per lane), clamped to [0, limit]; `limit` when there are no extents.
// Wave-uniform.
__device__ __forceinline__ int mask_extent(const int* extents, int bb, int limit) {
  if (!extents) return limit;
  int v = wave_max(extents[bb * 64 + (int)(threadIdx.x & 63)]);
  v = __builtin_amdgcn_readfirstlane(v);
  return v < 0 ? 0 : (v > limit ? limit : v);
}

// The bound of batch item bb for a persistent wave that visits items in order: the item's
// mask extent (re-read only when the item changes), or n without extents. Wave-uniform.
struct ExtentCache {
  int bb = -1, ext = 0;
};
__device__ __forceinline__ int item_bound(const int* extents, int bb, int n, ExtentCache& c) {
  if (!extents) return n;
  if (bb != c.bb) {
    c.ext = mask_extent(extents, bb, n);
    c.bb = bb;
  }
  return c.ext;
}

// The tiles inside each item's leading L_b x L_b square (L_b its mask extent), numbered
// item by item, row by row, `tw`-pair column tiles within a row: the work list of a
// persistent wave when padding is skipped, so that every wave gets an equal share of the
// tiles that are left. A wave visits its tiles in increasing order; the cursor keeps the
// item the last lookup landed in. Wave-uniform.
struct ActiveTiles {
  const int* extents;
  int n, batch, tw;
  int cb, cbase, ccount, cntw;  // cursor: item cb's tiles start at index cbase
  __device__ __forceinline__ void load(int b) {
    const int L = mask_extent(extents, b, n);
    cntw = (L + tw - 1) / tw;
    ccount = L * cntw;
  }
  __device__ __forceinline__ void init(const int* e, int n_, int batch_, int tw_) {
    extents = e;
    n = n_;
    batch = batch_;
    tw = tw_;
    cb = 0;
    cbase = 0;
    load(0);
  }
  // the number of tiles over all items
  __device__ __forceinline__ int total() {
    int sum = 0;
    for (int b = 0; b < batch; ++b) {
      const int L = mask_extent(extents, b, n);
      sum += L * ((L + tw - 1) / tw);
    }
    return sum;
  }
  // tile t -> item bb, row r, first column s0 (t below total())
  __device__ __forceinline__ void at(int t, int& bb, int& r, int& s0) {
    if (t < cbase) {
      cb = 0;
      cbase = 0;
      load(0);
    }
    while (t >= cbase + ccount && cb + 1 < batch) {
      cbase += ccount;
      ++cb;
      load(cb);
    }
    const int l = t - cbase;
    r = cntw > 0 ? l / cntw : 0;
    s0 = (l - r * cntw) * tw;
    bb = cb;
  }
};

// Orders this wave's earlier LDS writes before its later LDS reads of other lanes' data
// (LDS operations of one wave are executed in issue order; the fences stop the compiler
// from moving accesses across this point and wait for the writes to complete).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// out = p * m * sigmoid(g) with the gate pre-activation given as g2 = -g * log2(e)
// (the host scales the gate rows by -log2 e): sigmoid(g) = 1 / (1 + 2^g2).
__device__ __forceinline__ float gate_mul(float p_times_m, float g2) {
  return p_times_m * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g2));
}

// acc + lo(a)*lo(b) + hi(a)*hi(b) for two bf16 pairs, fp32 accumulation (the products are
// exact in fp32). Written as an instruction: the compiler's own route to the packed bf16
// dot product has fed every unrolled copy the same source register.
__device__ __forceinline__ float dot2_bf16(unsigned int a, unsigned int b, float acc) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(acc));
  return d;
}

// LayerNorm of one row held by the G consecutive lanes of a pair: lane `part` holds
// chunks part, part+G, ... of the row in v[0..NCH); chunk indices >= nreal are padding
// and must be zero on entry (they add nothing to the sums). Every chunk becomes
// (x - mean) * rstd over the `width` real values, so padding comes out as the finite
// value -mean*rstd, which the zero weight columns of the padding cancel; there is no
// branch on the chunk index. The bf16 version takes sum and sum of squares in one fp32
// pass (packed bf16 dot products); the fp32 version uses two passes.
template <int NCH, int G>
__device__ __forceinline__ void normalize_row_stats(const chunk_t (&v)[NCH], int part, int nreal,
                                                    int width, float& mean, float& rstd, bf16) {
  constexpr unsigned int kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
  float s = 0.f, q = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      s = dot2_bf16(v[i][d], kOnes, s);
      q = dot2_bf16(v[i][d], v[i][d], q);
    }
  (void)part;
  (void)nreal;
  // The sums come out of inline-asm instructions and go straight into DPP reads, which
  // need two wait states after the VALU write of their source; the compiler's hazard
  // check does not see inside the asm, so the wait states are provided here (the asm
  // takes s and q as operands, so the DPP reads cannot be scheduled ahead of it).
  asm volatile("s_nop 1" : "+v"(s), "+v"(q));
  const float inv_w = 1.0f / (float)width;
  mean = group_sum<G>(s) * inv_w;
  const float var = group_sum<G>(q) * inv_w - mean * mean;
  rstd = rsqrtf(fmaxf(var, 0.f) + TRI_MUL_LN_EPS_F);
}
template <int NCH, int G>
__device__ __forceinline__ void normalize_row_stats(const chunk_t (&v)[NCH], int part, int nreal,
                                                    int width, float& mean, float& rstd, float) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += __uint_as_float(v[i][e]);
  const float inv_w = 1.0f / (float)width;
  mean = group_sum<G>(s) * inv_w;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const float keep = part + G * i < nreal ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = (__uint_as_float(v[i][e]) - mean) * keep;
      q = fmaf(d, d, q);
    }
  }
  rstd = rsqrtf(group_sum<G>(q) * inv_w + TRI_MUL_LN_EPS_F);
}

// Value of `v` from lane `src` of the wave (LDS permute network; no LDS storage).
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}
// Sum over the lanes l, l^16, l^32, l^48 (the four lane groups of an MFMA operand row).
__device__ __forceinline__ float row_groups_sum(float v, int lane) {
  v += lane_value(v, lane ^ 16);
  v += lane_value(v, lane ^ 32);
  return v;
}

// LayerNorm of one pair's row held in MFMA operand layout: lane (p, q) = (lane%16,
// lane/16) holds chunk ks of the row at element ks*KG + q*E, for ks < KM; the four lanes
// p, p+16, p+32, p+48 hold the whole row. Chunks at or beyond `width` must be zero on entry
// (they add nothing to the sums); every chunk becomes (x - mean) * rstd, so padding chunks
// come out as the finite value -mean*rstd, which the zero weight columns of the padding
// cancel. No branch on the chunk index: the normalisation stays one straight-line block.
// bf16: one fp32 pass for sum and sum of squares (packed bf16 dot products); fp32: two
// passes, the second one masked to the real chunks.
template <int KM>
__device__ __forceinline__ void normalize_operand_row(chunk_t (&v)[KM], int width, int lane, bf16) {
  constexpr unsigned int kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
  float s = 0.f, q = 0.f;
#pragma unroll
  for (int ks = 0; ks < KM; ++ks)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      s = dot2_bf16(v[ks][d], kOnes, s);
      q = dot2_bf16(v[ks][d], v[ks][d], q);
    }
  const float inv_w = 1.0f / (float)width;
  const float mean = row_groups_sum(s, lane) * inv_w;
  const float var = row_groups_sum(q, lane) * inv_w - mean * mean;
  const float rstd = rsqrtf(fmaxf(var, 0.f) + TRI_MUL_LN_EPS_F);
  const float shift = -mean * rstd;
#pragma unroll
  for (int ks = 0; ks < KM; ++ks) {
    float f[8];
    unpack(v[ks], f, bf16());
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fmaf(f[e], rstd, shift);
    v[ks] = pack(f, bf16());
  }
}
template <int KM>
__device__ __forceinline__ void normalize_operand_row(chunk_t (&v)[KM], int width, int lane, float) {
  const int q0 = (lane >> 4) * 4;
  float s = 0.f;
#pragma unroll
  for (int ks = 0; ks < KM; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += __uint_as_float(v[ks][e]);
  const float inv_w = 1.0f / (float)width;
  const float mean = row_groups_sum(s, lane) * inv_w;
  float q = 0.f;
#pragma unroll
  for (int ks = 0; ks < KM; ++ks) {
    const float keep = ks * 16 + q0 < width ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = (__uint_as_float(v[ks][e]) - mean) * keep;
      q = fmaf(d, d, q);
    }
  }
  const float rstd = rsqrtf(row_groups_sum(q, lane) * inv_w + TRI_MUL_LN_EPS_F);
  const float shift = -mean * rstd;
#pragma unroll
  for (int ks = 0; ks < KM; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[ks][e] = __float_as_uint(fmaf(__uint_as_float(v[ks][e]), rstd, shift));
}

template <class T, int NCH, int G>
__device__ __forceinline__ void normalize_row(chunk_t (&v)[NCH], int part, int nreal, int width) {
  constexpr int E = Traits<T>::E;
  float mean, rstd;
  normalize_row_stats<NCH, G>(v, part, nreal, width, mean, rstd, T());
  const float shift = -mean * rstd;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    float f[E];
    unpack(v[i], f, T());
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = fmaf(f[e], rstd, shift);
    v[i] = pack(f, T());
  }
}

}  // namespace trimul
