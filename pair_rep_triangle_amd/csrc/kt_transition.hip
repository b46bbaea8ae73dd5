// kt: the pair transition as a masked residual, one kernel:
//   out = z + m * (W_2 relu(W_1 LN(z) + b_1) + b_2)
// RFProteína architecture page, "Kernel support": the table's pair-transition row and the
// pair-transition paragraph of "Dispatch and fallback" (both linears, the ReLU, the mask
// and the residual in one launch, the hidden activation kept on chip); and "Inside the
// velocity network" (the pair update ends with a pair transition
// applied as a masked residual). LN gamma/beta are folded into W_1 and b_1 on the host.
//
// The map is pointwise over pairs, so a wave tile is 32 consecutive pairs (two subtiles
// of 16). A workgroup of 8 waves copies W_1, W_2 and the biases into LDS once (each row
// padded by 16 bytes: the row stride is an odd multiple of 16 bytes, so the 16 rows one
// operand read touches land in 16 different bank groups, and every offset inside a k
// group is an immediate), then every wave loops over its own tiles with no workgroup
// barrier:
//   - z arrives straight in MFMA operand layout (lane (p, q) = (lane%16, lane/16) holds
//     chunk ks*4 + q of pair p); the raw chunks are kept for the residual, a copy is
//     normalised in registers;
//   - the hidden width goes in groups of one MFMA k extent (32 bf16 / 16 fp32 values).
//     First GEMM with W_1 rows as the A operand and zhat as B: lane (p, q) ends up with
//     hidden rows 4q..4q+3 of each 16-row unit for pair p. Bias (the accumulator's start)
//     and ReLU applied (after rounding to bf16, as a packed 16-bit integer max: rounding
//     keeps the sign), those values ARE the lane's B-operand chunk of the second GEMM once
//     W_2's columns are stored in the matching order (bf16: slots 8q..8q+3 <- rows 4q..4q+3
//     of the group's first unit, slots 8q+4..8q+7 <- of its second) - no data movement;
//   - second GEMM with W_2 rows as A: W_2's rows (output channels) are stored so that the
//     accumulator registers of lane (p, q) are exactly the channels its z chunks hold.
//     The epilogue z + m * acc is lane-local and leaves as 16-byte chunks.
// Loads and stores are buffer operations on per-subtile resources that end at the last
// pair: the ragged last tile reads zeros and its stores past the end are dropped.

#include "device_common.h"
#include "transition_launch.h"

namespace trimul {

constexpr int KT_WAVES = 8;
constexpr int KT_THREADS = 64 * KT_WAVES;
constexpr int KT_ST = 2;            // 16-pair subtiles per wave tile
constexpr int KT_TW = 16 * KT_ST;   // pairs per wave tile

// The scalar offset stays 0: a 16-byte store still reads its data registers after it
// issues, and the compiler only guards those registers against the next write when the
// store has no scalar offset register. Device-scope stores (sc1): the output is written
// through this XCD's L2 as it is produced, instead of sitting dirty there until the
// end-of-kernel release writes it back (each XCD has its own L2; the next kernel may
// read the output from any of them).
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, chunk_t v, unsigned int voff) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  constexpr int kDeviceScope = 0x10;  // cache policy bit sc1
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)voff, 0,
                                         kDeviceScope);
}

// max(x, 0) on packed storage values: a negative bf16 or fp32 value is a negative 16- or
// 32-bit integer (sign bit set), so a signed integer max with 0 is the ReLU, two bf16
// values per instruction (a float max would also canonicalise its input first). The
// empty asm keeps each packed dword whole, so the conversion before it stays one
// two-value instruction rather than two conversions and a byte permute.
__device__ __forceinline__ chunk_t relu_packed(chunk_t c, bf16) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned int u = c[i];
    asm volatile("" : "+v"(u));
    c[i] = __builtin_bit_cast(unsigned int,
                              __builtin_elementwise_max(__builtin_bit_cast(s16x2, u), (s16x2)0));
  }
  return c;
}
__device__ __forceinline__ chunk_t relu_packed(chunk_t c, float) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 v = __builtin_bit_cast(i32x4, c);
  return __builtin_bit_cast(chunk_t, __builtin_elementwise_max(v, (i32x4)0));
}

template <class T, int KZ>
__global__ __launch_bounds__(KT_THREADS) void pair_transition_kernel(
    const T* __restrict__ z, const T* __restrict__ mask, T* out,
    const chunk_t* __restrict__ image, int image_chunks, int tiles, int last_pairs, int hp,
    int mask_all) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int CZ = KZ * KG;       // pair width
  constexpr int UO = CZ / 16;       // output units of 16 channels
  constexpr int UPG = KG / 16;      // hidden units per k group of the second GEMM
  constexpr int RS1 = CZ + E;       // W_1 row stride in LDS (one chunk of padding)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int rs2 = hp + E;                    // W_2 row stride in LDS
  T* const w1s = (T*)smem;                   // [hp][RS1]
  T* const w2s = w1s + (size_t)hp * RS1;     // [CZ][rs2]
  float* const b1s = (float*)(w2s + (size_t)CZ * rs2);  // [hp]
  float* const b2s = b1s + hp;                           // [CZ]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;

  // tiles: 32-pair tiles in all (the last one holds last_pairs pairs)
  const int gw = blockIdx.x * KT_WAVES + wave;
  const int nw = gridDim.x * KT_WAVES;

  // per-lane byte offsets, the same in every tile: pair p of a subtile, chunk q of the
  // first k group (k groups step in the immediate). Each subtile has a resource of its
  // own: the bounds check covers the lane and immediate offsets, not the scalar one, so a
  // subtile's extent must start at the subtile.
  const unsigned int zoff = (unsigned int)((p * CZ + q * E) * sizeof(T));
  const unsigned int moff = mask_all ? 0u : (unsigned int)(p * sizeof(T));
  // resource of subtile st of tile t over `base` (pair-major, `unit` bytes per pair): it
  // ends at the last pair, so the ragged last tile reads zeros and drops its stores
  auto sub_rsrc = [&](const void* base, int t, int st, unsigned int unit) {
    const unsigned int left = (t < tiles - 1 ? KT_TW : last_pairs) * unit;  // from the tile start
    const unsigned int skip = st * 16 * unit;
    return buffer_rsrc_u32((const unsigned char*)base + (size_t)t * KT_TW * unit + skip,
                           bytes_after(left, skip));
  };

  struct Pre {
    chunk_t zv[KT_ST][KZ];
    T m[KT_ST];
  };
  auto fetch = [&](int t, Pre& f) {
    t = t < tiles ? t : tiles - 1;  // waves past the end refetch the last tile
#pragma unroll
    for (int st = 0; st < KT_ST; ++st) {
      const __amdgpu_buffer_rsrc_t rz = sub_rsrc(z, t, st, CZ * sizeof(T));
      const __amdgpu_buffer_rsrc_t rm =
          mask_all ? buffer_rsrc_u32(mask, sizeof(T)) : sub_rsrc(mask, t, st, sizeof(T));
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks)
        f.zv[st][ks] = load16(rz, zoff + ks * KG * (unsigned int)sizeof(T), 0);
      f.m[st] = load_elem(rm, moff, 0, T());
    }
  };

  chunk_t zr[KT_ST][KZ], za[KT_ST][KZ];
  float mv[KT_ST];
  Pre f;
  auto prepare = [&]() {
#pragma unroll
    for (int st = 0; st < KT_ST; ++st) {
      mv[st] = to_f32(f.m[st]);
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) {
        zr[st][ks] = f.zv[st][ks];
        za[st][ks] = f.zv[st][ks];
      }
      normalize_operand_row<KZ>(za[st], CZ, lane, T());
    }
  };

  // ---- weights and start values -> LDS: the device copy of the weights is the LDS image
  // itself (padded rows, then the biases), so the copy is flat: each thread has up to 16
  // of its 16-byte chunks in flight before it stores any (at c_z = 128, hidden 256: all
  // of them, one round trip), in a few dozen instructions. The first tile's z loads go
  // out after the weight loads: loads retire in order, and the weights are needed first.
  {
    copy_image<KT_THREADS>(image, (chunk_t*)smem, image_chunks, tid, [&]() { fetch(gw, f); });
  }
  __syncthreads();
  prepare();
  const int groups = hp / KG;
  for (int t = gw; t < tiles; t += nw) {
    fetch(t + nw, f);  // the next tile's loads have this whole tile to land
    int opaque;  // keeps the loop-invariant bias reads inside the loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));

    f32x4 acc2[UO][KT_ST];
#pragma unroll
    for (int v = 0; v < UO; ++v) {
      const f32x4 bv = ld16f(b2s + 16 * v + 4 * q + opaque);
#pragma unroll
      for (int st = 0; st < KT_ST; ++st) acc2[v][st] = bv;
    }
    // one k group of the second GEMM: its hidden units from the first GEMM, ReLU, then the
    // group's contribution to every output unit
    auto group = [&](int g) {
      f32x4 h[UPG][KT_ST];
      // this lane's row p of the group's first W_1 unit / chunk q of the group's W_2 columns
      const T* const w1g = w1s + (g * UPG * 16 + p) * RS1 + q * E;
      const T* const w2g = w2s + p * rs2 + (g * 4 + q) * E;
#pragma unroll
      for (int uu = 0; uu < UPG; ++uu) {
        const int u = g * UPG + uu;
        chunk_t wa[KZ];
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) wa[ks] = ld16(w1g + uu * 16 * RS1 + ks * 4 * E);
        const f32x4 bv = ld16f(b1s + 16 * u + 4 * q);
#pragma unroll
        for (int st = 0; st < KT_ST; ++st) {
          h[uu][st] = bv;
#pragma unroll
          for (int ks = 0; ks < KZ; ++ks) h[uu][st] = mma16(h[uu][st], wa[ks], za[st][ks], T());
        }
      }
      chunk_t hb[KT_ST];
#pragma unroll
      for (int st = 0; st < KT_ST; ++st) {
        float hv[8];
#pragma unroll
        for (int uu = 0; uu < UPG; ++uu)
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[4 * uu + r] = h[uu][st][r];
        hb[st] = relu_packed(pack(hv, T()), T());
      }
#pragma unroll
      for (int v = 0; v < UO; ++v) {
        const chunk_t wb = ld16(w2g + v * 16 * rs2);
#pragma unroll
        for (int st = 0; st < KT_ST; ++st) acc2[v][st] = mma16(acc2[v][st], wb, hb[st], T());
      }
    };
#pragma unroll 1
    for (int g = 0; g < groups; ++g) group(g);

    // out = z + m * acc: accumulator register r of output unit v is element
    // e = 4 (v % 2) + r of z chunk v / 2 (bf16), element r of chunk v (fp32)
#pragma unroll
    for (int st = 0; st < KT_ST; ++st) {
      const __amdgpu_buffer_rsrc_t ro = sub_rsrc(out, t, st, CZ * sizeof(T));
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) {
        float zf[8], o[8];
        unpack(zr[st][ks], zf, T());
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int v = ks * (E / 4) + e / 4, r = e % 4;
          o[e] = zf[e] + mv[st] * acc2[v][st][r];
        }
        store16(ro, pack(o, T()), zoff + ks * KG * (unsigned int)sizeof(T));
      }
    }
    prepare();
  }
}

template <class T, int KZ>
static hipError_t launch_kt(const TransitionArgs& a, hipStream_t st) {
  constexpr int E = Traits<T>::E;
  (void)E;
  const size_t lds = transition_lds_bytes(a.cz, a.hp, sizeof(T));
  if (lds != a.image_bytes || lds % 16) return hipErrorInvalidValue;
  auto fn = pair_transition_kernel<T, KZ>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const long long tiles = (a.pairs + KT_TW - 1) / KT_TW;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;  // tile indices are 32-bit
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, KT_THREADS, lds, occ, occ_lds);
  const long long cap = (long long)a.num_cus * (per_cu > 0 ? per_cu : 1);
  const long long need = (tiles + KT_WAVES - 1) / KT_WAVES;
  const int blocks = (int)(need < cap ? need : cap);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(KT_THREADS), lds, st, (const T*)a.z,
                     (const T*)a.mask, (T*)a.out, (const chunk_t*)a.image, (int)(lds / 16),
                     (int)tiles, (int)(a.pairs - (tiles - 1) * KT_TW), a.hp, a.mask_all);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_kt_dispatch(const TransitionArgs& a, hipStream_t st) {
  switch (a.cz / Traits<T>::KG) {
    case 1: return launch_kt<T, 1>(a, st);
    case 2: return launch_kt<T, 2>(a, st);
    case 3: return launch_kt<T, 3>(a, st);
    case 4: return launch_kt<T, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_transition(bool bf16_storage, const TransitionArgs& a, hipStream_t st) {
  if (a.wide) return bf16_storage ? launch_transition_wide(a, st) : hipErrorInvalidValue;
  return bf16_storage ? launch_kt_dispatch<bf16>(a, st) : launch_kt_dispatch<float>(a, st);
}

}  // namespace trimul
