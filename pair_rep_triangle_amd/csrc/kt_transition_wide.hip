// kt (wide): the pair transition out = z + m * (W_2 relu(W_1 LN(z) + b_1) + b_2) for pair
// widths whose two weight matrices do not fit one workgroup's LDS -- the released pair
// width of 384 with an expansion of 2 holds 1.2 MB of bf16 weights.
// RFProteína architecture page, "Kernel support" (the pair-transition row: both linears,
// the ReLU, the mask and the residual in one launch, the hidden activation on chip) and
// "Dispatch and fallback" (the released pair width with an expansion of 2 is the shape the
// fused kernel runs).
//
// At c_z = 384, hidden 768 the map does 1.2 MFLOP per pair against 1.5 kB of HBM traffic:
// it is bound by the matrix cores, not by memory, and the weights are the operand to keep
// moving. A workgroup of 8 waves takes a tile of 128 pairs (16 per wave) and streams the
// weights through LDS one hidden group of 32 units at a time: the group's 32 rows of W_1
// and 32 columns of W_2 (128 c_z bytes, 48 KB at c_z = 384) arrive by direct global-to-LDS
// loads into one of two buffers while the waves compute on the other, so every weight byte
// read from L2 serves all 128 pairs of the tile.
//   - z arrives in MFMA operand layout (lane (p, q) = (lane%16, lane/16) holds chunk
//     ks*4 + q of pair p) and is normalised in registers;
//   - per group: the first GEMM (W_1 rows as A, zhat as B, b_1 as the start value) leaves
//     lane (p, q) with hidden rows 4q..4q+3 of both 16-row units for pair p; ReLU'd and
//     rounded, they are the lane's B chunk of the second GEMM because W_2's columns are
//     stored in that order; the second GEMM adds the group to every output unit;
//   - W_2's rows are stored so that the output accumulators of lane (p, q) are the
//     channels of its own z chunks: z + m * acc is lane-local.
// In LDS, chunk c of W_1 row r sits at position c ^ (r & 15) and chunk q of W_2 row R at
// q ^ ((R >> 2) & 3), which keeps the operand reads free of bank conflicts; the host
// stores the weights in exactly that order, so the copy is linear.

#include "device_common.h"
#include "transition_launch.h"

namespace trimul {

constexpr int KTW_WAVES = 8;
constexpr int KTW_THREADS = 64 * KTW_WAVES;
constexpr int KTW_TP = 16 * KTW_WAVES;  // pairs per workgroup tile

// 16 bytes per lane through a buffer resource straight into LDS (lane i writes
// lds_base + 16 i); counted by vmcnt.
__device__ __forceinline__ void ktw_lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned int voff,
                                              void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, (int)voff, 0, 0, 0);
}

template <int KZ>
__global__ __launch_bounds__(KTW_THREADS) void pair_transition_wide_kernel(
    const bf16* __restrict__ z, const bf16* __restrict__ mask, bf16* out,
    const unsigned char* __restrict__ image, int tiles, long long pairs, int cz, int groups,
    int mask_all) {
  using T = bf16;
  constexpr int E = 8, KG = 32;
  constexpr int CZP = KZ * KG;          // compiled pair width (c_z padded with zeros)
  constexpr int UO = CZP / 16;          // output units of 16 channels
  constexpr int GB = 128 * CZP;         // bytes of one hidden group: W_1 rows | W_2 columns
  constexpr int W1B = 64 * CZP;         // its W_1 part: 32 rows of CZP
  constexpr int BLK = GB / 1024;        // 1 KB direct-load blocks per group
  static_assert(BLK % KTW_WAVES == 0, "whole blocks per wave");
  constexpr int BPW = BLK / KTW_WAVES;  // blocks per wave and group
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* const wbuf = smem;                    // two group buffers [2][GB]
  float* const b1s = (float*)(smem + 2 * GB);          // [groups * 32]
  float* const b2s = b1s + groups * 32;                // [CZP], kernel row order

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;

  // biases -> LDS once (they follow the groups in the image)
  {
    const float* src = (const float*)(image + (size_t)groups * GB);
    for (int k = tid; k < groups * 32 + CZP; k += KTW_THREADS) b1s[k] = src[k];
  }
  // the weight stream: step s copies group s % groups into buffer s % 2
  const __amdgpu_buffer_rsrc_t rimg = buffer_rsrc(image, (size_t)groups * GB);
  auto issue = [&](int s) {
    const int g = s % groups;
    unsigned char* dst = wbuf + (s & 1) * GB;
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int blk = wave * BPW + k;
      ktw_lds_dma16(rimg, (unsigned int)((size_t)g * GB + blk * 1024 + lane * 16), dst + blk * 1024);
    }
  };

  // pairs of this wave in tile t: 16 t_pairs.. ; each lane's z offset is the same in every
  // tile (pair p, chunk q of the first k group); a resource that ends at the last pair
  // makes the ragged last tile read zeros and drop its stores
  const unsigned int zoff = (unsigned int)((p * cz + q * E) * sizeof(T));
  const unsigned int moff = mask_all ? 0u : (unsigned int)(p * sizeof(T));
  auto sub_rsrc = [&](const void* base, int t, unsigned int unit) {
    const long long first = (long long)t * KTW_TP + wave * 16;
    const long long left = pairs - first;
    const unsigned int n16 = (unsigned int)(left < 0 ? 0 : (left > 16 ? 16 : left));
    return buffer_rsrc_u32((const unsigned char*)base + first * unit, n16 * unit);
  };
  // a tile's z goes into za (raw; normalised in place when its tile starts), the next
  // tile's loads right after the last use of za in the current one
  chunk_t za[KZ];
  T min_;
  auto fetch = [&](int t) {
    const __amdgpu_buffer_rsrc_t rz = sub_rsrc(z, t, cz * sizeof(T));
    const __amdgpu_buffer_rsrc_t rm =
        mask_all ? buffer_rsrc_u32(mask, sizeof(T)) : sub_rsrc(mask, t, sizeof(T));
#pragma unroll
    for (int ks = 0; ks < KZ; ++ks)
      za[ks] = ks * KG + q * E < cz ? load16(rz, zoff + ks * KG * (unsigned int)sizeof(T), 0)
                                    : chunk_t{0u, 0u, 0u, 0u};
    min_ = load_elem(rm, moff, 0, T());
  };

  const int gb = blockIdx.x, nb = gridDim.x;
  int s = 0;  // weight-stream step
  issue(0);
  if (gb < tiles) fetch(gb);
  for (int t = gb; t < tiles; t += nb) {
    // this tile's pairs, normalised; the raw z is read again for the residual at the end
    const float mv = to_f32(min_);
    normalize_operand_row<KZ>(za, cz, lane, T());

    f32x4 acc[UO];
    int opaque;  // keeps the loop-invariant LDS reads inside the loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
#pragma unroll
    for (int v = 0; v < UO; ++v) acc[v] = ld16f(b2s + 16 * v + 4 * q + opaque);

#pragma unroll 1
    for (int g = 0; g < groups; ++g, ++s) {
      // step s's group is in LDS once this thread's loads are done and every wave is past
      // the barrier; every wave is then also done with buffer (s + 1) % 2, which the next
      // step's loads overwrite
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(s + 1);  // the next group (the first again after the last: the next tile's)
      const unsigned char* gbuf = wbuf + (s & 1) * GB;
      const T* const w1 = (const T*)gbuf;               // [32][RC chunks], swizzled
      const T* const w2 = (const T*)(gbuf + W1B);       // [CZP][4 chunks], swizzled
      // first GEMM: hidden units u = 0, 1 of the group (rows 16u + p)
      f32x4 h[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float* bb = b1s + g * 32 + 16 * u + 4 * q;
        h[u] = ld16f(bb);
        const int row = 16 * u + p;
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) {
          const chunk_t wa = ld16(w1 + row * CZP + (((ks * 4 + q) ^ p) * E));
          h[u] = mma16(h[u], wa, za[ks], T());
        }
      }
      if (g == groups - 1 && t + nb < tiles) fetch(t + nb);  // za is free: next tile's z
      // ReLU on the rounded values: rows 4q..4q+3 of unit 0, then of unit 1, are k slots
      // 8q..8q+7 of the second GEMM
      float hv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hv[r] = fmaxf(h[0][r], 0.f);
        hv[4 + r] = fmaxf(h[1][r], 0.f);
      }
      const chunk_t hb = pack(hv, T());
      // second GEMM: every output unit v (rows 16v + p)
#pragma unroll
      for (int v = 0; v < UO; ++v) {
        const int row = 16 * v + p;
        const chunk_t wb = ld16(w2 + row * 32 + ((q ^ ((row >> 2) & 3)) * E));
        acc[v] = mma16(acc[v], wb, hb, T());
      }
    }

    // out = z + m * acc: accumulator register r of output unit v is element 4 (v % 2) + r
    // of the lane's z chunk v / 2
    const __amdgpu_buffer_rsrc_t rz = sub_rsrc(z, t, cz * sizeof(T));
    const __amdgpu_buffer_rsrc_t ro = sub_rsrc(out, t, cz * sizeof(T));
#pragma unroll
    for (int ks = 0; ks < KZ; ++ks) {
      if (ks * KG + q * E >= cz) continue;  // padded channels (compile-time KZ, runtime cz)
      const unsigned int off = zoff + ks * KG * (unsigned int)sizeof(T);
      float zf[8], o[8];
      unpack(load16(rz, off, 0), zf, T());
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = zf[e] + mv * acc[2 * ks + e / 4][e % 4];
      typedef __attribute__((ext_vector_type(4))) int i32x4;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, pack(o, T())), ro,
                                             (int)off, 0, 0);
    }
  }
  // the stream's last step issued one group more than was used: let it land before exit
  __builtin_amdgcn_s_waitcnt(0x0070);
}

size_t transition_wide_lds_bytes(int czp, int hp) {
  return (size_t)2 * 128 * czp + ((size_t)hp + czp) * 4;
}

template <int KZ>
static hipError_t launch_ktw(const TransitionArgs& a, hipStream_t st) {
  const int czp = KZ * 32;
  const size_t lds = transition_wide_lds_bytes(czp, a.hp);
  auto fn = pair_transition_wide_kernel<KZ>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const long long tiles = (a.pairs + KTW_TP - 1) / KTW_TP;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long need = tiles < a.num_cus ? tiles : a.num_cus;  // one workgroup per CU
  hipLaunchKernelGGL(fn, dim3((unsigned)need), dim3(KTW_THREADS), lds, st, (const bf16*)a.z,
                     (const bf16*)a.mask, (bf16*)a.out, (const unsigned char*)a.image,
                     (int)tiles, a.pairs, a.cz, a.hp / 32, a.mask_all);
  return hipGetLastError();
}

hipError_t launch_transition_wide(const TransitionArgs& a, hipStream_t st) {
  switch (a.czp / 32) {
    case 4: return launch_ktw<4>(a, st);
    case 8: return launch_ktw<8>(a, st);
    case 12: return launch_ktw<12>(a, st);
    case 16: return launch_ktw<16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace trimul
