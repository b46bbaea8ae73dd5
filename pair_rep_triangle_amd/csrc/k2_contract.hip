// k2: the contraction over the third residue, one NT GEMM per (batch, channel):
//   x[bc][i][j] = sum_k A[bc][i][k] * B[bc][j][k]
// RFProteína architecture page, "Triangle multiplication on SM90": K2 performs the
// contraction itself, compiled per direction. Here the direction is absorbed by the
// input-gate kernel's store layout (it writes the incoming operands transposed), so one
// kernel serves both.

#include "device_common.h"

namespace trimul {

// Workgroup tile 256 (i) x 128 (j), 4 waves as 2 x 2, each 128 x 64 (4 x 2 MFMA 32x32
// tiles, 128 fp32 accumulators per lane). k advances 64 bytes per row and stage; stages
// move from global memory straight into LDS (global_load_lds, no registers on the way)
// through a ring of three LDS buffers, so two stages are in flight while one is used.
// Inside a buffer a row is four 16-byte chunks; chunk c of row r sits at position
// c ^ ((r ^ (r >> 2)) & 3), which keeps the MFMA operand reads free of bank conflicts
// (checked for both 32- and 64-bank LDS). The output tile is staged in LDS and leaves as
// 16-byte row-contiguous stores.
// Flat grid of (np/256) * (np/128) * batch*c workgroups, remapped so that consecutive
// tiles of one channel land on the same XCD (workgroup ids are dealt round-robin over the
// 8 XCDs) and share its L2.
constexpr int K2_BM = 256, K2_BN = 128;
constexpr int K2_THREADS = 256;
constexpr int K2_STAGES = 3;
constexpr int K2_KC = 4;                                   // 16-byte chunks per row and stage
constexpr int K2_A_BYTES = K2_BM * K2_KC * 16;             // 16 KB
constexpr int K2_B_BYTES = K2_BN * K2_KC * 16;             // 8 KB
constexpr int K2_STAGE_BYTES = K2_A_BYTES + K2_B_BYTES;    // 24 KB
static_assert(N_PAD % K2_BM == 0 && N_PAD % K2_BN == 0, "padded side covers whole tiles");

__device__ __forceinline__ int k2_swizzle(int r) { return (r ^ (r >> 2)) & 3; }

template <class T>
__global__ __launch_bounds__(K2_THREADS, 2) void k2_contract(const T* __restrict__ A,
                                                             const T* __restrict__ B,
                                                             T* __restrict__ X, int np) {
  constexpr int E = Traits<T>::E;
  constexpr int KT = K2_KC * E;  // k per stage
  __shared__ __attribute__((aligned(16))) unsigned char lds[K2_STAGES * K2_STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int bid = blockIdx.x, total = gridDim.x;
  const int per = total >> 3;
  const int logical = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
  const int tn = np / K2_BN;
  const int tiles = (np / K2_BM) * tn;
  const int bc = logical / tiles, tile = logical - bc * tiles;
  const int ti = tile / tn, tj = tile - ti * tn;

  const size_t mat = (size_t)np * np;
  const T* Ab = A + bc * mat + (size_t)ti * K2_BM * np;
  const T* Bb = B + bc * mat + (size_t)tj * K2_BN * np;

  // this lane's slot in a 1 KB direct-load block: row lane/4 of the block's 16, position
  // lane%4, which holds chunk (position ^ swizzle(row)) of the row
  const int brow = lane >> 2;
  auto issue = [&](int s) {
    unsigned char* base = lds + (s % K2_STAGES) * K2_STAGE_BYTES;
    const int k0 = s * KT;
#pragma unroll
    for (int q = 0; q < K2_BM / 16 / 4; ++q) {  // A: 16 blocks of 16 rows, 4 per wave
      const int blk = wave + 4 * q, row = blk * 16 + brow;
      const int c = (lane & 3) ^ k2_swizzle(row);
      lds_dma16(Ab + (size_t)row * np + k0 + c * E, base + blk * 1024);
    }
#pragma unroll
    for (int q = 0; q < K2_BN / 16 / 4; ++q) {  // B: 8 blocks, 2 per wave
      const int blk = wave + 4 * q, row = blk * 16 + brow;
      const int c = (lane & 3) ^ k2_swizzle(row);
      lds_dma16(Bb + (size_t)row * np + k0 + c * E, base + K2_A_BYTES + blk * 1024);
    }
  };
  constexpr int LOADS_PER_STAGE = K2_BM / 16 / 4 + K2_BN / 16 / 4;  // per thread

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operand rows of this lane: i rows wm*128 + mt*32 + lane%32, j rows wn*64 + nt*32 +
  // lane%32; all have the same swizzle (the row bases are multiples of 32)
  const int sw = k2_swizzle(lane & 31);
  auto compute = [&](int s) {
    const unsigned char* cur = lds + (s % K2_STAGES) * K2_STAGE_BYTES;
#pragma unroll
    for (int step = 0; step < K2_KC / 2; ++step) {
      const int pos = ((2 * step + (lane >> 5)) ^ sw) * 16;
      chunk_t fa[4], fb[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        fa[mt] = ld16(cur + (wm * 128 + mt * 32 + (lane & 31)) * 64 + pos);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        fb[nt] = ld16(cur + K2_A_BYTES + (wn * 64 + nt * 32 + (lane & 31)) * 64 + pos);
      // operands swapped: the MFMA produces D[j][i] = x[i][j], so each lane ends up
      // with runs of 4 consecutive j of one row i.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32(acc[mt][nt], fb[nt], fa[mt], T());
    }
  };

  const int nst = np / KT;  // at least 2: np is a multiple of 256
  issue(0);
  issue(1);
  for (int s = 0; s < nst; ++s) {
    // this thread's loads of stage s are done once at most the next stage's remain
    if (s + 1 < nst)
      __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_STAGE);  // vmcnt(LOADS_PER_STAGE)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // every wave's part of stage s is in LDS, and every wave is done with stage s-1,
    // whose buffer the loads of stage s+2 overwrite (its LDS reads all fed MFMAs, so
    // they have completed). A bare s_barrier: __syncthreads() would also wait for the
    // stage s+1 loads still in flight. The empty asm statements keep the compiler from
    // moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 2 < nst) issue(s + 2);
    compute(s);
  }
  __syncthreads();  // all waves are done reading the ring before it holds the output

  T* Xb = X + bc * mat + (size_t)ti * K2_BM * np + tj * K2_BN;
  if constexpr (sizeof(T) == 2) {
    // stage the 256 x 128 tile as [i][j] rows, then 16-byte row-contiguous stores
    constexpr int XROW = K2_BN + E;
    static_assert(K2_BM * XROW * sizeof(T) <= K2_STAGES * K2_STAGE_BYTES, "output staging fits");
    T* xs = (T*)lds;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = wm * 128 + mt * 32 + (lane & 31);
          const int j = wn * 64 + nt * 32 + 8 * q + 4 * (lane >> 5);
          store4(xs + i * XROW + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
                 acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
        }
    __syncthreads();
    constexpr int CPR = K2_BN / E;
#pragma unroll 4
    for (int idx = tid; idx < K2_BM * CPR; idx += K2_THREADS) {
      const int row = idx / CPR, cc = idx - row * CPR;
      st16(Xb + (size_t)row * np + cc * E, ld16(xs + row * XROW + cc * E));
    }
  } else {
    // fp32: four consecutive j per lane are one 16-byte store
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = wm * 128 + mt * 32 + (lane & 31);
          const int j = wn * 64 + nt * 32 + 8 * q + 4 * (lane >> 5);
          store4(Xb + (size_t)i * np + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
                 acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
        }
  }
}

size_t k2_grid(int np, int batch, int c) {
  return (size_t)(np / K2_BM) * (np / K2_BN) * batch * c;
}

hipError_t launch_k2(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  dim3 grid((unsigned)k2_grid(a.np, a.batch, a.c));
  if (bf16_storage)
    hipLaunchKernelGGL(k2_contract<bf16>, grid, dim3(K2_THREADS), 0, st, (const bf16*)a.a,
                       (const bf16*)a.b, (bf16*)a.x, a.np);
  else
    hipLaunchKernelGGL(k2_contract<float>, grid, dim3(K2_THREADS), 0, st, (const float*)a.a,
                       (const float*)a.b, (float*)a.x, a.np);
  return hipGetLastError();
}

}  // namespace trimul
