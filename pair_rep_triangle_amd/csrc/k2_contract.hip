// k2: the contraction over the third residue, one NT GEMM per (batch, channel):
//   x[bc][i][j] = sum_k A[bc][i][k] * B[bc][j][k]
// RFProteína architecture page, "Triangle multiplication on SM90": K2 performs the
// contraction itself, compiled per direction. Here the direction is absorbed by the
// input-gate kernel's store layout (it writes the incoming operands transposed), so one
// kernel serves both.

#include "device_common.h"

namespace trimul {

// A 16-byte store through a buffer resource with device scope (cache policy sc1): the line
// is written through this XCD's L2 as it is produced, rather than left dirty there for the
// end-of-kernel release to write back (each XCD has its own L2, and the next kernel may read
// X from any of them). The scalar offset stays 0: a 16-byte store still reads its data
// registers after it issues, and the compiler only guards those registers against the next
// write when the store has no scalar offset register.
__device__ __forceinline__ void store16_sc1(__amdgpu_buffer_rsrc_t r, chunk_t v, unsigned int voff) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)voff, 0, 0x10);
}

// Workgroup tile 256 (i) x 128 (j), 4 waves as 2 x 2, each 128 x 64 (4 x 2 MFMA 32x32
// tiles, 128 fp32 accumulators per lane). k advances 64 bytes per row and stage; stages
// move from global memory straight into LDS (buffer loads with the LDS bit, no registers
// on the way) through a ring of three LDS buffers, so two stages are in flight while one
// is used. A lane's byte offset inside the tile's rows is the same for every stage (the
// stage is the scalar offset), so no address register is rewritten while a load that
// reads it may still be waiting to issue. The six loads that fetch stage s + 2 are spread
// between the sixteen MFMAs of stage s: a load waits for the CU's memory path to accept
// it, and the MFMAs already issued keep the matrix unit busy meanwhile.
// Inside a buffer a row is four 16-byte chunks; chunk c of row r sits at position
// c ^ ((r ^ (r >> 2)) & 3), which keeps the MFMA operand reads free of bank conflicts
// (checked for both 32- and 64-bank LDS). The output tile is staged in LDS and leaves as
// 16-byte row-contiguous stores.
// Flat grid of ceil(np/256) * ceil(np/128) * batch*c workgroups, remapped so that the
// tiles of one channel land on the same XCD and share its L2.
constexpr int K2_BM = 256, K2_BN = 128;
constexpr int K2_THREADS = 256;
constexpr int K2_STAGES = 3;
constexpr int K2_KC = 4;                                   // 16-byte chunks per row and stage
constexpr int K2_A_BYTES = K2_BM * K2_KC * 16;             // 16 KB
constexpr int K2_B_BYTES = K2_BN * K2_KC * 16;             // 8 KB
constexpr int K2_STAGE_BYTES = K2_A_BYTES + K2_B_BYTES;    // 24 KB
constexpr int K2_LOADS_A = K2_BM / 16 / 4;                 // per thread and stage: 4
constexpr int K2_LOADS = K2_LOADS_A + K2_BN / 16 / 4;      // 6
static_assert(N_PAD % 64 == 0, "operand rows of whole 128-byte lines; 64-pair input tiles");

__device__ __forceinline__ int k2_swizzle(int r) { return (r ^ (r >> 2)) & 3; }

// 16 bytes per lane through a buffer resource straight into LDS: lane i writes
// lds_base + 16 i (lds_base wave-uniform); completion is counted by vmcnt.
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, unsigned int voff,
                                              int soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, (int)voff, soff, 0, 0);
}

// Scheduling groups for the instructions of one basic block: NL times (the next share of
// MF MFMAs, then one memory load), spreading NL loads evenly over MF MFMAs.
template <int MF, int NL, int Q = 0>
__device__ __forceinline__ void mfma_load_groups() {
  if constexpr (Q < NL) {
    __builtin_amdgcn_sched_group_barrier(0x008, (MF * (Q + 1)) / NL - (MF * Q) / NL, 0);
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    mfma_load_groups<MF, NL, Q + 1>();
  }
}

// The operands are zero past row and column n (and, with mask extents from k0, past each
// item's extent L_b, inside which every nonzero pair lies): the k loop stops at that bound
// rounded up to a stage, the operand rows past it are not read (the buffer resources end
// there, so their loads return zeros), and a tile that lies wholly past it runs no stage
// and stores zeros. The padded side np is a multiple of 64, not of the tile: the last tile
// row and column may be partial, and their stores past np are dropped.
template <class T>
__global__ __launch_bounds__(K2_THREADS, 2) void k2_contract(const T* __restrict__ A,
                                                             const T* __restrict__ B,
                                                             T* __restrict__ X, int n, int np,
                                                             const int* __restrict__ extents,
                                                             int c) {
  constexpr int E = Traits<T>::E;
  constexpr int KT = K2_KC * E;  // k per stage
  // MFMA instructions per wave and stage (the fp32 form takes four per 16-byte chunk)
  constexpr int MFMAS = 16 * (sizeof(T) == 4 ? 4 : 1);
  __shared__ __attribute__((aligned(16))) unsigned char lds[K2_STAGES * K2_STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Workgroup ids are dealt round-robin over the 8 XCDs: XCD x runs ids x, x + 8, ...
  // Its k-th workgroup takes tile k % tiles of channel plane 8 (k / tiles) + x, so the tiles
  // of one plane stay on one XCD (sharing its L2) and every XCD holds planes of every batch
  // item (B * c is a multiple of 16), which keeps the XCDs evenly loaded when items differ
  // in extent.
  const int bid = blockIdx.x;
  const int tn = (np + K2_BN - 1) / K2_BN;
  const int tiles = ((np + K2_BM - 1) / K2_BM) * tn;
  const int xcd = bid & 7, k = bid >> 3;
  const int bc = (k / tiles) * 8 + xcd, tile = k - (k / tiles) * tiles;
  const int ti = tile / tn, tj = tile - ti * tn;

  // the bound past which both operands are zero: the item's extent, else n
  const int ext = extents ? mask_extent(extents, bc / c, n) : n;
  const size_t mat = (size_t)np * np;
  const T* Ab = A + bc * mat + (size_t)ti * K2_BM * np;
  const T* Bb = B + bc * mat + (size_t)tj * K2_BN * np;
  // the tile's rows of A and B that lie inside the bound (at most 256 rows of 32768
  // elements: within 32 bits); loads of the rows past them return zeros
  const int rows_a = min(max(ext - ti * K2_BM, 0), K2_BM);
  const int rows_b = min(max(ext - tj * K2_BN, 0), K2_BN);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc_u32(Ab, (unsigned int)(rows_a * np * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc_u32(Bb, (unsigned int)(rows_b * np * sizeof(T)));

  // this lane's slot in a 1 KB direct-load block: row lane/4 of the block's 16, position
  // lane%4, which holds chunk (position ^ swizzle(row)) of the row. Block q of this wave
  // is block wave + 4q of the stage (A: 16 blocks, B: 8).
  const int brow = lane >> 2;
  unsigned int voff[K2_LOADS];
#pragma unroll
  for (int q = 0; q < K2_LOADS; ++q) {
    const int blk = wave + 4 * (q < K2_LOADS_A ? q : q - K2_LOADS_A), row = blk * 16 + brow;
    const int c = (lane & 3) ^ k2_swizzle(row);
    voff[q] = (unsigned int)(((size_t)row * np + c * E) * sizeof(T));
  }
  auto issue_one = [&](int s, int q) {
    unsigned char* base = lds + (s % K2_STAGES) * K2_STAGE_BYTES;
    const int soff = s * KT * (int)sizeof(T);
    if (q < K2_LOADS_A)
      lds_dma16_buf(ra, voff[q], soff, base + (wave + 4 * q) * 1024);
    else
      lds_dma16_buf(rb, voff[q], soff, base + K2_A_BYTES + (wave + 4 * (q - K2_LOADS_A)) * 1024);
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int q = 0; q < K2_LOADS; ++q) issue_one(s, q);
  };

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
  // One stage: all operand reads first, then the MFMAs; with `next` >= 0 the loads of
  // stage `next` are placed between the MFMAs (sched_group_barrier: 2 or 3 MFMAs, one
  // load, six times).
  auto compute = [&](int s, int next) {
    const unsigned char* cur = lds + (s % K2_STAGES) * K2_STAGE_BYTES;
    chunk_t fa[2][4], fb[2][2];
#pragma unroll
    for (int step = 0; step < K2_KC / 2; ++step) {
      const int pos = ((2 * step + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        fa[step][mt] = ld16(cur + (wm * 128 + mt * 32 + (lane & 31)) * 64 + pos);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        fb[step][nt] = ld16(cur + K2_A_BYTES + (wn * 64 + nt * 32 + (lane & 31)) * 64 + pos);
    }
#pragma unroll
    for (int step = 0; step < K2_KC / 2; ++step)
      // operands swapped: the MFMA produces D[j][i] = x[i][j], so each lane ends up with
      // runs of 4 consecutive j of one row i.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = mma32(acc[mt][nt], fb[step][nt], fa[step][mt], T());
    if (next >= 0) {
      issue(next);
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // the operand reads
      mfma_load_groups<MFMAS, K2_LOADS>();
    }
  };
  // stage s's loads are done once at most the next stage's remain; every wave's part of
  // stage s is then in LDS after the barrier, and every wave is done with stage s-1, whose
  // buffer the loads of stage s+2 overwrite. A bare s_barrier: __syncthreads() would also
  // wait for the stage s+1 loads still in flight. The empty asm statements keep the
  // compiler from moving LDS accesses across it.
  // The wait also covers this wave's LDS reads (lgkmcnt(0)), so none of stage s-1 is still
  // pending when another wave's loads start to overwrite its buffer.
  auto arrive = [&](bool last) {
    if (!last)
      __builtin_amdgcn_s_waitcnt(0x0070 | K2_LOADS);  // vmcnt(K2_LOADS) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // stages of the k loop: up to the bound rounded up to a stage (np is a multiple of the
  // stage), none when the tile lies past the bound
  const int nst = (rows_a == 0 || rows_b == 0) ? 0 : (ext + KT - 1) / KT;
  if (nst >= 2) {
    issue(0);
    issue(1);
#pragma unroll 1
    for (int s = 0; s + 2 < nst; ++s) {
      arrive(false);
      compute(s, s + 2);
    }
    arrive(false);
    compute(nst - 2, -1);
    arrive(true);
    compute(nst - 1, -1);
  } else if (nst == 1) {
    issue(0);
    arrive(true);
    compute(0, -1);
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
    // the tile's part inside the padded plane (a partial last tile row or column)
    const int vrows = min(np - ti * K2_BM, K2_BM), vchunks = min(np - tj * K2_BN, K2_BN) / E;
    // whole rows with device-scope stores (byte offsets stay below 2^25)
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc_u32(Xb, 0xffffffffu);
#pragma unroll 4
    for (int idx = tid; idx < K2_BM * CPR; idx += K2_THREADS) {
      const int row = idx / CPR, cc = idx - row * CPR;
      if (row < vrows && cc < vchunks)
        store16_sc1(rx, ld16(xs + row * XROW + cc * E),
                    (unsigned int)((row * np + cc * E) * (int)sizeof(T)));
    }
  } else {
    // fp32: four consecutive j per lane are one 16-byte store (inside the padded plane)
    const int vrows = min(np - ti * K2_BM, K2_BM), vcols = min(np - tj * K2_BN, K2_BN);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = wm * 128 + mt * 32 + (lane & 31);
          const int j = wn * 64 + nt * 32 + 8 * q + 4 * (lane >> 5);
          if (i < vrows && j < vcols)
            store4(Xb + (size_t)i * np + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
                   acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
        }
  }
}

size_t k2_grid(int np, int batch, int c) {
  return (size_t)((np + K2_BM - 1) / K2_BM) * ((np + K2_BN - 1) / K2_BN) * batch * c;
}

hipError_t launch_k2(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  dim3 grid((unsigned)k2_grid(a.np, a.batch, a.c));
  if (bf16_storage)
    hipLaunchKernelGGL(k2_contract<bf16>, grid, dim3(K2_THREADS), 0, st, (const bf16*)a.a,
                       (const bf16*)a.b, (bf16*)a.x, a.n, a.np, a.extents, a.c);
  else
    hipLaunchKernelGGL(k2_contract<float>, grid, dim3(K2_THREADS), 0, st, (const float*)a.a,
                       (const float*)a.b, (float*)a.x, a.n, a.np, a.extents, a.c);
  return hipGetLastError();
}

}  // namespace trimul
