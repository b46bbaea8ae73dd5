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

// Workgroup tile 256 (i) x BN (j) with BN = 64 * WN: 2 x WN waves, each 128 x 64 (4 x 2 MFMA
// 32x32 tiles, 128 fp32 accumulators per lane). Two forms: WN = 2 (256 x 128, 4 waves, two
// workgroups per CU) and WN = 4 (256 x 256, 8 waves, one workgroup per CU), which moves
// a third fewer bytes from L2 into LDS per MFMA (32 KB per stage for 16 MFMAs per wave
// against 24 KB for 16 per wave with half the waves). k advances 64 bytes per row and
// stage; stages move from global memory straight into LDS (buffer loads with the LDS bit,
// no registers on the way) through a ring of three LDS buffers, so two stages are in
// flight while one is used. A lane's byte offset inside the tile's rows is the same for
// every stage (the stage is the scalar offset), so no address register is rewritten while
// a load that reads it may still be waiting to issue. The loads that fetch stage s + 2 are
// spread between the sixteen MFMAs of stage s: a load waits for the CU's memory path to
// accept it, and the MFMAs already issued keep the matrix unit busy meanwhile.
// Inside a buffer a row is four 16-byte chunks; chunk c of row r sits at position
// c ^ ((r ^ (r >> 2)) & 3), which keeps the MFMA operand reads free of bank conflicts
// (checked for both 32- and 64-bank LDS). The output tile is staged in LDS (128 rows at a
// time in the wide form) and leaves as 16-byte row-contiguous stores.
// Flat grid of ceil(np/256) * ceil(np/BN) * batch*c workgroups, remapped so that the
// tiles of one channel land on the same XCD and share its L2.
constexpr int K2_BM = 256;
constexpr int K2_KC = 4;                                   // 16-byte chunks per row and stage
constexpr int K2_A_BYTES = K2_BM * K2_KC * 16;             // 16 KB
static_assert(N_PAD % 64 == 0, "operand rows of whole 128-byte lines; 64-pair input tiles");

template <int WN, int NTW, int ST>
struct K2Shape {
  static constexpr int STAGES = ST;                        // LDS ring buffers
  static constexpr int WCOLS = 32 * NTW;                   // tile columns per wave
  static constexpr int BN = WCOLS * WN;
  static constexpr int WAVES = 2 * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int B_BYTES = BN * K2_KC * 16;
  static constexpr int STAGE_BYTES = K2_A_BYTES + B_BYTES;
  static constexpr int LOADS_A = K2_BM / 16 / WAVES;       // 1 KB blocks per wave and stage
  static constexpr int LOADS = LOADS_A + BN / 16 / WAVES;
  static constexpr int OUT_ROWS = BN == 128 ? K2_BM : 128; // output rows staged at a time
  static constexpr int RING_BYTES = ST * STAGE_BYTES;
  static constexpr int OUT_BYTES = OUT_ROWS * (BN + 8) * 2;
  static constexpr int LDS_BYTES = RING_BYTES > OUT_BYTES ? RING_BYTES : OUT_BYTES;
  static constexpr int MIN_BLOCKS = 2 * LDS_BYTES <= 160 * 1024 ? 2 : 1;  // per CU
};

// A buffer resource whose words are taken from the first lane. The operand bases and
// bounds are wave-uniform, but built with make_buffer_rsrc directly the compiler holds the
// descriptor in vector registers here and wraps every direct-to-LDS load (which needs it in
// scalar registers) in a loop over the distinct descriptors of the wave: one pass at run
// time, but each load then sits in a basic block of its own, away from the MFMAs it is
// meant to overlap.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void* base, unsigned int bytes) {
  const unsigned long long p = (unsigned long long)base;
  const unsigned int lo = __builtin_amdgcn_readfirstlane((unsigned int)p);
  const unsigned int hi = __builtin_amdgcn_readfirstlane((unsigned int)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

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
// Both forms keep two waves per SIMD (256 registers per lane).
template <class T, int WN, int NTW, int ST>
__global__ __launch_bounds__((K2Shape<WN, NTW, ST>::THREADS), (K2Shape<WN, NTW, ST>::MIN_BLOCKS))
void k2_contract(
    const T* __restrict__ A, const T* __restrict__ B, T* __restrict__ X, int n, int np,
    const int* __restrict__ extents, int c) {
  using S = K2Shape<WN, NTW, ST>;
  constexpr int BN = S::BN, NW = S::WAVES, NT = S::THREADS;
  constexpr int LOADS = S::LOADS, LOADS_A = S::LOADS_A;
  constexpr int E = Traits<T>::E;
  constexpr int KT = K2_KC * E;  // k per stage
  // MFMA instructions per wave and stage (the fp32 form takes four per 16-byte chunk)
  constexpr int MFMAS = 8 * NTW * (sizeof(T) == 4 ? 4 : 1);
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // Workgroup ids are dealt round-robin over the 8 XCDs: XCD x runs ids x, x + 8, ...
  // Its k-th workgroup takes tile k % tiles of channel plane 8 (k / tiles) + x, so the tiles
  // of one plane stay on one XCD (sharing its L2) and every XCD holds planes of every batch
  // item (B * c is a multiple of 16), which keeps the XCDs evenly loaded when items differ
  // in extent.
  const int bid = blockIdx.x;
  const int tn = (np + BN - 1) / BN;
  const int tiles = ((np + K2_BM - 1) / K2_BM) * tn;
  const int xcd = bid & 7, k = bid >> 3;
  const int bc = (k / tiles) * 8 + xcd, tile = k - (k / tiles) * tiles;
  const int ti = tile / tn, tj = tile - ti * tn;

  // the bound past which both operands are zero: the item's extent, else n
  const int ext = extents ? mask_extent(extents, bc / c, n) : n;
  const size_t mat = (size_t)np * np;
  const T* Ab = A + bc * mat + (size_t)ti * K2_BM * np;
  const T* Bb = B + bc * mat + (size_t)tj * BN * np;
  // the tile's rows of A and B that lie inside the bound (at most 256 rows of 32768
  // elements: within 32 bits); loads of the rows past them return zeros
  const int rows_a = min(max(ext - ti * K2_BM, 0), K2_BM);
  const int rows_b = min(max(ext - tj * BN, 0), BN);
  const __amdgpu_buffer_rsrc_t ra = rsrc_uniform(Ab, (unsigned int)(rows_a * np * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rb = rsrc_uniform(Bb, (unsigned int)(rows_b * np * sizeof(T)));

  // this lane's slot in a 1 KB direct-load block: row lane/4 of the block's 16, position
  // lane%4, which holds chunk (position ^ swizzle(row)) of the row. Block q of this wave
  // is block wave + NW q of the stage (A: 16 blocks, B: BN / 16).
  const int brow = lane >> 2;
  unsigned int voff[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int blk = wave + NW * (q < LOADS_A ? q : q - LOADS_A), row = blk * 16 + brow;
    const int c = (lane & 3) ^ k2_swizzle(row);
    voff[q] = (unsigned int)(((size_t)row * np + c * E) * sizeof(T));
  }
  auto issue_one = [&](int s, int q) {
    unsigned char* base = lds + (s % ST) * S::STAGE_BYTES;
    const int soff = s * KT * (int)sizeof(T);
    if (q < LOADS_A)
      lds_dma16_buf(ra, voff[q], soff, base + (wave + NW * q) * 1024);
    else
      lds_dma16_buf(rb, voff[q], soff, base + K2_A_BYTES + (wave + NW * (q - LOADS_A)) * 1024);
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) issue_one(s, q);
  };

  f32x16 acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operand rows of this lane: i rows wm*128 + mt*32 + lane%32, j rows wn*64 + nt*32 +
  // lane%32; all have the same swizzle (the row bases are multiples of 32)
  const int sw = k2_swizzle(lane & 31);
  // One stage: all operand reads first, then the MFMAs; with `next` >= 0 the loads of
  // stage `next` are placed between the MFMAs (sched_group_barrier: 2 or 3 MFMAs, one
  // load, six times).
  auto compute = [&](int s, int next, int next2 = -1) {
    const unsigned char* cur = lds + (s % ST) * S::STAGE_BYTES;
    chunk_t fa[2][4], fb[2][NTW];
#pragma unroll
    for (int step = 0; step < K2_KC / 2; ++step) {
      const int pos = ((2 * step + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        fa[step][mt] = ld16(cur + (wm * 128 + mt * 32 + (lane & 31)) * 64 + pos);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        fb[step][nt] = ld16(cur + K2_A_BYTES + (wn * S::WCOLS + nt * 32 + (lane & 31)) * 64 + pos);
    }
#pragma unroll
    for (int step = 0; step < K2_KC / 2; ++step)
      // operands swapped: the MFMA produces D[j][i] = x[i][j], so each lane ends up with
      // runs of 4 consecutive j of one row i.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[mt][nt] = mma32(acc[mt][nt], fb[step][nt], fa[step][mt], T());
    if (next2 >= 0) {
      issue(next);
      issue(next2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (4 + NTW), 0);  // the operand reads
      mfma_load_groups<MFMAS, 2 * LOADS>();
    } else if (next >= 0) {
      issue(next);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (4 + NTW), 0);  // the operand reads
      mfma_load_groups<MFMAS, LOADS>();
    }
  };
  // Stage s's loads are done once at most the later stages' loads (P of them) remain;
  // every wave's part of stage s is then in LDS after the barrier, and every wave is done
  // with the stages whose buffers the next loads overwrite. A bare s_barrier:
  // __syncthreads() would also wait for the later stages' loads still in flight. The empty
  // asm statements keep the compiler from moving LDS accesses across it.
  // The wait also covers this wave's LDS reads (lgkmcnt(0)), so none of stage s-1 is still
  // pending when another wave's loads start to overwrite its buffer.
  auto arrive = [&](auto pending) {
    constexpr int P = decltype(pending)::value;
    static_assert(P * LOADS < 16, "vmcnt in the low field");
    __builtin_amdgcn_s_waitcnt(0x0070 | (P * LOADS));  // vmcnt(P * LOADS) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  static_assert(ST == 3 || ST == 4, "three buffers one stage at a time, or four in pairs");

  // stages of the k loop: up to the bound rounded up to a stage (np is a multiple of the
  // stage), none when the tile lies past the bound
  const int nst = (rows_a == 0 || rows_b == 0) ? 0 : (ext + KT - 1) / KT;
  if constexpr (ST == 3) {
    // one barrier per stage, two stages ahead
    if (nst >= 2) {
      issue(0);
      issue(1);
#pragma unroll 1
      for (int s = 0; s + 2 < nst; ++s) {
        arrive(P1());
        compute(s, s + 2);
      }
      arrive(P1());
      compute(nst - 2, -1);
      arrive(P0());
      compute(nst - 1, -1);
    } else if (nst == 1) {
      issue(0);
      arrive(P0());
      compute(0, -1);
    }
  } else {
    // one barrier per pair of stages (buffers 0-1 and 2-3 alternate): the first stage of a
    // pair issues the loads of both stages of the next pair between its MFMAs, so they
    // have the second stage's compute to arrive
    if (nst > 0) {
      issue(0);
      if (nst > 1) issue(1);
      int s = 0;
#pragma unroll 1
      for (; s + 2 < nst; s += 2) {
        arrive(P0());
        compute(s, s + 2, s + 3 < nst ? s + 3 : -1);
        compute(s + 1, -1);
      }
      arrive(P0());
      compute(s, -1);
      if (s + 1 < nst) compute(s + 1, -1);
    }
  }
  __syncthreads();  // all waves are done reading the ring before it holds the output

  T* Xb = X + bc * mat + (size_t)ti * K2_BM * np + tj * BN;
  if constexpr (sizeof(T) == 2) {
    // stage OUT_ROWS rows of the tile at a time as [i][j] rows (the waves of those rows
    // write them), then 16-byte row-contiguous stores by all waves
    constexpr int XROW = BN + E, OR = S::OUT_ROWS, CPR = BN / E;
    static_assert(OR * XROW * sizeof(T) <= S::LDS_BYTES, "output staging fits");
    T* xs = (T*)lds;
    // the tile's part inside the padded plane (a partial last tile row or column)
    const int vrows = min(np - ti * K2_BM, K2_BM), vchunks = min(np - tj * BN, BN) / E;
    // whole rows with device-scope stores (byte offsets stay below 2^25)
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc_u32(Xb, 0xffffffffu);
#pragma unroll
    for (int h = 0; h < K2_BM / OR; ++h) {
      if (h > 0) __syncthreads();  // the previous rows have left LDS
      if (wm * 128 / OR == h) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = wm * 128 - h * OR + mt * 32 + (lane & 31);
              const int j = wn * S::WCOLS + nt * 32 + 8 * q + 4 * (lane >> 5);
              store4(xs + i * XROW + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
                     acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
            }
      }
      __syncthreads();
#pragma unroll 4
      for (int idx = tid; idx < OR * CPR; idx += NT) {
        const int row = idx / CPR, cc = idx - row * CPR, grow = h * OR + row;
        if (grow < vrows && cc < vchunks)
          store16_sc1(rx, ld16(xs + row * XROW + cc * E),
                      (unsigned int)((grow * np + cc * E) * (int)sizeof(T)));
      }
    }
  } else {
    // fp32: four consecutive j per lane are one 16-byte store (inside the padded plane)
    const int vrows = min(np - ti * K2_BM, K2_BM), vcols = min(np - tj * BN, BN);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = wm * 128 + mt * 32 + (lane & 31);
          const int j = wn * S::WCOLS + nt * 32 + 8 * q + 4 * (lane >> 5);
          if (i < vrows && j < vcols)
            store4(Xb + (size_t)i * np + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
                   acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
        }
  }
}

// bf16 storage: 256 x 256 tiles, 8 waves of 128 x 64 (at N = 2048 the matrix unit time
// per tile is 9% lower than with 256 x 128 tiles; 4 waves of 128 x 128 each run as fast but
// move accumulators between register files inside the loop). While a and b (all planes
// of the launch) fit the 256 MiB last-level cache, the operands come back quickly and one
// barrier per pair of stages is faster (N = 512, 134 MB: 39.7 against 42.1 us); when they
// stream from HBM, a pair's eight loads bunched into one stage's MFMAs cost more than the
// barriers saved (B = 2, N = 768, 604 MB: 322 against 286 us; N = 2048: 2254 against
// 2039 us), so there one stage at a time, two ahead.
constexpr int K2_BF16_WN = 4, K2_BF16_NTW = 2;
constexpr size_t K2_PAIRED_MAX_OPERAND_BYTES = size_t(256) << 20;

template <int BN>
static size_t k2_grid_of(int np, int batch, int c) {
  return (size_t)((np + K2_BM - 1) / K2_BM) * ((np + BN - 1) / BN) * batch * c;
}

// the larger of the two forms' grids (the narrow form's)
size_t k2_grid(int np, int batch, int c) { return k2_grid_of<128>(np, batch, c); }

template <class T, int WN, int NTW, int ST>
static void launch_k2_form(const StageArgs& a, hipStream_t st) {
  using S = K2Shape<WN, NTW, ST>;
  dim3 grid((unsigned)k2_grid_of<S::BN>(a.np, a.batch, a.c));
  hipLaunchKernelGGL((k2_contract<T, WN, NTW, ST>), grid, dim3(S::THREADS), 0, st,
                     (const T*)a.a, (const T*)a.b, (T*)a.x, a.n, a.np, a.extents, a.c);
}

// fp32 storage keeps the 256 x 128 form (its stage holds four times the MFMAs of a bf16
// stage, so its loads are already a smaller share)
hipError_t launch_k2(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  const size_t operand_bytes = 2 * (size_t)a.batch * a.c * a.np * a.np * sizeof(bf16);
  // fewer 256 x 256 tiles than two per CU leave CUs idle (N = 256: 128 tiles): there the
  // 256 x 128 form, two workgroups per CU
  const bool wide_fills = k2_grid_of<256>(a.np, a.batch, a.c) >= 2 * (size_t)a.num_cus;
  if (bf16_storage && !wide_fills)
    launch_k2_form<bf16, 2, 2, 3>(a, st);
  else if (bf16_storage && operand_bytes <= K2_PAIRED_MAX_OPERAND_BYTES)
    launch_k2_form<bf16, K2_BF16_WN, K2_BF16_NTW, 4>(a, st);
  else if (bf16_storage)
    launch_k2_form<bf16, K2_BF16_WN, K2_BF16_NTW, 3>(a, st);
  else
    launch_k2_form<float, 2, 2, 3>(a, st);
  return hipGetLastError();
}

}  // namespace trimul
