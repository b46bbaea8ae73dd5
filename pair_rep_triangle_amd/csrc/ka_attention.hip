// Triangular attention (starting and ending node), two kernels:
//   ka_project: LayerNorm of z and every projection (q, k, gate, v, per-head pair bias)
//               with MFMAs, written in stored coordinates;
//   ka_core:    per stored row, flash attention for every head over 32-key tiles, the
//               gate, and the output projection, written to out.
// Definition and sources: include/tri_attention.h (yage.ai summary of the
// biomolecular-software report: triangular attention as a pair operation of cubic cost
// with a fused kernel; OpenFold-TRT summary: triangular attention among the pair
// kernels). Stored coordinates (r, c) are (i, j) around the starting node and (j, i)
// around the ending node: both nodes then attend along a stored row, keys indexed by the
// stored column, and the pair bias of query column qc and key column kc is the bias of
// stored pair (qc, kc).

#include <type_traits>

#include "attention_launch.h"
#include "device_common.h"

namespace trimul {

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int KA_WAVES = 8;                  // projection kernel
constexpr int KA_THREADS = 64 * KA_WAVES;
constexpr int KA_TW = 32;                    // pairs per projection wave tile
constexpr int KC_WAVES = 4;                  // attention kernel
constexpr int KC_THREADS = 64 * KC_WAVES;
constexpr int KC_QB = 4;                     // 16-query blocks per attention tile
constexpr int KC_KB = 2;                     // 16-key blocks per attention step (2 or 4)
constexpr int KC_MIN_SPLIT = 4;              // workgroups per stored row, at least
// A query's softmax reference starts at 0 and moves up only when a score exceeds it by more
// than KC_HI (base 2), so the unnormalised probabilities stay below 2^16, far inside the
// range of fp32 and bf16 (both keep 8 exponent bits: their relative precision does not
// depend on the scale). At its first valid key a query whose largest score lies below
// KC_LO takes that score as its reference instead, so that a row of very small scores
// cannot underflow.
constexpr float KC_HI = 16.f;
constexpr float KC_LO = -16.f;

// The bias planes and the v^T planes are stored in tiles of 16 rows x 32 columns (1 KB in
// bf16, row-major inside the tile): element (row, col) of a plane with np columns sits at
// tile_off(row, col, np). A wave's 16 rows x 32 keys of a key step are then one 1 KB run.
__device__ __forceinline__ size_t tile_off(int row, int col, int np) {
  return ((size_t)(row >> 4) * (np >> 5) + (col >> 5)) * 512 + (row & 15) * 32 + (col & 31);
}

// A 16-byte store with device scope (cache policy sc1) through a resource on a
// wave-uniform base: written through this XCD's L2 as produced rather than left dirty for
// the end-of-kernel release (every store instruction of ka_project writes whole lines).
// The scalar offset stays 0 (a 16-byte store reads its data registers after it issues; the
// compiler guards them only for stores without a scalar offset register).
__device__ __forceinline__ void store16_sc1(__amdgpu_buffer_rsrc_t r, chunk_t v, unsigned int voff) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)voff, 0, 0x10);
}
// The same store non-temporal (cache policy nt): for output that nothing here reads again.
__device__ __forceinline__ void store16_nt(__amdgpu_buffer_rsrc_t r, chunk_t v, unsigned int voff) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)voff, 0, 0x2);
}

// ---------------------------------------------------------------------------------------
// ka_project. A wave tile is 32 consecutive stored columns (two 16-pair subtiles) of one
// stored row; row p of subtile st is the tile's pair 8 (p / 4) + 4 st + p % 4. z arrives
// in MFMA operand layout (lane (p, q): chunk ks*4 + q of that pair), is normalised in
// registers and is the B operand of the q, k and gate heads (W rows as A, stored
// permuted per head: lane (p, q) ends with channels 8q..8q+7 of its pair) and the A
// operand of the v and bias units (W rows as B: lane (p, q) ends with stored columns
// 8q..8q+7 of output p). Every result leaves as one 16-byte store per lane.
// The weights (LDS image, rows padded by 16 bytes) are loaded once per workgroup. When
// they come in several parts (STREAM), the workgroup's waves take their tiles together
// and the parts pass through LDS one after the other for every round of tiles, with a
// barrier before and after each part's copy; z is read once.
template <int KZ, bool STREAM>
__global__ __launch_bounds__(KA_THREADS) void ka_project(
    const bf16* __restrict__ z, const bf16* __restrict__ mask, const chunk_t* __restrict__ image,
    bf16* __restrict__ qo, bf16* __restrict__ ko, bf16* __restrict__ go, bf16* __restrict__ vto,
    bf16* __restrict__ bo, unsigned int* __restrict__ mwo, int batch, int n, int np, int heads,
    int ending, int mask_all, AttnParts parts) {
  constexpr int E = 8, KG = 32, CZ = KZ * KG, RS = CZ + 8;  // LDS row stride (elements)
  // up to four chunk groups the next tile's z is fetched while this one computes; wider
  // pairs fetch it after the tile (both copies would not fit the registers)
  constexpr bool PREFETCH = KZ <= 4 && !STREAM;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int hd = heads * ATT_D;
  // the part of the projection rows in LDS: [lo, hi), as rows then start values
  int lo = parts.bounds[0], hi = parts.bounds[1];
  const bf16* const wl = (const bf16*)smem;
  const float* tl = (const float*)(smem + (size_t)(hi - lo) * RS * 2);  // start values
  // 16-byte chunks of a part's image
  auto part_chunks = [&](int rows) { return (rows * (CZ + 8) * 2 + rows * 4 + 15) / 16; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;
  const int ctiles = np / KA_TW;
  const int tiles = batch * np * ctiles;
  const int gw = blockIdx.x * KA_WAVES + wave, nw = gridDim.x * KA_WAVES;
  // stored (r, c) -> z pair (x, y); consecutive stored columns are 1 (starting) or n
  // (ending) z pairs apart
  const size_t pstride = ending ? (size_t)n : 1;

  struct Pre {
    chunk_t zv[2][KZ];
    bf16 m[2];
  };
  auto coords = [&](int t, int& b, int& r, int& c0) {
    b = t / (np * ctiles);
    const int rem = t - b * np * ctiles;
    r = rem / ctiles;
    c0 = (rem - r * ctiles) * KA_TW;
  };
  // Row p of subtile st is the tile's pair pp(st) = 8 (p / 4) + 4 st + p % 4, so that the
  // v^T and bias units end with eight consecutive pairs per lane. Pairs outside n x n read
  // as zero (the resource extent ends at the last real pair of the tile's run; rows past
  // n get an empty extent).
  auto pair_of = [&](int st) { return 8 * (p >> 2) + 4 * st + (p & 3); };
  auto fetch = [&](int t, Pre& f) {
    int b, r, c0;
    coords(t < tiles ? t : tiles - 1, b, r, c0);
    const bool ok = r < n && c0 < n;
    const size_t x = ending ? (size_t)c0 : (size_t)r, y = ending ? (size_t)r : (size_t)c0;
    const size_t p0 = ok ? ((size_t)b * n + x) * n + y : 0;
    // pairs from the tile's first to the last real one of its run
    const size_t span = ok ? (size_t)(n - 1 - c0) * pstride + 1 : 0;
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(z + p0 * CZ, span * CZ * 2);
    const __amdgpu_buffer_rsrc_t rm =
        mask_all ? buffer_rsrc(mask, 2) : buffer_rsrc(mask + p0, span * 2);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const unsigned int zoff = (unsigned int)(((size_t)pair_of(st) * pstride * CZ + q * E) * 2);
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) f.zv[st][ks] = load16(rz, zoff + ks * KG * 2, 0);
      f.m[st] = load_elem(rm, mask_all ? 0u : (unsigned int)(pair_of(st) * pstride * 2), 0,
                          bf16());
    }
  };

  Pre f;
  if constexpr (!STREAM) {
    copy_image<KA_THREADS>(image, (chunk_t*)smem, part_chunks(hi - lo), tid, [&]() { fetch(gw, f); });
    __syncthreads();
  }

  // a workgroup-uniform trip count: with STREAM every wave of the workgroup takes part in
  // each round's barriers, also past the last tile
  for (int t0 = blockIdx.x * KA_WAVES; t0 < tiles; t0 += nw) {
    const int t = t0 + wave;
    const bool active = t < tiles;  // wave-uniform
    if (!STREAM && !active) break;
    if constexpr (STREAM) fetch(t, f);  // clamped to the last tile when past it
    int b, r, c0;
    coords(active ? t : tiles - 1, b, r, c0);
    chunk_t za[2][KZ];
    float mv[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      mv[st] = (r < n && c0 + pair_of(st) < n) ? to_f32(f.m[st]) : 0.f;
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) za[st][ks] = f.zv[st][ks];
      normalize_operand_row<KZ>(za[st], CZ, lane, bf16());
    }
    if constexpr (PREFETCH) fetch(t + nw, f);  // the next tile's loads have this tile's MFMAs to land

    const size_t rowbase = ((size_t)b * np + r) * heads;  // [b][r][h] of q, k, g, v^T
    int opaque;  // keeps the loop-invariant LDS reads inside the tile loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));

    // q, k and gate: one head (two 16-row halves, W rows as A) at a time. The handle
    // stores a head's 32 rows permuted: row 4q + rr of half hf is channel 8q + 4 hf + rr,
    // so after both halves lane (p, q) holds channels 8q .. 8q + 7 of the head for pair
    // c0 + 16 st + p, and one 16-byte store per lane writes the pair's whole 64-byte row.
    auto head_a = [&](int row0, int which, bf16* dst) {
      if (row0 < lo || row0 + 32 > hi) return;  // another part's head (uniform)
      const int h = (row0 - which * hd) / ATT_D;
      const int lr = row0 - lo;  // the head's first row in this part's image
      f32x4 acc[2][2];  // [half][st]
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16* const wrow = wl + (lr + 16 * hf + p) * RS + q * E + opaque;
        chunk_t wa[KZ];
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) wa[ks] = ld16(wrow + ks * KG);
        const f32x4 t0 = ld16f(tl + lr + 16 * hf + 4 * q + opaque);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          acc[hf][st] = t0;
#pragma unroll
          for (int ks = 0; ks < KZ; ++ks) acc[hf][st] = mma16(acc[hf][st], wa[ks], za[st][ks], bf16());
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = acc[e >> 2][st][e & 3];
          // gate: rows scaled by -log2(e), sigmoid = 1 / (1 + 2^acc)
          if (which == 2) v[e] = __builtin_amdgcn_rcpf(1.f + exp2f(v[e]));
        }
        const int c = c0 + pair_of(st);
        store16_sc1(buffer_rsrc_u32(dst + (rowbase + h) * np * ATT_D, 0xffffffffu),
                    pack(v, bf16()), (unsigned int)((c * ATT_D + 8 * q) * 2));
      }
    };
    // v and bias units: W rows as B. Lane (p, q): pairs c0 + 8q + 4 st .. +3 (rows 4q .. 4q
    // + 3 of subtile st), output 16u' + p of the block; the two subtiles leave as one
    // 16-byte store of pairs c0 + 8q .. c0 + 8q + 7.
    auto unit_b = [&](int row0, bool bias) {
      if (row0 < lo || row0 + 16 > hi) return;  // another part's unit (uniform)
      const int lr = row0 - lo;
      const bf16* const wrow = wl + (lr + p) * RS + q * E + opaque;
      chunk_t wb[KZ];
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) wb[ks] = ld16(wrow + ks * KG);
      const float t0 = tl[lr + p + opaque];
      // v output row0 - 3 hd + p: its head is the same for the block's 16 rows (row0 - 3 hd
      // is a multiple of 16, a head 32 rows), so the store's base stays wave-uniform
      const int o0 = row0 - 3 * hd;
      const int h = o0 / ATT_D, dd = o0 - h * ATT_D + p;
      float v[8];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 acc = {t0, t0, t0, t0};
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) acc = mma16(acc, za[st][ks], wb[ks], bf16());
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * st + e] = acc[e];
      }
      const int c = c0 + 8 * q;
      if (bias) {
        if (p < heads)
          st16(bo + ((size_t)b * heads + p) * np * np + tile_off(r, c, np), pack(v, bf16()));
      } else {
        store16_sc1(buffer_rsrc_u32(vto + (rowbase + h) * ATT_D * np, 0xffffffffu),
                    pack(v, bf16()), (unsigned int)(tile_off(dd, c, np) * 2));
      }
    };
    // the heads and units of the rows in LDS ([lo, hi))
    auto compute_rows = [&]() {
#pragma unroll 1
      for (int hh = 0; hh < heads; ++hh) head_a(ATT_D * hh, 0, qo);
#pragma unroll 1
      for (int hh = 0; hh < heads; ++hh) head_a(hd + ATT_D * hh, 1, ko);
#pragma unroll 1
      for (int hh = 0; hh < heads; ++hh) head_a(2 * hd + ATT_D * hh, 2, go);
#pragma unroll 1
      for (int u = 0; u < hd / 16; ++u) unit_b(3 * hd + 16 * u, false);
      unit_b(4 * hd, true);
    };
    if constexpr (STREAM) {
      const chunk_t* src = image;
#pragma unroll 1
      for (int pi = 0; pi < parts.count; ++pi) {
        lo = parts.bounds[pi];
        hi = parts.bounds[pi + 1];
        tl = (const float*)(smem + (size_t)(hi - lo) * RS * 2);
        const int chunks = part_chunks(hi - lo);
        __syncthreads();  // every wave is done with the previous part
        copy_image<KA_THREADS>(src, (chunk_t*)smem, chunks, tid, []() {});
        __syncthreads();
        if (active) compute_rows();
        src += chunks;
      }
      if (!active) continue;
    } else {
      compute_rows();
    }
    // key-valid bits in stored coordinates (0 on padding): bit k of word c0 / 32 of
    // stored row r is column c0 + k (nonzero mask value); lanes q = 0 hold the tile's
    // 32 values
    // (lane p of subtile st holds pair 8 (p / 4) + 4 st + p % 4: nibble g of a ballot
    // goes to bits 8g + 4 st)
    const unsigned long long v0 = __ballot(q == 0 && mv[0] != 0.f);
    const unsigned long long v1 = __ballot(q == 0 && mv[1] != 0.f);
    unsigned int word = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      word |= (unsigned int)((v0 >> (4 * g)) & 0xfu) << (8 * g) |
              (unsigned int)((v1 >> (4 * g)) & 0xfu) << (8 * g + 4);
    if (lane == 0) mwo[((size_t)b * np + r) * (np / 32) + c0 / 32] = word;
    if constexpr (!PREFETCH && !STREAM) fetch(t + nw, f);
  }
}

// ---------------------------------------------------------------------------------------
// ka_core. Stored row r is shared by `split` workgroups (query tiles share, share +
// split, ...); the four waves of a workgroup take the heads (wave w: heads
// w, w + 4). Per tile of 16 QB query columns and head, a wave runs the keys in steps of
// 16 KB, with the step's keys permuted so that lane q owns 4 KB consecutive ones:
//   S^T = K Q^T (key rows, query columns) with the pair bias minus the query's softmax
//     reference as the accumulator start: lane (p, q) of block kb holds keys
//     4 KB q + 4 kb + e (e < 4) of query 16 qb + p (the K operand's row p is key
//     4 KB (p / 4) + 4 kb + p % 4);
//   online softmax per query in base 2 (log2(e) / sqrt(d) is folded into W_q and
//     log2(e) into the bias rows), masked keys left out. The reference starts at 0 and
//     moves only when a score exceeds it by more than KC_HI, or when the query's first
//     valid scores all lie below KC_LO (then the four lanes p, p^16, p^32, p^48, which
//     hold all keys of a query, agree on the new one); the sum is kept per lane until the
//     end;
//   O^T += V^T P^T: each run of eight of the lane's probabilities of a query ARE its
//     B-operand chunk once V^T's A chunk holds the same eight keys, one 16-byte run of
//     the transposed v.
// Then o = O^T / l * gate goes to LDS as [query][h*d + channel]; after a barrier the
// waves split the output channels: out^T = W_o o^T + b_o with W_o rows from LDS as A.
// Three waves per SIMD (at most 170 registers): at c_z = 128 the kernel needs 166 with no
// spills; at the other widths 2 to 20 registers spill, all outside the key loop, which
// costs less than the third wave would (wide ka_core 1484 -> 1370 us when the W_o slices
// came in).
template <int KZ, int QB, int KB>
__global__ __launch_bounds__(KC_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void ka_core(
    const bf16* __restrict__ qi, const bf16* __restrict__ ki, const bf16* __restrict__ gi,
    const bf16* __restrict__ vti, const bf16* __restrict__ bi, const unsigned int* __restrict__ mwi,
    const chunk_t* __restrict__ image, int image_chunks, bf16* __restrict__ out, int n, int np,
    int heads, int ending, int rows, int split) {
  constexpr int CZ = KZ * 32;
  constexpr int QT = 16 * QB;  // queries per tile
  // W_o lives in LDS a slice of ATT_WO_ROWS output rows at a time: the whole matrix up to
  // c_z = 128 (copied once), else slice after slice for every query tile
  constexpr int SROWS = CZ < ATT_WO_ROWS ? CZ : ATT_WO_ROWS;
  constexpr int NSLICE = (CZ + SROWS - 1) / SROWS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int hd = heads * ATT_D, os_stride = hd + 8;
  const bf16* const wo = (const bf16*)smem;                                    // [SROWS][hd + 8]
  const float* const bo = (const float*)(smem + (size_t)SROWS * os_stride * 2);  // [SROWS]
  bf16* const os = (bf16*)(smem + (size_t)SROWS * os_stride * 2 + SROWS * 4);    // [64][hd + 8]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;
  // XCD-aware order: workgroup ids are dealt to the eight XCDs in turn. The `split`
  // workgroups of stored row `row` get ids equal mod 8 and within 8 * split of each other,
  // so they run together on one XCD and read the row's K and V^T through its L2 once.
  const int grp = blockIdx.x / (8 * split), w8 = blockIdx.x - grp * 8 * split;
  const int share = w8 >> 3, row = grp * 8 + (w8 & 7);
  if (row >= rows) return;  // the last group of eight may be partial (whole workgroup)
  const int b = row / n, r = row - b * n;
  if constexpr (NSLICE == 1) {
    copy_image<KC_THREADS>(image, (chunk_t*)smem, image_chunks, tid, []() {});
    __syncthreads();
  }

  constexpr int KT = 16 * KB;  // keys per step
  const int ksteps = (n + KT - 1) / KT;  // key steps past n would be all masked
  const unsigned int* const mwrow = mwi + ((size_t)b * np + r) * (np / 32);
  // a row without any valid key (a padded residue) adds nothing: its queries get a zero
  // attention output without running the key steps
  unsigned int anyv = 0;
  for (int t = lane; t < np / 32; t += 64) anyv |= mwrow[t];
  const int kend = __any(anyv != 0u) ? ksteps : 0;
  const float NEG = -__builtin_huge_valf();

  for (int qt = share; qt < np / QT; qt += split) {
    const int qc0 = qt * QT;
    for (int h = wave; h < heads; h += KC_WAVES) {
      const size_t rh = ((size_t)b * np + r) * heads + h;
      const bf16* const qrow = qi + rh * np * ATT_D;
      const bf16* const krow = ki + rh * np * ATT_D;
      const bf16* const vrow = vti + rh * ATT_D * np;
      const bf16* const brow = bi + ((size_t)b * heads + h) * np * np;
      chunk_t qf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qf[qb] = ld16(qrow + (size_t)(qc0 + 16 * qb + p) * ATT_D + 8 * q);
      // Per query (the same on its four lanes): the reference mref that every score is
      // taken relative to, and whether the query has seen a valid key (bit `lane` of
      // hasref). lsum and o are the sum of the probabilities and O^T, both relative to
      // 2^mref.
      f32x4 o[2][QB];
      float mref[QB], lsum[QB];
      unsigned long long hasref[QB];  // wave-uniform
      bool zref = true;               // every mref of the wave is 0 (wave-uniform)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mref[qb] = 0.f;
        hasref[qb] = 0ull;
        lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < 2; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // One key step's operands (KB blocks of 16 keys): K chunks, the bias tiles (the
      // accumulator start of S^T), the key-valid bits and V^T chunks. Each is reloaded for
      // the next step right after its last use in this one (bias, K and the bits after the
      // S^T MFMAs, V^T after the O^T MFMAs), so the loads run a step ahead with no copies.
      // Key order: lane q of a step owns the 4 KB consecutive keys 4 KB q .. 4 KB q + 4 KB - 1
      // (row 4q + e of S^T block kb is key 4 KB q + 4 kb + e), so its bias values and its
      // V^T chunks are whole 16-byte runs.
      chunk_t kf[KB], vf[KB / 2][2];
      chunk_t sb[KB / 2][QB];  // eight bf16 bias values per chunk and lane
      unsigned long long mw;  // the step's key-valid bits (bit k: key k0 + k), wave-uniform
      // Every load of a step is a step-uniform base plus a per-lane byte offset that is the
      // same in every step (keys advance in whole bias and V^T tiles: KT is a multiple of
      // 32): a step adds the new bases to offsets computed once per tile.
      // K: A row p of block kb is key 4 KB (p / 4) + 4 kb + p % 4 (block kb: + 8 kb rows of
      // ATT_D bf16)
      const unsigned int ko = (unsigned int)(((4 * KB * (p >> 2) + (p & 3)) * ATT_D + 8 * q) * 2);
      // bias of query 16 qb + p, keys 4 KB q + 8 j .. + 7: tile row p of query tile row
      // qc0 / 16 + qb, tile column k0 / 32 + c / 32 (c = 4 KB q + 8 j)
      unsigned int bo[KB / 2];
#pragma unroll
      for (int j = 0; j < KB / 2; ++j) {
        const int c = 4 * KB * q + 8 * j;
        bo[j] = (unsigned int)(((c >> 5) * 512 + p * 32 + (c & 31)) * 2);
      }
      // V^T row p of block db is channel 8 (p / 4) + 4 db + p % 4, so that O^T lane (p, q)
      // ends with channels 8q .. 8q + 7 of its query across the two blocks (one 16-byte
      // gate load and one 16-byte staging store); half kh of the step: keys 4 KB q + 8 kh
      // .. + 7 (the keys of the lane's probabilities pv[8 kh .. 8 kh + 7])
      unsigned int vo[KB / 2][2];
#pragma unroll
      for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int vr = 8 * (p >> 2) + 4 * db + (p & 3), c = 4 * KB * q + 8 * kh;
          vo[kh][db] = (unsigned int)((((vr >> 4) * (np >> 5) + (c >> 5)) * 512 + (vr & 15) * 32 + (c & 31)) * 2);
        }
      const size_t bq = (size_t)np * 32;  // bytes from one query tile row of the bias to the next
      const unsigned char* const bq0 = (const unsigned char*)(brow + (size_t)(qc0 >> 4) * (np >> 5) * 512);
      auto load_kbm = [&](int ks) {
        const int k0 = (ks < ksteps ? ks : ksteps - 1) * KT;
        if constexpr (KB == 2) {
          mw = (unsigned int)__builtin_amdgcn_readfirstlane(mwrow[k0 / 32]);  // zero-extended
        } else {
          const u32x2 w2 = *(const u32x2*)(mwrow + k0 / 32);
          mw = (unsigned long long)(unsigned int)__builtin_amdgcn_readfirstlane(w2[0]) |
               ((unsigned long long)(unsigned int)__builtin_amdgcn_readfirstlane(w2[1]) << 32);
        }
        const unsigned char* const kbase = (const unsigned char*)(krow + (size_t)k0 * ATT_D);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[kb] = ld16(kbase + ko + kb * 8 * ATT_D);
        const unsigned char* const bbase = bq0 + (size_t)k0 * 32;  // k0 / 32 tiles of 1 KB
#pragma unroll
        for (int j = 0; j < KB / 2; ++j)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sb[j][qb] = ld16(bbase + qb * bq + bo[j]);
      };
      auto load_v = [&](int ks) {
        const int k0 = (ks < ksteps ? ks : ksteps - 1) * KT;
        const unsigned char* const vbase = (const unsigned char*)(vrow + (size_t)k0 * 16);
#pragma unroll
        for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
          for (int db = 0; db < 2; ++db) vf[kh][db] = ld16(vbase + vo[kh][db]);
      };
      load_kbm(0);
      load_v(0);
#pragma unroll 1
      for (int ks = 0; ks < kend; ++ks) {
        const unsigned long long w = mw;
        // S^T relative to the reference: the accumulator starts at bias - mref, or at the
        // bias itself while every reference of the wave is 0 (the common case)
        f32x4 s[KB][QB];
        auto scores = [&](auto zero_ref) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const unsigned int b01 = sb[kb >> 1][qb][2 * (kb & 1)];
              const unsigned int b23 = sb[kb >> 1][qb][2 * (kb & 1) + 1];
              f32x4 b0 = {__uint_as_float(b01 << 16), __uint_as_float(b01 & 0xffff0000u),
                          __uint_as_float(b23 << 16), __uint_as_float(b23 & 0xffff0000u)};
              if constexpr (!decltype(zero_ref)::value) {
                const float m = mref[qb];
                b0 = f32x4{b0[0] - m, b0[1] - m, b0[2] - m, b0[3] - m};
              }
              s[kb][qb] = mma16(b0, kf[kb], qf[qb], bf16());
            }
        };
        if (zref)
          scores(std::true_type{});
        else
          scores(std::false_type{});
        load_kbm(ks + 1);  // the last step reloads itself (unused)
        // A step with masked keys first turns their scores into -inf, so that their
        // exponentials below are exactly 0; the common case (every key of the step valid)
        // runs no select at all (the key word is wave-uniform: a scalar branch).
        if (w != (KB == 2 ? 0xffffffffull : ~0ull)) {
          const unsigned long long wl = w >> (4 * KB * q);  // keys 4 KB q + 4 kb + e
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool valid = (wl >> (4 * kb + e)) & 1u;
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) s[kb][qb][e] = valid ? s[kb][qb][e] : NEG;
            }
        }
        // Online softmax with a reference that moves only when it must: a score more than
        // KC_HI above it (or, at the query's first valid key, a largest score below KC_LO)
        // moves the query's reference to its largest score of the step and scales what it
        // has summed so far. Otherwise the step's probabilities are 2^s directly, at most
        // 2^KC_HI, with no maximum across lanes and no rescaling. The test is per lane, the
        // branch per wave (rare after the first step). The result is the same softmax: o
        // and l carry the same factor 2^-mref, which the division at the end removes.
        // The lane's largest score of query block qb in this step:
        auto lane_max = [&](int qb) {
          float v = s[0][qb][0];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb + e > 0) v = fmaxf(v, s[kb][qb][e]);
          return v;
        };
        bool move = false, unset = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          move |= lane_max(qb) > KC_HI;
          unset |= hasref[qb] != ~0ull;
        }
        if (unset || __any(move)) {
          bool moved = false;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            // the query's largest score of the step relative to its reference (-inf when
            // every key of the step is masked)
            const float lm = lane_max(qb);
            float rm = fmaxf(lm, lane_value(lm, lane ^ 16));
            rm = fmaxf(rm, lane_value(rm, lane ^ 32));
            const bool has = (hasref[qb] >> lane) & 1ull;  // a valid key was seen before
            const bool valid = rm > NEG;                   // the step has a valid key
            const bool mv = has ? rm > KC_HI : valid && (rm > KC_HI || rm < KC_LO);
            const float delta = mv ? rm : 0.f;
            // before the first valid key nothing was summed: o and lsum are 0
            const float f = has ? __builtin_amdgcn_exp2f(-delta) : 0.f;
            lsum[qb] *= f;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int e = 0; e < 4; ++e) o[db][qb][e] *= f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int e = 0; e < 4; ++e) s[kb][qb][e] -= delta;
            mref[qb] += delta;
            moved |= mv;
            hasref[qb] = __ballot(has || valid);
          }
          zref = zref && !__any(moved);
        }
        // probabilities in base 2 (results below 2^-126 flush to 0)
        chunk_t pb[KB / 2][QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float pv[4 * KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[4 * kb + e] = __builtin_amdgcn_exp2f(s[kb][qb][e]);
          float ps = pv[0];
#pragma unroll
          for (int e = 1; e < 4 * KB; ++e) ps += pv[e];
          lsum[qb] += ps;
#pragma unroll
          for (int kh = 0; kh < KB / 2; ++kh) pb[kh][qb] = pack(pv + 8 * kh, bf16());
        }
#pragma unroll
        for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < 2; ++db)
              o[db][qb] = mma16(o[db][qb], vf[kh][db], pb[kh][qb], bf16());
        load_v(ks + 1);
      }
      // normalise, gate, stage: o^T lane (p, q) reg e of block db = channel 8q + 4 db + e
      // of query 16 qb + p
      const bf16* const grow = gi + rh * np * ATT_D;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float l = lsum[qb];
        l += lane_value(l, lane ^ 16);
        l += lane_value(l, lane ^ 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int qc = qc0 + 16 * qb + p;
        float gv[8], ov[8];
        unpack(ld16(grow + (size_t)qc * ATT_D + 8 * q), gv, bf16());
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = o[e >> 2][qb][e & 3] * inv * gv[e];
        st16(os + (16 * qb + p) * os_stride + h * ATT_D + 8 * q, pack(ov, bf16()));
      }
    }
    __syncthreads();
    // out^T = W_o o^T + b_o per group of 32 output channels, as two 16-row halves. The
    // handle stores W_o's rows (and b_o) permuted per group: row 4q + rr of half hf is
    // channel 8q + 4 hf + rr, so lane (p, q) ends with channels 32g + 8q .. + 7 of query
    // 16 qb + p. Each wave takes one block of 16 queries and runs the groups two at a
    // time: after a swap of one 16-byte chunk between lanes p and p ^ 8 of each row of 16
    // lanes (a DPP rotation by 8 written to half of the row), each of the two store
    // instructions writes whole 128-byte lines (one query's 64 channels from 8 lanes),
    // non-temporal: the output is not read again here and would only displace K, V^T and
    // the bias from the caches (ka_core 156.3 -> 154.7 us, wide 1403 -> 1340 us, against
    // half lines from two waves; device-scope or default-policy stores of the same lines
    // made the step slower). A group left over (c_z an odd number of groups) is written
    // in half lines.
#pragma unroll 1
    for (int sl = 0; sl < NSLICE; ++sl) {
      const int g0 = sl * (SROWS / 32);  // the slice's first group
      const int ng = CZ / 32 - g0 < SROWS / 32 ? CZ / 32 - g0 : SROWS / 32;  // its groups
      if constexpr (NSLICE > 1) {
        // the slice's W_o rows and b_o values into LDS (after every wave is done with the
        // previous slice)
        if (sl > 0) __syncthreads();
        const int srows = 32 * ng;
        const chunk_t* const src = (const chunk_t*)((const unsigned char*)image +
                                                    (size_t)32 * g0 * os_stride * 2);
        const int wchunks = srows * os_stride * 2 / 16;
        for (int i = tid; i < wchunks; i += KC_THREADS) ((chunk_t*)smem)[i] = src[i];
        const chunk_t* const bsrc = (const chunk_t*)((const unsigned char*)image +
                                                     (size_t)CZ * os_stride * 2 + 32 * g0 * 4);
        for (int i = tid; i < srows / 4; i += KC_THREADS) ((chunk_t*)bo)[i] = bsrc[i];
        __syncthreads();
      }
      for (int qb = wave; qb < QB; qb += KC_WAVES) {
        const int qbase = qc0 + 16 * qb;
        // the block's first query is the stores' (wave-uniform) base: the offsets of its 16
        // queries stay below 15 n c_z + c_z elements, inside 32 bits at any supported n
        const size_t x0 = ending ? (size_t)qbase : (size_t)r, y0 = ending ? (size_t)r : (size_t)qbase;
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc_u32(out + (((size_t)b * n + x0) * n + y0) * CZ, 0xffffffffu);
        const unsigned int qstride = (unsigned int)(ending ? n * CZ : CZ) * 2u;  // bytes per query
        auto unit = [&](int g, int hf) {
          const int u = 2 * (g - g0) + hf;  // the unit's rows in the slice
          f32x4 acc = ld16f(bo + 16 * u + 4 * q);
          for (int kk = 0; kk < hd / 32; ++kk)
            acc = mma16(acc, ld16(wo + (16 * u + p) * os_stride + 32 * kk + 8 * q),
                        ld16(os + (16 * qb + p) * os_stride + 32 * kk + 8 * q), bf16());
          return acc;
        };
        auto chunk = [&](const f32x4& h0, const f32x4& h1) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = h0[e];
            v[4 + e] = h1[e];
          }
          return pack(v, bf16());
        };
        int gi = 0;
#pragma unroll 1
        for (; gi + 1 < ng; gi += 2) {
          const int g = g0 + gi;
          const chunk_t c0 = chunk(unit(g, 0), unit(g, 1));
          const chunk_t c1 = chunk(unit(g + 1, 0), unit(g + 1, 1));
          // lo: lanes p < 8 keep group g of query p, lanes p >= 8 take group g + 1 of query
          // p - 8 from lane p - 8; hi: lanes p < 8 take group g of query p + 8 from lane
          // p + 8, lanes p >= 8 keep group g + 1 of query p
          chunk_t lo, hi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            lo[d] = (unsigned int)__builtin_amdgcn_update_dpp((int)c0[d], (int)c1[d], 0x128, 0xf, 0xc, false);
            hi[d] = (unsigned int)__builtin_amdgcn_update_dpp((int)c1[d], (int)c0[d], 0x128, 0xf, 0x3, false);
          }
          const int qa = p & 7;  // query of lo (hi: qa + 8)
          const unsigned int off = (unsigned int)qa * qstride + (unsigned int)(32 * (g + (p >> 3)) + 8 * q) * 2u;
          if (qbase + qa < n) store16_nt(ro, lo, off);
          if (qbase + qa + 8 < n) store16_nt(ro, hi, off + 8u * qstride);
        }
        if (gi < ng) {
          const int g = g0 + gi;
          const chunk_t c0 = chunk(unit(g, 0), unit(g, 1));
          const int qc = qbase + p;
          if (qc < n) {
            const size_t x = ending ? (size_t)qc : (size_t)r, y = ending ? (size_t)r : (size_t)qc;
            __builtin_nontemporal_store(c0, (chunk_t*)(out + (((size_t)b * n + x) * n + y) * CZ + 32 * g + 8 * q));
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------

template <int KZ>
static hipError_t launch_attention_kz(const AttnArgs& a, int stages, hipStream_t st) {
  const int np = att_np(a.n);
  const AttnWorkspace L = att_workspace(a.batch, a.n, a.heads);
  unsigned char* ws = (unsigned char*)a.ws;
  bf16* q = (bf16*)(ws + L.q);
  bf16* k = (bf16*)(ws + L.k);
  bf16* g = (bf16*)(ws + L.g);
  bf16* vt = (bf16*)(ws + L.vt);
  bf16* bias = (bf16*)(ws + L.bias);
  unsigned int* mw = (unsigned int*)(ws + L.ms);

  // projection: persistent waves over 32-pair tiles of the padded stored grid; weights in
  // several parts pass through LDS part after part
  if (stages & 1) {
    const AttnParts parts = att_proj_parts(a.cz, a.heads);
    if (parts.count < 1) return hipErrorInvalidValue;
    size_t lds = 0;
    for (int i = 0; i < parts.count; ++i) {
      const size_t b = att_part_bytes(a.cz, parts.bounds[i + 1] - parts.bounds[i]);
      lds = b > lds ? b : lds;
    }
    if (lds > ATT_LDS_MAX) return hipErrorInvalidValue;
    auto fn = parts.count == 1 ? ka_project<KZ, false> : ka_project<KZ, true>;
    static std::atomic<int> granted1{0}, granted2{0};
    hipError_t e = ensure_dynamic_lds((const void*)fn, parts.count == 1 ? granted1 : granted2, lds);
    if (e != hipSuccess) return e;
    const long long tiles = (long long)a.batch * np * (np / KA_TW);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    static std::atomic<int> occ1{0}, occ2{0};
    static std::atomic<size_t> occ_lds1{0}, occ_lds2{0};
    const int per_cu = parts.count == 1
                           ? resident_blocks((const void*)fn, KA_THREADS, lds, occ1, occ_lds1)
                           : resident_blocks((const void*)fn, KA_THREADS, lds, occ2, occ_lds2);
    const long long need = (tiles + KA_WAVES - 1) / KA_WAVES;
    const long long cap = (long long)a.num_cus * per_cu;
    const int blocks = (int)(need < cap ? need : cap);
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(KA_THREADS), lds, st, (const bf16*)a.z,
                       (const bf16*)a.mask, (const chunk_t*)a.proj_image, q, k, g, vt, bias, mw,
                       a.batch, a.n, np, a.heads, a.node, a.mask_all, parts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // attention: one workgroup per stored row
  if (stages & 2) {
    const size_t img = att_out_image_bytes(a.cz, a.heads);
    const size_t lds = att_core_lds_bytes(a.cz, a.heads);
    if (img % 16) return hipErrorInvalidValue;
    constexpr int QB = KC_QB;
    static_assert(KC_KB == 2 || KC_KB == 4, "a step is 32 or 64 keys");
    auto fn = ka_core<KZ, QB, KC_KB>;
    static std::atomic<int> granted{0};
    hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.batch * a.n;
    if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
    // a row's query tiles are shared by `split` workgroups on one XCD: at least
    // KC_MIN_SPLIT (they share the row's K and V^T through L2), enough for four per CU
    const int qtiles = np / (16 * QB);
    const long long rows8 = (rows + 7) / 8 * 8;
    long long split = ((long long)a.num_cus * 4 + rows - 1) / rows;
    if (split < KC_MIN_SPLIT) split = KC_MIN_SPLIT;
    if (split > qtiles) split = qtiles;
    while (split > 1 && rows8 * split > 0x7fffffffLL) --split;
    if (rows8 * split > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned int)(rows8 * split)), dim3(KC_THREADS), lds, st, q, k,
                       g, vt, bias, mw, (const chunk_t*)a.out_image, (int)(img / 16),
                       (bf16*)a.out, a.n, np, a.heads, a.node, (int)rows, (int)split);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, int stages, hipStream_t st) {
  switch (a.cz / 32) {
    case 1: return launch_attention_kz<1>(a, stages, st);
    case 2: return launch_attention_kz<2>(a, stages, st);
    case 3: return launch_attention_kz<3>(a, stages, st);
    case 4: return launch_attention_kz<4>(a, stages, st);
    case 5: return launch_attention_kz<5>(a, stages, st);
    case 6: return launch_attention_kz<6>(a, stages, st);
    case 7: return launch_attention_kz<7>(a, stages, st);
    case 8: return launch_attention_kz<8>(a, stages, st);
    case 9: return launch_attention_kz<9>(a, stages, st);
    case 10: return launch_attention_kz<10>(a, stages, st);
    case 11: return launch_attention_kz<11>(a, stages, st);
    case 12: return launch_attention_kz<12>(a, stages, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace trimul
