// k1: input LayerNorm + gated dual projection + pair mask -> a, b (channel-major).
//
// RFProteína architecture page, "Triangle multiplication on SM90" (K1: the input
// projection with the input LayerNorm, producing the gated operands) and "Dual-GEMM
// gates" (x_x form sigma(x W_g^T + b_g) * (x W_p^T + b_p); the input gate absorbs the
// pair mask and writes its output already laid out for the contraction).
//
// Work split (persistent): a tile is TP = 64 consecutive storage columns of one storage
// row r; for outgoing the z pairs are (r, s), for incoming (s, r), so both directions
// store a[b][ch][r][s] contiguously along s. A workgroup of 8 waves loops over tiles.
// Each wave owns UPW "units" (a unit = the gate and proj rows of 16 channels of a or b)
// and keeps their weights in registers for the whole launch; the tile's normalised z
// (the MFMA A operand) is shared through double-buffered LDS. The LayerNorm gamma is
// folded into the weights and beta / the bias into the accumulator's initial value (host
// side); the gate rows carry an extra -log2(e) so the gate is one exp2 and one reciprocal.
// The k extent is a compile-time constant: the host pads c_z to exactly KMAX chunk groups.
// The next tile's z is fetched into registers while the MFMAs of the current tile run.
// Results are staged per wave in LDS and written as whole rows of TP contiguous pairs.

#include <type_traits>

#include "device_common.h"
#include "k1w_layout.h"

namespace trimul {

constexpr int K1_TP = 64;

template <class T, int KMAX, int UPW, int W>
__global__ __launch_bounds__(64 * W) void k1_input_gate(
    const T* __restrict__ z, const T* __restrict__ mask, T* __restrict__ a_out,
    T* __restrict__ b_out, const T* __restrict__ w1, const float* __restrict__ t1, int n, int np,
    int cz, int czp, int c, int incoming, int mask_all, int nbuf, int total_tiles) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int TP = K1_TP;
  constexpr int THREADS = 64 * W;
  constexpr int TPP = THREADS / TP;  // threads per pair when staging a tile
  constexpr int NCH = (KMAX * KG / E + TPP - 1) / TPP;  // z chunks per thread
  // staging row (one channel, TP pairs): for bf16 an 8-byte-aligned stride of 34 dwords so
  // the 8-byte writes of 16 consecutive rows hit distinct banks; fp32 rows stay 16-byte
  // aligned (68 dwords).
  constexpr int SROW = TP + 4;
  constexpr int CPT = TP / E;       // 16-byte chunks per staged row
  constexpr int NST = UPW * 16 * CPT / 64;  // 16-byte stores per lane per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int zstride = czp + E;
  // LDS: normalised z tiles [nbuf][TP][zstride], masks [nbuf][TP], per-wave output
  // staging [UPW*16 channels][SROW]. nbuf = 2 double-buffers the z tile; wide c_z that does
  // not fit uses one buffer and an extra barrier per tile.
  T* const zbase = (T*)smem;
  float* const mvbuf = (float*)(zbase + nbuf * TP * zstride);
  auto zbuf = [&](int b) { return zbase + b * TP * zstride; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const stg = (T*)(mvbuf + nbuf * TP) + (size_t)wave * UPW * 16 * SROW;
  const int cblocks = c / 16, units = 2 * cblocks;
  const int ntx = np / TP;
  const size_t plane = (size_t)np * np;  // one channel of a or b

  // ---- this wave's units: weights and biases into registers ----
  chunk_t wgt[UPW][2][KMAX];
  f32x4 bias[UPW][2];
  int uq[UPW], ucb[UPW];
  bool uok[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = blockIdx.y * (W * UPW) + wave + W * j;
    uok[j] = u < units;
    uq[j] = uok[j] ? u / cblocks : 0;
    ucb[j] = uok[j] ? (u - uq[j] * cblocks) * 16 : 0;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const size_t row = (size_t)(2 * uq[j] + gp) * c + ucb[j] + (lane & 15);
      const float bv = uok[j] ? t1[row] : 0.f;
      bias[j][gp] = f32x4{bv, bv, bv, bv};
#pragma unroll
      for (int ks = 0; ks < KMAX; ++ks)
        wgt[j][gp][ks] = uok[j] ? ld16(w1 + row * czp + ks * KG + (lane >> 4) * E)
                                : chunk_t{0u, 0u, 0u, 0u};
    }
  }
  // per-lane offsets of the staged rows this lane stores (k-th store: row, chunk)
  size_t soff[NST];
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const int idx = k * 64 + lane, row = idx / CPT, cc = idx - row * CPT;
    soff[k] = (size_t)(ucb[row >> 4] + (row & 15)) * plane + cc * E;
  }

  // ---- tile staging: thread (t, part) handles chunks part, part+TPP, ... of pair t ----
  const int t = tid / TPP, part = tid % TPP;
  const int czc = cz / E, cpr = czp / E;
  // pair t of a tile sits t pairs (outgoing) or t rows (incoming) after the tile's first pair
  const size_t tstep = incoming ? (size_t)n : 1;

  // Tiles are visited as tile = blockIdx.x + k * gridDim.x with tile = (bb*np + r)*ntx + sx;
  // the coordinates advance incrementally (no divisions in the loop).
  struct Coord {
    int bb, r, sx;
  };
  auto decompose = [&](int tile) {
    Coord q;
    q.bb = tile / (np * ntx);
    const int rem = tile - q.bb * np * ntx;
    q.r = rem / ntx;
    q.sx = rem - q.r * ntx;
    return q;
  };
  const Coord step = decompose(gridDim.x);
  auto advance = [&](Coord q) {
    q.sx += step.sx;
    q.r += step.r;
    q.bb += step.bb;
    if (q.sx >= ntx) {
      q.sx -= ntx;
      ++q.r;
    }
    if (q.r >= np) {
      q.r -= np;
      ++q.bb;
    }
    return q;
  };

  // The next tile is fetched into registers with unconditional loads from clamped,
  // in-bounds addresses (no branches), and every select that depends on the loaded data
  // happens in stage(), after the current tile's MFMAs: the loads stay in flight meanwhile.
  // `mask_all` (no mask given) reads the one-valued element at mask[0].
  struct Pre {
    chunk_t v[NCH];
    T m;
    bool valid;
  };
  auto fetch = [&](Coord q, Pre& f) {
    const int s0 = q.sx * TP;
    const bool tile_ok = q.r < n && s0 < n;  // uniform
    f.valid = tile_ok && s0 + t < n;
    // first pair of the tile: (r, s0) outgoing, (s0, r) incoming
    const size_t p0 = tile_ok ? (incoming ? ((size_t)q.bb * n + s0) * n + q.r
                                          : ((size_t)q.bb * n + q.r) * n + s0)
                              : 0;
    const size_t pair = p0 + (f.valid ? t * tstep : 0);
    const T* src = z + pair * cz;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = part + TPP * i;
      f.v[i] = ld16(src + (ch < czc ? ch : 0) * E);
    }
    f.m = mask[mask_all ? 0 : pair];
  };
  auto stage = [&](int buf, Pre& f) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (!(f.valid && part + TPP * i < czc)) f.v[i] = chunk_t{0u, 0u, 0u, 0u};
    normalize_row<T, NCH, TPP>(f.v, part, czc, cz);
    // every lane stores (no branch): a chunk index past the padded row lands in the row's
    // spare last E columns, which no MFMA operand read touches
    T* row = zbuf(buf) + t * zstride;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = part + TPP * i;
      st16(row + (ch < cpr ? ch * E : czp), f.v[i]);
    }
    if (part == 0) mvbuf[buf * TP + t] = f.valid ? to_f32(f.m) : 0.f;
  };

  // staging -> global: UPW*16 channel rows of TP contiguous elements (full cache lines).
  // A tile's rows are stored at the start of the next iteration (or after the loop), so
  // that the stores are long complete when stage() waits for the next tile's loads.
  auto store_tile = [&](Coord q) {
    wave_lds_sync();
    const size_t tbase = (size_t)q.bb * c * plane + (size_t)q.r * np + q.sx * TP;
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int idx = k * 64 + lane, row = idx / CPT, cc = idx - row * CPT;
      const int j = (k * 64) / CPT / 16;  // the same unit for the whole store
      if (uok[j]) {                       // wave-uniform
        T* dst = (uq[j] ? b_out : a_out) + tbase + soff[k];
        st16(dst, ld16_lds8(stg + row * SROW + cc * E));
      }
    }
  };

  int tile = blockIdx.x;  // the grid never exceeds the tile count
  Coord cur_c = decompose(tile);
  Coord pend = cur_c;
  {
    Pre f;
    fetch(cur_c, f);
    stage(0, f);
  }
  __syncthreads();

  for (int it = 0; tile < total_tiles; tile += gridDim.x, ++it) {
    if (it > 0) store_tile(pend);
    const int cur = nbuf == 2 ? (it & 1) : 0;
    const bool has_next = tile + (int)gridDim.x < total_tiles;
    const Coord next_c = has_next ? advance(cur_c) : cur_c;
    Pre pre;
    fetch(next_c, pre);  // the last iteration refetches the current tile, unused

    const T* zs = zbuf(cur);
    const float* mv = mvbuf + cur * TP;
    // Software pipeline over the four 16-pair row tiles: the MFMAs of row tile rt+1 are
    // issued before the gate epilogue of row tile rt, so the matrix cores and the
    // VALU/transcendental units work on different row tiles at the same time.
    auto mma_rt = [&](int rt, f32x4 (&acc)[UPW][2]) {
      const T* arow = zs + (rt * 16 + (lane & 15)) * zstride + (lane >> 4) * E;
      chunk_t af[KMAX];
#pragma unroll
      for (int ks = 0; ks < KMAX; ++ks) af[ks] = ld16(arow + ks * KG);
#pragma unroll
      for (int j = 0; j < UPW; ++j) {
        acc[j][0] = mma16(bias[j][0], af[0], wgt[j][0][0], T());
        acc[j][1] = mma16(bias[j][1], af[0], wgt[j][1][0], T());
      }
#pragma unroll
      for (int ks = 1; ks < KMAX; ++ks)
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
          acc[j][0] = mma16(acc[j][0], af[ks], wgt[j][0][ks], T());
          acc[j][1] = mma16(acc[j][1], af[ks], wgt[j][1][ks], T());
        }
    };
    // accumulator register rr <-> pair rt*16 + 4*(lane/16) + rr, channel lane%16 of unit
    auto epi_rt = [&](int rt, const f32x4 (&acc)[UPW][2]) {
      const int p0 = rt * 16 + 4 * (lane >> 4);
      T* const srow = stg + (lane & 15) * SROW + p0;
      const f32x4 m4 = ld16f(mv + p0);
#pragma unroll
      for (int j = 0; j < UPW; ++j)
        store4(srow + j * 16 * SROW, gate_mul(acc[j][1][0] * m4[0], acc[j][0][0]),
               gate_mul(acc[j][1][1] * m4[1], acc[j][0][1]),
               gate_mul(acc[j][1][2] * m4[2], acc[j][0][2]),
               gate_mul(acc[j][1][3] * m4[3], acc[j][0][3]));
    };
    static_assert(TP == 64, "four row tiles per tile");
    if (__all(mv[lane] == 0.f)) {  // whole tile padded: zeros, no MFMA (wave-uniform)
#pragma unroll
      for (int rt = 0; rt < TP / 16; ++rt) {
        T* const srow = stg + (lane & 15) * SROW + rt * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < UPW; ++j) store4(srow + j * 16 * SROW, 0.f, 0.f, 0.f, 0.f);
      }
    } else {
      f32x4 acc0[UPW][2], acc1[UPW][2];
      mma_rt(0, acc0);
      mma_rt(1, acc1);
      epi_rt(0, acc0);
      mma_rt(2, acc0);
      epi_rt(1, acc1);
      mma_rt(3, acc1);
      epi_rt(2, acc0);
      epi_rt(3, acc1);
    }
    pend = cur_c;
    if (nbuf == 1) __syncthreads();  // every wave is done reading the single z buffer
    stage(nbuf == 2 ? cur ^ 1 : 0, pre);
    __syncthreads();
    cur_c = next_c;
  }
  store_tile(pend);
}

// ---------------------------------------------------------------------------------------
// Wave-independent form for c_z of four chunk groups (97..128 channels in bf16, 49..64 in
// fp32: sixteen 16-byte chunks per weight row). A workgroup of 8 waves copies the
// gate/projection rows of its group of units (a unit = 16 channels of a or b) into LDS
// once; then every wave runs its own loop over 64-pair tiles (one storage row, 64
// consecutive columns) with no workgroup barrier:
//   - z comes straight from global memory into MFMA operand layout and is normalised in
//     registers. Row i of the A operand of subtile st (st = 0..3) holds pair
//     16*(i/4) + 4*st + i%4 of the tile, so that accumulator register rr of lane
//     (p, q) = (lane%16, lane/16) is pair 16q + 4st + rr, channel p: across the subtiles a
//     lane holds 16 consecutive pairs of one channel and writes them as whole 16-byte
//     pieces of the [c][Np][Np] operand, with no staging;
//   - per unit, the gate and projection rows (the B operand) come from LDS and the start
//     vectors initialise the accumulators; the epilogue is m * p / (1 + 2^g);
//   - units go two at a time through a software pipeline: the MFMAs of one unit are
//     issued alongside the epilogue of the previous one.
// In LDS a weight row is sixteen chunks with chunk c at position c ^ (row & 15), which
// keeps the reads free of bank conflicts without padding.
// Cache policy of the bf16 output stores: device scope (sc1). Each store instruction
// writes whole 128-byte lines, so the lines go through this XCD's L2 to memory as they are
// produced instead of waiting, dirty, for the end-of-kernel release (K1 51.2 against 53.8
// us at N = 512 with the default policy; with half-lines per instruction, as before the
// lane exchange, written-through stores took 78 us).
constexpr int K1_STORE_POLICY = 0x10;

// Issue priority from a wave's progress (level = half tiles done): the wave of a SIMD that
// is behind issues first, so the two waves sharing a SIMD finish together instead of the
// younger one running alone at the end.
__device__ __forceinline__ void progress_priority(int level) {
  if (level <= 0) __builtin_amdgcn_s_setprio(3);
  else if (level == 1) __builtin_amdgcn_s_setprio(2);
  else if (level == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// XM: 0 without mask extents; 1 with extents, every tile visited and the ones outside
// skipped; 2 with extents and the compact list of the tiles inside them. (A template
// parameter, so the plain form carries none of the extent bookkeeping in registers.)
template <class T, int XM>
__global__ __launch_bounds__(K1W_THREADS) void k1_input_gate_waves(
    const T* __restrict__ z, const T* __restrict__ mask, T* __restrict__ a_out,
    T* __restrict__ b_out, const chunk_t* __restrict__ image, int n, int np, int cz, int c,
    int incoming, int mask_all, int ug, int total_tiles, const int* __restrict__ extents) {
  constexpr bool compact = XM == 2;
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int KZ = 4;               // chunk groups along c_z
  constexpr int RC = KZ * KG / E;     // 16 chunks per weight row
  constexpr int ST = K1W_TP / 16;     // 16-pair subtiles per tile
  constexpr int NOUT = 16 / E;        // 16-byte stores per lane and unit (16 pairs)
  static_assert(RC == 16, "chunk count the swizzle assumes");
  static_assert(KZ * KG * sizeof(T) == K1W_ROW_BYTES, "row size of the weight image");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int czp = KZ * KG;
  const int rows = ug * 32;  // gate and projection rows of this group's units
  T* const wl = (T*)smem;                                 // [rows][czp], swizzled chunks
  float* const tl = (float*)(wl + (size_t)rows * czp);    // [rows]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* const mb = tl + rows + wave * K1W_TP;            // per-wave tile masks [64]
  const int p = lane & 15, q = lane >> 4;
  const int cblocks = c / 16;
  const int u0 = blockIdx.y * ug;  // first unit of this group
  const size_t plane = (size_t)np * np;
  const int ntx = np / K1W_TP;
  const int arow = 16 * (p >> 2) + (p & 3);  // tile pair of A row p in subtile 0 (+4 per st)

  // tile t -> (bb, r, sx): storage row r, columns sx*64 .. +63; the z pairs are (r, s)
  // outgoing and (s, r) incoming. With `compact` (mask extents, few items) the tiles are
  // those inside each item's extent only, so every wave gets an equal share of the work
  // that is left.
  ActiveTiles sched;
  if constexpr (compact) {
    sched.init(extents, n, total_tiles / (np * ntx), K1W_TP);
    total_tiles = sched.total();
    if (total_tiles == 0) return;  // workgroup-uniform: no item has a valid pair
  }
  auto coords = [&](int t, int& bb, int& r, int& s0) {
    if constexpr (compact) {
      sched.at(t, bb, r, s0);
      return;
    }
    bb = t / (np * ntx);
    const int rem = t - bb * np * ntx;
    r = rem / ntx;
    s0 = (rem - r * ntx) * K1W_TP;
  };
  struct Pre {
    chunk_t zv[ST][KZ];
    T m[ST];
  };
  // Buffer loads: per subtile a scalar base (its first pair) and an extent ending at the
  // last real pair of its storage row; per lane a byte offset that is the same in every
  // tile (consecutive pairs of a tile are 1 (outgoing) or n (incoming) pairs apart). The
  // bounds check covers the lane and immediate offsets only, so each subtile gets its own
  // resource rather than a scalar offset. Pairs past the extent, and whole tiles in
  // padding rows, read as zero.
  const size_t pstride = incoming ? (size_t)n : 1;  // pairs between consecutive columns
  // lane offsets: pair arow of the subtile, chunk q of the first chunk group; subtile st
  // starts 4 * st columns on, chunk group ks adds the immediate ks * KG elements
  const unsigned int zoff = (unsigned int)(((size_t)arow * pstride * cz + q * E) * sizeof(T));
  const unsigned int moff = mask_all ? 0u : (unsigned int)((size_t)arow * pstride * sizeof(T));
  // byte sizes below 2^31: this form runs only where one batch item of z is under 2 GiB
  const unsigned int zstep = (unsigned int)(4 * pstride * cz * sizeof(T));
  const unsigned int mstep = (unsigned int)(4 * pstride * sizeof(T));
  // With mask extents, a tile outside its item's leading L x L square is inactive: its
  // loads read nothing (zero extents), it writes nothing (the contraction reads no operand
  // row or column past L), and the pairs of an active tile past L count as masked.
  ExtentCache ecache;
  auto fetch = [&](int t, Pre& f) {
    int bb, r, s0;
    coords(t < total_tiles ? t : total_tiles - 1, bb, r, s0);  // waves past the end refetch
    const int lim = XM ? item_bound(extents, bb, n, ecache) : n;
    const bool row_ok = r < lim && s0 < lim;
    const size_t p0 = row_ok ? (incoming ? ((size_t)bb * n + s0) * n + r : ((size_t)bb * n + r) * n + s0) : 0;
    // pairs of the storage row from the tile's first one to the last real one
    const unsigned int span = row_ok ? (unsigned int)(lim - s0 - 1) * (unsigned int)pstride + 1 : 0u;
    const unsigned int zext = span * (unsigned int)(cz * sizeof(T));
    const unsigned int mext = span * (unsigned int)sizeof(T);
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const unsigned int zs = st * zstep, ms = st * mstep;
      const __amdgpu_buffer_rsrc_t rz =
          buffer_rsrc_u32((const unsigned char*)(z + p0 * cz) + zs, bytes_after(zext, zs));
      const __amdgpu_buffer_rsrc_t rm =
          mask_all ? buffer_rsrc_u32(mask, sizeof(T))
                   : buffer_rsrc_u32((const unsigned char*)(mask + p0) + ms, bytes_after(mext, ms));
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks)
        f.zv[st][ks] = load16(rz, zoff + ks * KG * (unsigned int)sizeof(T), 0);
      f.m[st] = load_elem(rm, moff, 0, T());
    }
  };

  const int gw = blockIdx.x * K1W_WAVES + wave;
  const int nw = gridDim.x * K1W_WAVES;
  // this lane's output offset from its unit's row block at the tile's first pair: bf16,
  // in bytes, channel p % 8, pairs 16q + 8 (p / 8) (the second store 8 channels on, hofs
  // bytes further); fp32, in elements, channel p, pairs 16q. Both below 2^32: one batch
  // item of z is under 2 GiB.
  const unsigned int lofs =
      sizeof(T) == 2 ? (unsigned int)((((size_t)(p & 7)) * plane + 16 * q + 8 * (p >> 3)) * 2)
                     : (unsigned int)((size_t)p * plane + 16 * q);
  const unsigned int hofs = (unsigned int)(8 * plane * sizeof(T));
  Pre f;
  // ---- the group's weights -> LDS. The handle keeps each group's weights as the LDS
  // image itself (swizzled rows, then their start values), so the copy is flat: each
  // thread has up to 16 of its 16-byte chunks in flight before it stores any. The first
  // tile's z loads go out after the first weight loads (loads retire in order, and the
  // weights are needed first) and land while the weights are stored. ----
  {
    const int chunks = (int)(k1w_image_bytes(ug) / 16);
    const chunk_t* const src = image + (size_t)blockIdx.y * chunks;
    copy_image<K1W_THREADS>(src, (chunk_t*)smem, chunks, tid, [&]() { fetch(gw, f); });
  }
  __syncthreads();

  typedef chunk_t WUnit[2][KZ];  // gate and projection chunks of one unit
  typedef f32x4 AUnit[ST][2];    // gate and projection accumulators of one unit


  // Tile t's fetched z -> normalised A operand in za; masks -> m4 (lane (p, q): pairs
  // 16q + 4st + rr). Pairs outside n x n become zero rows with mask 0 (branch-free). The
  // pass runs at the end of the previous tile, right after the fetch and the last stores,
  // so its waits count only those.
  chunk_t za[ST][KZ];
  f32x4 m4[ST];
  bool ones = false;   // every mask value of the tile is 1 (wave-uniform)
  bool zeros = false;  // every mask value of the tile is 0: its outputs are zero
  auto prepare = [&](int t) {
    int bb, r, s0;
    coords(t < total_tiles ? t : total_tiles - 1, bb, r, s0);
    const int lim = XM ? item_bound(extents, bb, n, ecache) : n;
    int opaque;  // keeps the loop-invariant masks inside the loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
    float mv[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const unsigned int okm = 0u - (unsigned int)(r < lim && s0 + arow + 4 * st < lim);
      mv[st] = __uint_as_float(__float_as_uint(to_f32(f.m[st])) & okm);
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) {
        const unsigned int keep = 0u - (unsigned int)(ks * KG + q * E + opaque < cz);
        za[st][ks] = f.zv[st][ks] & (okm & keep);
      }
    }
    // A row p of subtile st -> mb[st*16 + p] (lanes of equal p write equal values), read
    // back as the four pairs 16q + 4st + 0..3 = A rows 4q..4q+3
#pragma unroll
    for (int st = 0; st < ST; ++st) mb[st * 16 + p] = mv[st];
    ones = __all(mv[0] == 1.f && mv[1] == 1.f && mv[2] == 1.f && mv[3] == 1.f);
    zeros = __all(mv[0] == 0.f && mv[1] == 0.f && mv[2] == 0.f && mv[3] == 0.f);
    wave_lds_sync();
#pragma unroll
    for (int st = 0; st < ST; ++st) m4[st] = ld16f(mb + st * 16 + 4 * q);
#pragma unroll
    for (int st = 0; st < ST; ++st) normalize_operand_row<KZ>(za[st], cz, lane, T());
  };

  prepare(gw);
  int done = 0;  // tiles this wave has finished
  for (int t = gw; t < total_tiles; t += nw) {
    int bb, r, s0;
    coords(t, bb, r, s0);
    int opaque;  // keeps the loop-invariant LDS reads inside the loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
    // the tile's first pair in channel 0 (wave-uniform; the unit's channel block is added
    // per unit, the lane's channel and pairs in store16)
    const size_t tbase = (size_t)bb * c * plane + (size_t)r * np + s0;
    const T* const wlt = wl + opaque;
    const float* const tlt = tl + opaque;

    // unit uu's weights (B operand) and start values from LDS
    auto load_w = [&](int uu, WUnit& w, float (&bias)[2]) {
      const int lr0 = uu * 32 + p;  // gate row; the projection row is 16 further
      bias[0] = tlt[lr0];
      bias[1] = tlt[lr0 + 16];
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) {
        const int pos = ((ks * 4 + q) ^ p) * E;
        w[0][ks] = ld16(wlt + lr0 * czp + pos);
        w[1][ks] = ld16(wlt + (lr0 + 16) * czp + pos);
      }
    };
    auto mma_unit = [&](const WUnit& w, const float (&bias)[2], AUnit& acc) {
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        acc[st][0] = f32x4{bias[0], bias[0], bias[0], bias[0]};
        acc[st][1] = f32x4{bias[1], bias[1], bias[1], bias[1]};
      }
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks)
#pragma unroll
        for (int st = 0; st < ST; ++st) {
          acc[st][0] = mma16(acc[st][0], za[st][ks], w[0][ks], T());
          acc[st][1] = mma16(acc[st][1], za[st][ks], w[1][ks], T());
        }
    };
    // output row block of unit uu: channel rows ucb .. ucb+15 of a or b
    auto unit_dst = [&](int uu) {
      const int u = u0 + uu;
      const bool isb = u >= cblocks;  // units 0 .. c/16-1 are a, the rest b
      return (isb ? b_out : a_out) + tbase + (size_t)((isb ? u - cblocks : u) * 16) * plane;
    };
    // 16 outputs (pairs 16q .. 16q+15 of channel p) of the unit whose row block starts at
    // ub. bf16: lanes p and p + 8 of a row swap a chunk, so that each of the two stores
    // writes whole 128-byte lines: the first holds channel p % 8 (pairs 16q .. +7 from
    // lanes p < 8, 16q + 8 .. +15 from lanes p >= 8), the second channel p % 8 + 8.
    // fp32: four 16-byte stores of the lane's own pairs.
    auto store16 = [&](T* ub, const float (&o)[16]) {
      T ot[16];
#pragma unroll
      for (int j = 0; j < 16; j += 4) store4(ot + j, o[j], o[j + 1], o[j + 2], o[j + 3]);
      if constexpr (sizeof(T) == 2) {
        const chunk_t c0 = ld16(ot), c1 = ld16(ot + 8);
        chunk_t lo, hi;
        constexpr int kRowRor8 = 0x128;  // DPP: lane i of a row of 16 reads lane i ^ 8
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // lanes p >= 8 (banks 2, 3) take chunk 1 of lane p - 8; lanes p < 8 chunk 0 of p + 8
          lo[d] = (unsigned int)__builtin_amdgcn_update_dpp((int)c0[d], (int)c1[d], kRowRor8, 0xf, 0xc, false);
          hi[d] = (unsigned int)__builtin_amdgcn_update_dpp((int)c1[d], (int)c0[d], kRowRor8, 0xf, 0x3, false);
        }
        const __amdgpu_buffer_rsrc_t rd = buffer_rsrc_u32(ub, 0xffffffffu);
        typedef __attribute__((ext_vector_type(4))) int i32x4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, lo), rd, (int)lofs, 0, K1_STORE_POLICY);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, hi), rd, (int)(lofs + hofs), 0, K1_STORE_POLICY);
      } else {
        T* const dst = ub + lofs;
#pragma unroll
        for (int k = 0; k < NOUT; ++k) st16(dst + k * E, ld16(ot + k * E));
      }
    };
    // m * p / (1 + 2^g) of one unit, on its own (the last unit of a tile)
    auto emit = [&](T* dst, const AUnit& acc, auto masked) {
      float o[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pm = masked ? acc[j >> 2][1][j & 3] * m4[j >> 2][j & 3] : acc[j >> 2][1][j & 3];
        o[j] = gate_mul(pm, acc[j >> 2][0][j & 3]);
      }
      store16(dst, o);
    };
    // One pipeline step, scheduled by hand: the 32 MFMAs of a unit (weights w, start values
    // bias -> acc), each followed by two or three VALU instructions of the previous unit's
    // epilogue (old -> dst), so that matrix and vector work issue side by side from one
    // wave; the next unit's weights are read from LDS in the first slots. The epilogue of
    // value v (pair 16q + v) runs as a five-stage pipeline over the slots -- exp2 and p*m in
    // slot 2v, +1 in slot 2v+1, the reciprocal in slot 2v+2, the product in slot 2v+5 --
    // so no instruction of a slot waits on another of the same slot.
    auto step = [&](const WUnit& w, const float (&bias)[2], AUnit& acc, const AUnit& old,
                    T* dst, bool load_next, int next_uu, WUnit& wn, float (&bn)[2],
                    auto masked) {
      const f32x4 bg = {bias[0], bias[0], bias[0], bias[0]};
      const f32x4 bp = {bias[1], bias[1], bias[1], bias[1]};
      float e[16], a[16], d[16], r[16], o[16];
      const int lr0 = next_uu * 32 + p;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int ks = k >> 3, st = (k >> 1) & 3, gp = k & 1;
        acc[st][gp] = mma16(ks == 0 ? (gp ? bp : bg) : acc[st][gp], za[st][ks], w[gp][ks], T());
        if (load_next && k < 8) {
          const int nks = k >> 1, ngp = k & 1;
          wn[ngp][nks] = ld16(wlt + (lr0 + 16 * ngp) * czp + (((nks * 4 + q) ^ p) * E));
          if (k == 7) {
            bn[0] = tlt[lr0];
            bn[1] = tlt[lr0 + 16];
          }
        }
        const int v = k >> 1;
        // the empty volatile statements pin each slot's results in program order
        if ((k & 1) == 0) {
          e[v] = __builtin_amdgcn_exp2f(old[v >> 2][0][v & 3]);
          a[v] = masked ? old[v >> 2][1][v & 3] * m4[v >> 2][v & 3] : old[v >> 2][1][v & 3];
          if (v >= 1) {
            r[v - 1] = __builtin_amdgcn_rcpf(d[v - 1]);
            asm volatile("" : "+v"(acc[st][gp]), "+v"(e[v]), "+v"(a[v]), "+v"(r[v - 1]));
          } else {
            asm volatile("" : "+v"(acc[st][gp]), "+v"(e[v]), "+v"(a[v]));
          }
        } else {
          d[v] = 1.0f + e[v];
          if (v >= 2) {
            o[v - 2] = a[v - 2] * r[v - 2];
            asm volatile("" : "+v"(acc[st][gp]), "+v"(d[v]), "+v"(o[v - 2]));
          } else {
            asm volatile("" : "+v"(acc[st][gp]), "+v"(d[v]));
          }
        }
      }
      r[15] = __builtin_amdgcn_rcpf(d[15]);
      o[14] = a[14] * r[14];
      o[15] = a[15] * r[15];
      store16(dst, o);
    };

    // Software pipeline over the group's units, two at a time (ug is even). Tiles whose
    // mask is all ones skip the multiply by m.
    auto run_units = [&](auto masked) {
      progress_priority(2 * done);
      WUnit wa, wb;
      float ba[2], bbias[2];
      AUnit acca, accb;
      load_w(0, wa, ba);
      mma_unit(wa, ba, acca);
      load_w(1, wb, bbias);
#pragma unroll 1
      for (int uu = 0; uu + 2 < ug; uu += 2) {
        step(wb, bbias, accb, acca, unit_dst(uu), true, uu + 2, wa, ba, masked);      // MFMA uu+1
        step(wa, ba, acca, accb, unit_dst(uu + 1), true, uu + 3, wb, bbias, masked);  // MFMA uu+2
        if (2 * (uu + 2) == ug) progress_priority(2 * done + 1);
      }
      step(wb, bbias, accb, acca, unit_dst(ug - 2), false, 0, wa, ba, masked);        // MFMA ug-1
      fetch(t + nw, f);  // za is dead: the next tile's z loads go out now
      emit(unit_dst(ug - 1), accb, masked);
    };
    const int lim = XM ? item_bound(extents, bb, n, ecache) : n;
    if (XM && !(r < lim && s0 < lim)) {
      fetch(t + nw, f);  // inactive (outside the item's extent): nothing to compute or write
    } else if (zeros) {
      // a tile wholly outside the mask: no MFMA and no epilogue, its unit rows are zeros
      fetch(t + nw, f);
      const float zo[16] = {};
#pragma unroll 1
      for (int uu = 0; uu < ug; ++uu) store16(unit_dst(uu), zo);
    } else if (ones) {
      run_units(std::false_type{});
    } else {
      run_units(std::true_type{});
    }
    prepare(t + nw);
    ++done;
  }
}

// Launches the wave-independent form if the units split into groups that fit LDS;
// *done = false leaves the launch to the tile-shared form.
template <class T, int XM>
static hipError_t launch_k1w_x(const StageArgs& a, hipStream_t st, int ug, int total) {
  const size_t lds = k1w_lds_bytes(ug);
  auto fn = k1_input_gate_waves<T, XM>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const int groups = 2 * (a.c / 16) / ug;
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, K1W_THREADS, lds, occ, occ_lds);
  const int cap = a.num_cus * per_cu / groups > 0 ? a.num_cus * per_cu / groups : 1;
  const int need = (total + K1W_WAVES - 1) / K1W_WAVES;
  const int blocks = need < cap ? need : cap;
  const int mask_all = a.mask == nullptr;
  hipLaunchKernelGGL(fn, dim3(blocks, groups), dim3(K1W_THREADS), lds, st, (const T*)a.z,
                     (const T*)(mask_all ? a.one : a.mask), (T*)a.a, (T*)a.b,
                     (const chunk_t*)a.k1w_image, a.n, a.np, a.cz, a.c, a.incoming, mask_all, ug,
                     total, a.extents);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_k1w(const StageArgs& a, hipStream_t st, bool* done) {
  *done = false;
  // the per-lane z offsets are 32-bit byte offsets within one batch item's z
  if ((size_t)a.n * a.n * a.cz * sizeof(T) >= 0x80000000ull) return hipSuccess;
  // the handle's weight images are built for this group size (units go in pairs)
  const int units = 2 * (a.c / 16);
  const int ug = a.k1w_image ? k1w_group_units(a.c) : 0;
  if (ug == 0) return hipSuccess;
  // each wave pays the weight copy and its first tile's loads up front: with fewer than
  // two tiles per wave of a full grid the tile-shared form is faster
  const int total = a.batch * a.np * (a.np / K1W_TP);
  if (total < 2 * a.num_cus * K1W_WAVES) return hipSuccess;
  if (a.plan) {
    a.plan->k1_form = 0;
    *done = true;
    return hipSuccess;
  }
  (void)units;
  *done = true;
  if (!a.extents) return launch_k1w_x<T, 0>(a, st, ug, total);
  if (a.batch <= COMPACT_MAX_ITEMS) return launch_k1w_x<T, 2>(a, st, ug, total);
  return launch_k1w_x<T, 1>(a, st, ug, total);
}

// ---------------------------------------------------------------------------------------

template <class T, int KMAX, int UPW, int W>
static hipError_t launch_k1_t(const StageArgs& a, hipStream_t st) {
  if (a.plan) {
    a.plan->k1_form = 1;
    return hipSuccess;
  }
  constexpr int E = Traits<T>::E;
  auto lds_for = [&](int nb) {
    return nb * ((size_t)K1_TP * (a.czp + E) * sizeof(T) + K1_TP * sizeof(float)) +
           (size_t)W * UPW * 16 * (K1_TP + 4) * sizeof(T);
  };
  const int nbuf = lds_for(2) <= LDS_PER_CU ? 2 : 1;
  const size_t lds = lds_for(nbuf);
  auto fn = k1_input_gate<T, KMAX, UPW, W>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const int units = 2 * (a.c / 16);
  const int groups = (units + W * UPW - 1) / (W * UPW);
  const int total = a.batch * a.np * (a.np / K1_TP);
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, 64 * W, lds, occ, occ_lds);
  const int cap = a.num_cus * per_cu / groups > 0 ? a.num_cus * per_cu / groups : 1;
  const int blocks = total < cap ? total : cap;
  const int mask_all = a.mask == nullptr;
  hipLaunchKernelGGL(fn, dim3(blocks, groups), dim3(64 * W), lds, st, (const T*)a.z,
                     (const T*)(mask_all ? a.one : a.mask), (T*)a.a, (T*)a.b, (const T*)a.w1, a.t1,
                     a.n, a.np, a.cz, a.czp, a.c, a.incoming, mask_all, nbuf, total);
  return hipGetLastError();
}

// Units per wave: as many as the register budget allows for the k extent (the weights of
// one unit take 8 * KMAX registers).
template <class T>
static hipError_t launch_k1_dispatch(const StageArgs& a, hipStream_t st) {
  switch (a.czp / Traits<T>::KG) {
    case 1: return launch_k1_t<T, 1, 2, 8>(a, st);
    case 2: return launch_k1_t<T, 2, 2, 8>(a, st);
    case 4: {
      bool done = false;
      hipError_t e = launch_k1w<T>(a, st, &done);
      if (e != hipSuccess || done) return e;
      return launch_k1_t<T, 4, 1, 16>(a, st);
    }
    case 8: return launch_k1_t<T, 8, 1, 8>(a, st);
    case 12: return launch_k1_t<T, 12, 1, 8>(a, st);
    case 16: return launch_k1_t<T, 16, 1, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_k1(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  return bf16_storage ? launch_k1_dispatch<bf16>(a, st) : launch_k1_dispatch<float>(a, st);
}

}  // namespace trimul
