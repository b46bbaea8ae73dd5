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

#include "device_common.h"

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

template <class T, int KMAX, int UPW, int W>
static hipError_t launch_k1_t(const StageArgs& a, hipStream_t st) {
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
    case 4: return launch_k1_t<T, 4, 1, 16>(a, st);
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
