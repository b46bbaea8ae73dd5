// k3: output LayerNorm over c + projection c -> c_z + output gate from the re-normalised
// z + pair mask -> out [B][N][N][c_z].
//
// RFProteína architecture page, "Triangle multiplication on SM90" (K3: the output gate
// and projection with both LayerNorms) and "Dual-GEMM gates" (x0_x1 form
// sigma(x0 W_g^T + b_g) * (x1 W_p^T + b_p) with x0 the normalised input pair tensor and
// x1 the contracted hidden tensor).
//
// The k extents are compile-time constants: the host pads c and c_z to exactly KXM / KZM
// chunk groups.
// Work split (persistent): a tile is TP = 64 consecutive pairs (i, j0 .. j0+63) of one row
// i. Per tile the workgroup stages x (read channel-major, transposed on the way in
// through registers) and z in LDS and normalises both rows in place; then each of the 4
// waves computes UPW=2 units of 16 output channels for the 64 pairs with the weights of its
// units held in registers (W_o as A operand against xhat, W_g against zhat). Biases and
// beta terms start the accumulators; the gate rows carry -log2(e) (host side). The next
// tile's x and z are fetched into registers while the current tile's MFMAs run.

#include <type_traits>

#include "device_common.h"

namespace trimul {


constexpr int K3_TP = 64;
constexpr int K3_WAVES = 4;
constexpr int K3_THREADS = 64 * K3_WAVES;
constexpr int K3_TPP = K3_THREADS / K3_TP;  // threads per pair when staging a tile
constexpr int K3_UPW = 2;                   // 16-channel output units per wave
constexpr size_t K3_LDS_BUDGET = 80 * 1024;  // double-buffer only while two workgroups fit a CU

template <class T, int KXM, int KZM, int XB, bool RESID>
__global__ __launch_bounds__(K3_THREADS) void k3_output_gate(
    const T* __restrict__ x, ZIn<T, RESID> z, const T* __restrict__ mask, ZOut<T, RESID> out,
    const T* __restrict__ wo, const float* __restrict__ to,
    const T* __restrict__ wg, const float* __restrict__ tg, int n, int np, int cz, int czp, int c,
    int cp, int mask_all, int nbuf, int total_tiles) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int TP = K3_TP;
  constexpr int KMAX = KXM > KZM ? KXM : KZM;
  constexpr int TPP = K3_TPP;
  constexpr int UPW = K3_UPW;
  constexpr int NCH = (KMAX * KG / E + TPP - 1) / TPP;  // chunks per thread of one LDS row
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int xstride = cp + E, zstride = czp + E;
  // LDS: x tiles [nbuf][TP][xstride], z tiles [nbuf][TP][zstride], masks [nbuf][TP].
  // nbuf = 2 double-buffers the staging; wide widths that do not fit use one buffer and an
  // extra barrier per tile.
  T* const xbase = (T*)smem;
  T* const zbase = xbase + nbuf * TP * xstride;
  float* const mvbuf = (float*)(zbase + nbuf * TP * zstride);
  auto xbuf = [&](int b) { return xbase + b * TP * xstride; };
  auto zbuf = [&](int b) { return zbase + b * TP * zstride; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int units = cz / 16;
  const int ntx = (n + TP - 1) / TP;

  // ---- this wave's units: 16 output channels each, weights in registers ----
  chunk_t wor[UPW][KXM], wgr[UPW][KZM];
  f32x4 bo[UPW], bg[UPW];
  bool uok[UPW];
  int oc0[UPW];  // accumulator register rr <-> output channel oc0 + rr
#pragma unroll
  for (int jj = 0; jj < UPW; ++jj) {
    const int u = blockIdx.y * (K3_WAVES * UPW) + wave + K3_WAVES * jj;
    uok[jj] = u < units;
    const int orow = uok[jj] ? u * 16 + (lane & 15) : 0;  // A-operand row this lane hands in
#pragma unroll
    for (int ks = 0; ks < KXM; ++ks)
      wor[jj][ks] = uok[jj] ? ld16(wo + (size_t)orow * cp + ks * KG + (lane >> 4) * E)
                            : chunk_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < KZM; ++ks)
      wgr[jj][ks] = uok[jj] ? ld16(wg + (size_t)orow * czp + ks * KG + (lane >> 4) * E)
                            : chunk_t{0u, 0u, 0u, 0u};
    oc0[jj] = uok[jj] ? u * 16 + 4 * (lane >> 4) : 0;
    bo[jj] = uok[jj] ? ld16f(to + oc0[jj]) : f32x4{0.f, 0.f, 0.f, 0.f};
    bg[jj] = uok[jj] ? ld16f(tg + oc0[jj]) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging maps ----
  // x: the (c/E)*(TP/E) blocks of E channels x E pairs are moved through registers, XB
  // per thread (block tid + k*THREADS); the channel block varies fastest across lanes so
  // that the transposed LDS writes of neighbouring lanes land in different banks.
  const int cbn = c / E;
  const int xblocks = cbn * (TP / E);
  // z and the row normalisation: thread (t, part) owns chunks part, part+TPP, ... of pair t
  const int t = tid / TPP, part = tid % TPP;
  const int czc = cz / E, ccz = czp / E, cxc = c / E, ccx = cp / E;

  auto tile_coords = [&](int tile, int& bb, int& i, int& j0) {
    bb = tile / (n * ntx);
    const int rem = tile - bb * n * ntx;
    i = rem / ntx;
    j0 = (rem - i * ntx) * TP;
  };
  // The next tile is fetched into registers with unconditional loads from clamped,
  // in-bounds addresses (no branches); every select that depends on loaded data happens in
  // stage(), after the current tile's MFMAs, so the loads stay in flight meanwhile.
  // `mask_all` (no mask given) reads the one-valued element at mask[0].
  struct Pre {
    chunk_t xv[XB][E];
    chunk_t zv[NCH];
    T m;
    bool valid;
  };
  auto fetch = [&](int tile, Pre& f) {
    int bb, i, j0;
    tile_coords(tile, bb, i, j0);
#pragma unroll
    for (int k = 0; k < XB; ++k) {
      const int blk = tid + k * K3_THREADS;
      const int bl = blk < xblocks ? blk : 0;
      const int pb = bl / cbn, cb = bl - pb * cbn;
      const T* src = x + (((size_t)bb * c + cb * E) * np + i) * np + j0 + pb * E;
#pragma unroll
      for (int e = 0; e < E; ++e) f.xv[k][e] = ld16(src + (size_t)e * np * np);
    }
    const int j = j0 + t;
    f.valid = j < n;
    const size_t pair = f.valid ? ((size_t)bb * n + i) * n + j : 0;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = part + TPP * q;
      f.zv[q] = ld16(z + pair * cz + (ch < czc ? ch : 0) * E);
    }
    f.m = mask[mask_all ? 0 : pair];
  };
  // writes the fetched tile into LDS buffer `buf`; z rows normalised on the way
  auto stage = [&](int buf, Pre& f) {
#pragma unroll
    for (int k = 0; k < XB; ++k) {
      const int blk = tid + k * K3_THREADS;
      if (blk < xblocks) {
        const int pb = blk / cbn, cb = blk - pb * cbn;
        T tb[E][E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const T* pv = (const T*)&f.xv[k][e];
#pragma unroll
          for (int ff = 0; ff < E; ++ff) tb[e][ff] = pv[ff];
        }
#pragma unroll
        for (int ff = 0; ff < E; ++ff) {
          T col[E];
#pragma unroll
          for (int e = 0; e < E; ++e) col[e] = tb[e][ff];
          st16(xbuf(buf) + (pb * E + ff) * xstride + cb * E, __builtin_bit_cast(chunk_t, col));
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NCH; ++q)
      if (!(f.valid && part + TPP * q < czc)) f.zv[q] = chunk_t{0u, 0u, 0u, 0u};
    normalize_row<T, NCH, TPP>(f.zv, part, czc, cz);
    T* zrow = zbuf(buf) + t * zstride;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = part + TPP * q;
      if (ch < ccz) st16(zrow + ch * E, f.zv[q]);
    }
    if (part == 0) mvbuf[buf * TP + t] = f.valid ? to_f32(f.m) : 0.f;
  };
  // normalises the x rows of buffer `buf` in place (after the transposed writes landed)
  auto norm_x = [&](int buf) {
    T* xrow = xbuf(buf) + t * xstride;
    chunk_t v[NCH];
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = part + TPP * q;
      v[q] = ch < cxc ? ld16(xrow + ch * E) : chunk_t{0u, 0u, 0u, 0u};
    }
    normalize_row<T, NCH, TPP>(v, part, cxc, c);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = part + TPP * q;
      if (ch < ccx) st16(xrow + ch * E, v[q]);
    }
  };

  int tile = blockIdx.x;  // the grid never exceeds the tile count
  {
    Pre f;
    fetch(tile, f);
    stage(0, f);
  }
  __syncthreads();
  norm_x(0);
  __syncthreads();

  for (int it = 0; tile < total_tiles; tile += gridDim.x, ++it) {
    const int cur = nbuf == 2 ? (it & 1) : 0;
    const int nxt = nbuf == 2 ? (cur ^ 1) : 0;
    const int next = tile + gridDim.x;
    Pre pre;
    fetch(next < total_tiles ? next : tile, pre);  // the last iteration refetches, unused

    int bb, i, j0;
    tile_coords(tile, bb, i, j0);
    const T* xs = xbuf(cur);
    const T* zs = zbuf(cur);
    const float* mv = mvbuf + cur * TP;
    // a tile wholly outside the mask runs no MFMA: with m = 0 the finite start values give
    // a zero update (its x is never read)
    static_assert(TP == 64, "one mask value per lane");
    const bool skip = __all(mv[lane] == 0.f);
#pragma unroll
    for (int pt = 0; pt < TP / 16; ++pt) {
      f32x4 ap[UPW], ag[UPW];
#pragma unroll
      for (int jj = 0; jj < UPW; ++jj) {
        ap[jj] = bo[jj];
        ag[jj] = bg[jj];
      }
      const int pr = pt * 16 + (lane & 15);  // B-operand column = pair
      const T* xr = xs + pr * xstride + (lane >> 4) * E;
      const T* zr = zs + pr * zstride + (lane >> 4) * E;
      if (!skip) {
#pragma unroll
        for (int ks = 0; ks < KXM; ++ks) {
          const chunk_t xf = ld16(xr + ks * KG);
#pragma unroll
          for (int jj = 0; jj < UPW; ++jj) ap[jj] = mma16(ap[jj], wor[jj][ks], xf, T());
        }
#pragma unroll
        for (int ks = 0; ks < KZM; ++ks) {
          const chunk_t zf = ld16(zr + ks * KG);
#pragma unroll
          for (int jj = 0; jj < UPW; ++jj) ag[jj] = mma16(ag[jj], wgr[jj][ks], zf, T());
        }
      }
      const int j = j0 + pr;
      const float m = mv[pr];
#pragma unroll
      for (int jj = 0; jj < UPW; ++jj) {
        if (uok[jj] && j < n) {
          const size_t off = (((size_t)bb * n + i) * n + j) * cz + oc0[jj];
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = gate_mul(ap[jj][r] * m, ag[jj][r]);
          if constexpr (RESID) add4(o4, z + off);  // out = z + update (out may be z)
          store4(out + off, o4[0], o4[1], o4[2], o4[3]);
        }
      }
    }
    if (nbuf == 1) __syncthreads();  // every wave is done reading the single buffer
    stage(nxt, pre);
    __syncthreads();
    norm_x(nxt);
    __syncthreads();
  }
}

// A 16-byte store through a resource on a wave-uniform base (32-bit lane offsets instead
// of 64-bit addresses), non-temporal (cache policy nt). The scalar offset stays 0.
constexpr int K3_STORE_POLICY = 0x2;
__device__ __forceinline__ void k3_store16(__amdgpu_buffer_rsrc_t r, chunk_t v, unsigned int voff) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)voff, 0, K3_STORE_POLICY);
}

// ---------------------------------------------------------------------------------------
// Wave-independent form (used whenever the weight slice and the per-wave staging fit
// LDS). Workgroup = 8 waves; blockIdx.y selects a group of `ug` output units (16 output
// channels each) whose W_o and W_g rows and start vectors are copied into LDS once. Every
// wave then runs its own persistent loop over wave tiles of TW = 16*ST consecutive pairs
// (i, j0 .. j0+TW-1), with no workgroup barrier:
//   - x arrives channel-major; E x E blocks (E channels x E pairs, one 16-byte load per
//     channel) are transposed in registers and written pair-major into the wave's LDS
//     staging rows, then read back in MFMA operand layout; z is loaded straight from
//     global memory in operand layout (lane (p, q) = (lane%16, lane/16) holds elements
//     ks*KG + q*E .. of pair p);
//   - both LayerNorms run on the operand registers (the four lanes of a pair reduce
//     through the lane permute network);
//   - per unit: W_o / W_g rows from LDS are the A operand, xhat / zhat the B operand, the
//     start vectors initialise the accumulators, and m * p / (1 + 2^g2) goes to the
//     staging rows (the same LDS, free again once the x operands are in registers);
//   - the staged rows leave as whole 16-byte chunks of the group's channel range of
//     each pair: consecutive pairs are consecutive lines of `out`.
// The next tile's x blocks, z chunks and mask values are loaded while the current one is
// computed.
template <class T, int KXM, int KZM, int ST, int UGM, int W, int XBC, bool RESID>
__global__ __launch_bounds__(64 * W) void k3_output_gate_waves(
    const T* __restrict__ x, ZIn<T, RESID> z, const T* __restrict__ mask, ZOut<T, RESID> out,
    const T* __restrict__ wo, const float* __restrict__ to,
    const T* __restrict__ wg, const float* __restrict__ tg, int n, int np, int cz, int czp, int c,
    int cp, int mask_all, int ug, int total_tiles, const int* __restrict__ extents,
    int compact) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int THREADS = 64 * W;
  constexpr int TW = 16 * ST;        // pairs per wave tile
  constexpr int PO = TW / E;         // E-pair column blocks per wave tile
  // x moves in blocks of XBC channels x E pairs (XBC loads of 16 bytes per block)
  constexpr int XBM = (KXM * (KG / XBC) * PO + 63) / 64;  // x blocks per lane (at most)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int gch = ug * 16;           // output channels of this group
  const int ch0 = blockIdx.y * gch;  // its first output channel
  const int wos = cp + E, wgs = czp + E;
  const int sst = (cp > gch ? cp : gch) + E;  // staging row stride (elements)
  T* const wo_s = (T*)smem;                   // [gch][wos]
  T* const wg_s = wo_s + gch * wos;           // [gch][wgs]
  float* const to_s = (float*)(wg_s + gch * wgs);
  float* const tg_s = to_s + gch;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const stg = (T*)(tg_s + gch) + wave * TW * sst;  // [TW][sst]
  const int p = lane & 15, q = lane >> 4;

  // ---- this group's weight rows and start vectors -> LDS ----
  // All loads of a thread are issued before any LDS store (one memory round trip, not one
  // per chunk): the trip counts are compile-time bounds with the real extents as guards.
  {
    constexpr int WCX = KXM * KG / E, WCZ = KZM * KG / E;  // chunks per weight row
    constexpr int NWO = (UGM * 16 * WCX + THREADS - 1) / THREADS;
    constexpr int NWG = (UGM * 16 * WCZ + THREADS - 1) / THREADS;
    chunk_t vo[NWO], vg[NWG];
#pragma unroll
    for (int k = 0; k < NWO; ++k) {
      const int idx = tid + THREADS * k, r = idx / WCX, cc = idx - r * WCX;
      const int rr = r < gch ? r : 0;
      vo[k] = ld16(wo + (size_t)(ch0 + rr) * cp + cc * E);
    }
#pragma unroll
    for (int k = 0; k < NWG; ++k) {
      const int idx = tid + THREADS * k, r = idx / WCZ, cc = idx - r * WCZ;
      const int rr = r < gch ? r : 0;
      vg[k] = ld16(wg + (size_t)(ch0 + rr) * czp + cc * E);
    }
    const float vto = tid < gch ? to[ch0 + tid] : 0.f, vtg = tid < gch ? tg[ch0 + tid] : 0.f;
#pragma unroll
    for (int k = 0; k < NWO; ++k) {
      const int idx = tid + THREADS * k, r = idx / WCX, cc = idx - r * WCX;
      if (r < gch) st16(wo_s + r * wos + cc * E, vo[k]);
    }
#pragma unroll
    for (int k = 0; k < NWG; ++k) {
      const int idx = tid + THREADS * k, r = idx / WCZ, cc = idx - r * WCZ;
      if (r < gch) st16(wg_s + r * wgs + cc * E, vg[k]);
    }
    if (tid < gch) {
      to_s[tid] = vto;
      tg_s[tid] = vtg;
    }
  }
  __syncthreads();

  const int ntw = (n + TW - 1) / TW;
  const int cbn = c / XBC;          // XBC-channel blocks of x
  const int xblocks = cbn * PO;     // blocks per wave tile
  const size_t plane = (size_t)np * np;

  struct Pre {
    chunk_t xv[XBM][XBC];
    chunk_t zv[ST][KZM];
    T m[ST];
  };
  // The loads are buffer loads: a scalar base and byte offset per tile plus a per-lane
  // offset that is the same in every tile. No address arithmetic lands in a register a
  // load still has to read, so the loads issue back to back. The z and mask resources end
  // at the row end n: pairs past it read as zero (their mask is 0). Every load is
  // unconditional; selects happen at use.
  unsigned int xoff[XBM][XBC], zoff[ST][KZM], moff[ST];
#pragma unroll
  for (int k = 0; k < XBM; ++k) {
    const int blk = lane + 64 * k;
    const int bl = blk < xblocks ? blk : 0;
    const int o = bl / cbn, cb = bl - o * cbn;
#pragma unroll
    for (int e = 0; e < XBC; ++e)
      xoff[k][e] = (unsigned int)(((size_t)(cb * XBC + e) * plane + o * E) * sizeof(T));
  }
#pragma unroll
  for (int st = 0; st < ST; ++st) {
#pragma unroll
    for (int ks = 0; ks < KZM; ++ks) {
      const int ch = ks * KG + q * E;
      zoff[st][ks] = (unsigned int)(((st * 16 + p) * cz + (ch < cz ? ch : 0)) * sizeof(T));
    }
    moff[st] = mask_all ? 0u : (unsigned int)((st * 16 + p) * sizeof(T));
  }
  // With mask extents, the pairs past the item's extent L read as zero (mask 0) and a
  // tile outside the leading L x L square reads nothing: it is a zero update (skipped).
  // With `compact` (few items) the tile list holds only the tiles inside the extents, so
  // the remaining work is shared evenly; the outputs of the pairs outside are written by
  // k3_fill_outside.
  ExtentCache ecache;
  ActiveTiles sched;
  if (compact) {
    sched.init(extents, n, total_tiles / (n * ntw), TW);
    total_tiles = sched.total();
    if (total_tiles == 0) return;  // no item has a valid pair (no barrier follows)
  }
  auto coords = [&](int t, int& bb, int& i, int& j0) {
    if (compact) {
      sched.at(t, bb, i, j0);
      return;
    }
    bb = t / (n * ntw);
    const int rem = t - bb * n * ntw;
    i = rem / ntw;
    j0 = (rem - i * ntw) * TW;
  };
  auto fetch = [&](int t, Pre& f) {
    t = t < total_tiles ? t : total_tiles - 1;  // waves without a tile fetch the last one
    int bb, i, j0;
    coords(t, bb, i, j0);
    const int lim = item_bound(extents, bb, n, ecache);
    const bool act = i < lim && j0 < lim;
    const size_t xext = act ? (size_t)c * plane * sizeof(T) : 0;  // below 2^31 (launch check)
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + (size_t)bb * c * plane, xext);
    const size_t row0 = ((size_t)bb * n + i) * n + j0;  // first pair of the tile
    const size_t live = act ? (size_t)(lim - j0) : 0;    // pairs of the tile that are read
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(z + row0 * cz, live * cz * sizeof(T));
    const __amdgpu_buffer_rsrc_t rm =
        buffer_rsrc(mask_all ? mask : mask + row0,
                    mask_all ? (act ? sizeof(T) : 0) : live * sizeof(T));
    const int xs = (int)(((size_t)i * np + j0) * sizeof(T));
#pragma unroll
    for (int k = 0; k < XBM; ++k)
#pragma unroll
      for (int e = 0; e < XBC; ++e) f.xv[k][e] = load16(rx, xoff[k][e], xs);
#pragma unroll
    for (int st = 0; st < ST; ++st) {
#pragma unroll
      for (int ks = 0; ks < KZM; ++ks) f.zv[st][ks] = load16(rz, zoff[st][ks], 0);
      f.m[st] = load_elem(rm, moff[st], 0, T());
    }
  };

  const int gw = blockIdx.x * W + wave;
  const int nw = gridDim.x * W;
  int t = gw;
  Pre f;
  fetch(t, f);
  for (; t < total_tiles; t += nw) {
    int bb, i, j0;
    coords(t, bb, i, j0);
    float mrow[ST];
    bool ones = true, none = true;
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      mrow[st] = j0 + st * 16 + p < n ? to_f32(f.m[st]) : 0.f;
      ones = ones && mrow[st] == 1.f;
      none = none && mrow[st] == 0.f;
    }
    // a tile wholly outside the mask: zero update, no x transpose, LayerNorm or MFMA (its
    // x is never read)
    const bool skip = __all(none);
    if (skip) {
      fetch(t + nw < total_tiles ? t + nw : t, f);
    } else {
      // x: transpose the XBC x E blocks into pair-major staging rows. Every lane stores (no
      // predicated-off memory operations in the loop): a lane without a block writes its
      // junk into the last E columns of the rows, which nothing reads.
#pragma unroll
      for (int k = 0; k < XBM; ++k) {
        const int blk = lane + 64 * k;
        const bool real = blk < xblocks;
        const int bl = real ? blk : 0;
        const int o = bl / cbn, cb = bl - o * cbn;
        const int col0 = real ? cb * XBC : sst - E;
        T tb[XBC][E];
#pragma unroll
        for (int e = 0; e < XBC; ++e) {
          const T* pv = (const T*)&f.xv[k][e];
#pragma unroll
          for (int ff = 0; ff < E; ++ff) tb[e][ff] = pv[ff];
        }
#pragma unroll
        for (int ff = 0; ff < E; ++ff) {
          if constexpr (XBC == E) {
            T col[E];
#pragma unroll
            for (int e = 0; e < E; ++e) col[e] = tb[e][ff];
            st16(stg + (o * E + ff) * sst + col0, __builtin_bit_cast(chunk_t, col));
          } else {
            static_assert(XBC * 2 == E, "half-width x blocks");
            T col[XBC];
#pragma unroll
            for (int e = 0; e < XBC; ++e) col[e] = tb[e][ff];
            *(half_t*)(stg + (o * E + ff) * sst + col0) = __builtin_bit_cast(half_t, col);
          }
        }
      }
      // The weight and start-vector addresses and the padding masks are the same in every
      // tile; an opaque zero, produced anew each tile, keeps the compiler from hoisting them
      // out of the tile loop (which would pin all of them in registers for the whole launch).
      int opaque;
      asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));
      chunk_t bx[ST][KXM], bz[ST][KZM];
#pragma unroll
      for (int st = 0; st < ST; ++st)
#pragma unroll
        for (int ks = 0; ks < KZM; ++ks) bz[st][ks] = f.zv[st][ks];
      wave_lds_sync();
#pragma unroll
      for (int st = 0; st < ST; ++st)
#pragma unroll
        for (int ks = 0; ks < KXM; ++ks)
          bx[st][ks] = ld16(stg + (st * 16 + p) * sst + ks * KG + q * E);
      // widths that do not fill the compiled chunk count: zero the chunks past the real
      // channels (a wave-uniform branch, not taken at full width)
      if (c < cp || cz < czp) {
        const int ch0q = q * E + opaque;
#pragma unroll
        for (int ks = 0; ks < KXM; ++ks) {
          const unsigned int kx = ks * KG + ch0q < c ? ~0u : 0u;
#pragma unroll
          for (int st = 0; st < ST; ++st) bx[st][ks] &= kx;
        }
#pragma unroll
        for (int ks = 0; ks < KZM; ++ks) {
          const unsigned int kz = ks * KG + ch0q < cz ? ~0u : 0u;
#pragma unroll
          for (int st = 0; st < ST; ++st) bz[st][ks] &= kz;
        }
      }

      // the next tile's loads are in flight from here on (the last tile refetches itself)
      fetch(t + nw < total_tiles ? t + nw : t, f);

#pragma unroll
      for (int st = 0; st < ST; ++st) {
        normalize_operand_row<KXM>(bx[st], c, lane, T());
        normalize_operand_row<KZM>(bz[st], cz, lane, T());
      }

      // units of this group (a rolled loop: unrolled, the scheduler overlaps the units' LDS
      // reads beyond the register budget). Tiles whose pairs all have mask 1 skip the
      // multiply by m (a wave-uniform branch).
      const T* const wo_t = wo_s + opaque;
      const T* const wg_t = wg_s + opaque;
      const float* const to_t = to_s + opaque;
      const float* const tg_t = tg_s + opaque;
      auto units = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll 1
        for (int u = 0; u < ug; ++u) {
          {
            const int r0 = u * 16;
            const f32x4 bo4 = ld16f(to_t + r0 + 4 * q), bg4 = ld16f(tg_t + r0 + 4 * q);
            f32x4 ap[ST], ag[ST];
#pragma unroll
            for (int st = 0; st < ST; ++st) {
              ap[st] = bo4;
              ag[st] = bg4;
            }
            // all of the unit's weight chunks are requested before the first MFMA, so the
            // LDS latency is paid once per unit rather than once per chunk
            const T* wor = wo_t + (r0 + p) * wos + q * E;
            const T* wgr = wg_t + (r0 + p) * wgs + q * E;
            chunk_t wa[KXM], wb[KZM];
#pragma unroll
            for (int ks = 0; ks < KXM; ++ks) wa[ks] = ld16(wor + ks * KG);
#pragma unroll
            for (int ks = 0; ks < KZM; ++ks) wb[ks] = ld16(wgr + ks * KG);
#pragma unroll
            for (int ks = 0; ks < KXM; ++ks)
#pragma unroll
              for (int st = 0; st < ST; ++st) ap[st] = mma16(ap[st], wa[ks], bx[st][ks], T());
#pragma unroll
            for (int ks = 0; ks < KZM; ++ks)
#pragma unroll
              for (int st = 0; st < ST; ++st) ag[st] = mma16(ag[st], wb[ks], bz[st][ks], T());
            // accumulator register r <-> output channel ch0 + r0 + 4q + r of pair st*16 + p
#pragma unroll
            for (int st = 0; st < ST; ++st) {
              float o4[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                o4[r] = gate_mul(MASKED ? ap[st][r] * mrow[st] : ap[st][r], ag[st][r]);
              store4(stg + (st * 16 + p) * sst + r0 + 4 * q, o4[0], o4[1], o4[2], o4[3]);
            }
          }
        }
      };
      if (__all(ones))
        units(std::false_type());
      else
        units(std::true_type());
    }  // not skipped

    // staging -> out: the group's channel range of TW consecutive pairs. The number of
    // stores is fixed and none is predicated off: a lane whose chunk lies past the row end
    // (or past the group's channels) rewrites the last real chunk with the same bytes.
    // With an unconditional store count the wait for the next tile's loads does not have
    // to wait for these stores as well.
    wave_lds_sync();
    constexpr int CPPM = UGM * 16 / E;  // chunks per staged row, at most
    const int cpp = gch / E;
    const int last = n - 1 - j0;        // last real pair of the tile (< TW when ragged)
    const size_t row0 = ((size_t)bb * n + i) * n + j0;
    constexpr int NOUT = (TW * CPPM + 63) / 64;
    // chunk k of the lane: element offset from the tile's first output element (pair j0,
    // channel ch0), the same for out and z
    unsigned int goff[NOUT];
    int soff[NOUT];
#pragma unroll
    for (int k = 0; k < NOUT; ++k) {
      const int idx = k * 64 + lane;
      int pr = idx / CPPM, cc = idx - pr * CPPM;
      pr = pr < last ? pr : last;
      pr = pr < TW ? pr : TW - 1;
      cc = cc < cpp ? cc : cpp - 1;
      goff[k] = (unsigned int)(pr * cz + cc * E);
      soff[k] = pr * sst + cc * E;
    }
    // The output is the last thing the update writes and nothing in the update reads it
    // again: non-temporal stores keep it from displacing x and z in the caches (K3 took
    // 52.7 instead of 55.2 us at N = 512, c_z = c = 128). Device-scope stores of the same
    // whole lines made K3 alone 0.3 us faster but the two-direction step 8% slower.
    const size_t obase = row0 * cz + ch0;
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc_u32(out + obase, 0xffffffffu);
    // a skipped tile's update is zero: its staging rows are not read
    const chunk_t zero = {0u, 0u, 0u, 0u};
    if constexpr (RESID) {
      // out = z + update. Every z chunk is read before any chunk is written, so the
      // duplicate stores past the row end also add the update to the original z (out may
      // be z itself: each pair is read and written only by this wave, in this tile).
      chunk_t zr[NOUT];
#pragma unroll
      for (int k = 0; k < NOUT; ++k) zr[k] = ld16(z + obase + goff[k]);
#pragma unroll
      for (int k = 0; k < NOUT; ++k)
        k3_store16(ro, add_chunks(skip ? zero : ld16(stg + soff[k]), zr[k], T()), goff[k] * (unsigned int)sizeof(T));
    } else {
#pragma unroll
      for (int k = 0; k < NOUT; ++k)
        k3_store16(ro, skip ? zero : ld16(stg + soff[k]), goff[k] * (unsigned int)sizeof(T));
    }
  }
}

// The outputs of the pairs outside each item's extent (its leading L x L square), where
// the update is zero: out = 0, or out = z with the residual add. Workgroup (i, b) writes
// row i of item b from column L on (the whole row when i >= L); the row's pairs are one
// contiguous run of 16-byte chunks.
template <class T, bool RESID>
__global__ __launch_bounds__(256) void k3_fill_outside(const T* __restrict__ z,
                                                       T* __restrict__ out,
                                                       const int* __restrict__ extents, int n,
                                                       int cz) {
  constexpr int E = Traits<T>::E;
  const int i = blockIdx.x, bb = blockIdx.y;
  const int L = mask_extent(extents, bb, n);
  const int j0 = i < L ? L : 0;
  const size_t row = ((size_t)bb * n + i) * n;
  const size_t c0 = (row + j0) * cz / E, c1 = (row + n) * cz / E;  // chunk range
  const chunk_t zero = {0u, 0u, 0u, 0u};
  for (size_t k = c0 + threadIdx.x; k < c1; k += 256) {
    if constexpr (RESID)
      __builtin_nontemporal_store(ld16(z + k * E), (chunk_t*)(out + k * E));
    else
      __builtin_nontemporal_store(zero, (chunk_t*)(out + k * E));
  }
}

template <class T, bool RESID>
static hipError_t launch_fill_outside(const StageArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k3_fill_outside<T, RESID>), dim3(a.n, a.batch), dim3(256), 0, st,
                     (const T*)a.z, (T*)a.out, a.extents, a.n, a.cz);
  return hipGetLastError();
}

// Shapes of the wave-independent form: 8 waves per workgroup; narrow rows (KXM + KZM <= 8
// chunk groups) take 32-pair wave tiles, wider rows 16-pair tiles, if the operands and the
// next tile's loads fit the register budget. (16-pair tiles with 16 waves and half-width x
// blocks are faster with hot caches but fetch x poorly from DRAM.)
template <class T, int KXM, int KZM>
struct K3WShape {
  static constexpr int E = Traits<T>::E;
  static constexpr bool NARROW = KXM + KZM <= 8;
  static constexpr int ST = NARROW ? 2 : 1;
  static constexpr int W = 8;
  static constexpr int XBC = E;
  static constexpr int XBM = (KXM * (Traits<T>::KG / XBC) * (16 * ST / E) + 63) / 64;
  static constexpr int VGPRS = 4 * (ST * (KXM + KZM) + XBM * XBC + ST * KZM);
  static constexpr bool OK = VGPRS <= (NARROW ? 128 : 160);
  static constexpr int UGM = KZM * Traits<T>::KG / 16 < 8 ? KZM * Traits<T>::KG / 16 : 8;
};

template <class T>
static size_t k3w_lds(const StageArgs& a, int ug, int st, int waves) {
  constexpr int E = Traits<T>::E;
  const int gch = ug * 16;
  const int sst = (a.cp > gch ? a.cp : gch) + E;
  return (size_t)gch * ((a.cp + E) + (a.czp + E)) * sizeof(T) + 2 * (size_t)gch * sizeof(float) +
         (size_t)waves * 16 * st * sst * sizeof(T);
}

// Launches the wave-independent form if some unit grouping fits LDS; *done = false leaves
// the launch to the tile-shared form.
template <class T, int KXM, int KZM, bool RESID>
static hipError_t launch_k3w_t(const StageArgs& a, hipStream_t st, bool* done) {
  *done = false;
  // the per-lane x offsets of the wave-independent form are 32-bit byte offsets into one
  // batch item's x: larger x goes to the tile-shared form
  if ((size_t)a.c * a.np * a.np * sizeof(T) >= 0x80000000ull) return hipSuccess;
  if constexpr (K3WShape<T, KXM, KZM>::OK) {
    constexpr int ST = K3WShape<T, KXM, KZM>::ST;
    constexpr int W = K3WShape<T, KXM, KZM>::W;
    constexpr int XBC = K3WShape<T, KXM, KZM>::XBC;
    constexpr int UGM = K3WShape<T, KXM, KZM>::UGM;
    const int units = a.cz / 16;
    int ug = 0;
    for (int g = units < UGM ? units : UGM; g >= 1; --g)
      if (units % g == 0 && k3w_lds<T>(a, g, ST, W) <= LDS_PER_CU) {
        ug = g;
        break;
      }
    if (ug == 0) return hipSuccess;
    if (a.plan) {
      a.plan->k3_form = 0;
      a.plan->k3_groups = units / ug;
      *done = true;
      return hipSuccess;
    }
    const size_t lds = k3w_lds<T>(a, ug, ST, W);
    auto fn = k3_output_gate_waves<T, KXM, KZM, ST, UGM, W, XBC, RESID>;
    static std::atomic<int> granted{0};
    hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
    if (e != hipSuccess) return e;
    const int groups = units / ug;
    constexpr int TW = 16 * ST;
    const int total = a.batch * a.n * ((a.n + TW - 1) / TW);
    static std::atomic<int> occ{0};
    static std::atomic<size_t> occ_lds{0};
    const int per_cu = resident_blocks((const void*)fn, 64 * W, lds, occ, occ_lds);
    const int cap = a.num_cus * per_cu / groups > 0 ? a.num_cus * per_cu / groups : 1;
    const int need = (total + W - 1) / W;
    const int blocks = need < cap ? need : cap;
    const int mask_all = a.mask == nullptr;
    // with extents and few items, the kernel runs only the tiles inside the extents and the
    // outputs outside are written first (in place they already hold z + 0)
    const bool compact = a.extents && a.batch <= COMPACT_MAX_ITEMS;
    if (compact && !(RESID && a.out == a.z)) {
      hipError_t e2 = launch_fill_outside<T, RESID>(a, st);
      if (e2 != hipSuccess) return e2;
    }
    hipLaunchKernelGGL(fn, dim3(blocks, groups), dim3(64 * W), lds, st, (const T*)a.x,
                       (const T*)a.z, (const T*)(mask_all ? a.one : a.mask), (T*)a.out,
                       (const T*)a.wo, a.to, (const T*)a.wg, a.tg, a.n, a.np, a.cz, a.czp, a.c,
                       a.cp, mask_all, ug, total, a.extents, compact ? 1 : 0);
    *done = true;
    return hipGetLastError();
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------

template <class T, int KXM, int KZM, int XB, bool RESID>
static hipError_t launch_k3_t(const StageArgs& a, hipStream_t st) {
  if (a.plan) {
    a.plan->k3_form = 1;
    a.plan->k3_groups = (a.cz / 16 + K3_WAVES * K3_UPW - 1) / (K3_WAVES * K3_UPW);
    return hipSuccess;
  }
  constexpr int E = Traits<T>::E;
  auto lds_for = [&](int nb) {
    return (size_t)nb * K3_TP * ((a.cp + E) + (a.czp + E)) * sizeof(T) +
           (size_t)nb * K3_TP * sizeof(float);
  };
  const int nbuf = lds_for(2) <= K3_LDS_BUDGET ? 2 : 1;
  const size_t lds = lds_for(nbuf);
  auto fn = k3_output_gate<T, KXM, KZM, XB, RESID>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const int units = a.cz / 16;
  const int groups = (units + K3_WAVES * K3_UPW - 1) / (K3_WAVES * K3_UPW);
  const int total = a.batch * a.n * ((a.n + K3_TP - 1) / K3_TP);
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, K3_THREADS, lds, occ, occ_lds);
  const int cap = a.num_cus * per_cu / groups > 0 ? a.num_cus * per_cu / groups : 1;
  const int blocks = total < cap ? total : cap;
  const int mask_all = a.mask == nullptr;
  hipLaunchKernelGGL(fn, dim3(blocks, groups), dim3(K3_THREADS), lds, st, (const T*)a.x,
                     (const T*)a.z, (const T*)(mask_all ? a.one : a.mask), (T*)a.out,
                     (const T*)a.wo, a.to, (const T*)a.wg, a.tg, a.n, a.np, a.cz, a.czp, a.c, a.cp,
                     mask_all, nbuf, total);
  return hipGetLastError();
}

// The compiled (KX, KZ) variants are listed in launch.h (TRIMUL_K3_VARIANTS); the host
// pads cp and czp to exactly one of them.
template <class T, bool RESID>
static hipError_t launch_k3_dispatch(const StageArgs& a, hipStream_t st) {
  constexpr int E = Traits<T>::E;
  const int kx = a.cp / Traits<T>::KG, kz = a.czp / Traits<T>::KG;
  const int xblocks = (a.c / E) * (K3_TP / E);
  const int xb = (xblocks + K3_THREADS - 1) / K3_THREADS;
  // a second x block per thread is needed only for wide c (KX >= 8 after padding)
#define TRIMUL_CALL(X_, Z_)                                      \
  if (kx == X_ && kz == Z_) {                                    \
    bool done = false;                                           \
    hipError_t e = launch_k3w_t<T, X_, Z_, RESID>(a, st, &done); \
    if (e != hipSuccess || done) return e;                       \
    if (xb == 1) return launch_k3_t<T, X_, Z_, 1, RESID>(a, st); \
    if (X_ >= 8 && xb == 2) return launch_k3_t<T, X_, Z_, (X_ >= 8 ? 2 : 1), RESID>(a, st); \
  }
  TRIMUL_K3_VARIANTS(TRIMUL_CALL)
#undef TRIMUL_CALL
  return hipErrorInvalidValue;
}

hipError_t launch_k3(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  if (bf16_storage) {
    bool done = false;
    hipError_t e = launch_k3_stream(a, st, &done);
    if (e != hipSuccess || done) return e;
  }
  if (a.residual)
    return bf16_storage ? launch_k3_dispatch<bf16, true>(a, st)
                        : launch_k3_dispatch<float, true>(a, st);
  return bf16_storage ? launch_k3_dispatch<bf16, false>(a, st)
                      : launch_k3_dispatch<float, false>(a, st);
}

}  // namespace trimul
