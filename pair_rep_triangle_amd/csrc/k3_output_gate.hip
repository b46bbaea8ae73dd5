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

#include "device_common.h"

namespace trimul {

constexpr int K3_TP = 64;
constexpr int K3_WAVES = 4;
constexpr int K3_THREADS = 64 * K3_WAVES;
constexpr int K3_TPP = K3_THREADS / K3_TP;  // threads per pair when staging a tile
constexpr int K3_UPW = 2;                   // 16-channel output units per wave
constexpr size_t K3_LDS_BUDGET = 80 * 1024;  // double-buffer only while two workgroups fit a CU

template <class T, int KXM, int KZM, int XB>
__global__ __launch_bounds__(K3_THREADS) void k3_output_gate(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ mask,
    T* __restrict__ out, const T* __restrict__ wo, const float* __restrict__ to,
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
      const int j = j0 + pr;
      const float m = mv[pr];
#pragma unroll
      for (int jj = 0; jj < UPW; ++jj) {
        if (uok[jj] && j < n) {
          T* dst = out + (((size_t)bb * n + i) * n + j) * cz + oc0[jj];
          store4(dst, gate_mul(ap[jj][0] * m, ag[jj][0]), gate_mul(ap[jj][1] * m, ag[jj][1]),
                 gate_mul(ap[jj][2] * m, ag[jj][2]), gate_mul(ap[jj][3] * m, ag[jj][3]));
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

// ---------------------------------------------------------------------------------------

template <class T, int KXM, int KZM, int XB>
static hipError_t launch_k3_t(const StageArgs& a, hipStream_t st) {
  constexpr int E = Traits<T>::E;
  auto lds_for = [&](int nb) {
    return (size_t)nb * K3_TP * ((a.cp + E) + (a.czp + E)) * sizeof(T) +
           (size_t)nb * K3_TP * sizeof(float);
  };
  const int nbuf = lds_for(2) <= K3_LDS_BUDGET ? 2 : 1;
  const size_t lds = lds_for(nbuf);
  auto fn = k3_output_gate<T, KXM, KZM, XB>;
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
template <class T>
static hipError_t launch_k3_dispatch(const StageArgs& a, hipStream_t st) {
  constexpr int E = Traits<T>::E;
  const int kx = a.cp / Traits<T>::KG, kz = a.czp / Traits<T>::KG;
  const int xblocks = (a.c / E) * (K3_TP / E);
  const int xb = (xblocks + K3_THREADS - 1) / K3_THREADS;
  // a second x block per thread is needed only for wide c (KX >= 8 after padding)
#define TRIMUL_CALL(X_, Z_)                                      \
  if (kx == X_ && kz == Z_) {                                    \
    if (xb == 1) return launch_k3_t<T, X_, Z_, 1>(a, st);        \
    if (X_ >= 8 && xb == 2) return launch_k3_t<T, X_, Z_, (X_ >= 8 ? 2 : 1)>(a, st); \
  }
  TRIMUL_K3_VARIANTS(TRIMUL_CALL)
#undef TRIMUL_CALL
  return hipErrorInvalidValue;
}

hipError_t launch_k3(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  return bf16_storage ? launch_k3_dispatch<bf16>(a, st) : launch_k3_dispatch<float>(a, st);
}

}  // namespace trimul
