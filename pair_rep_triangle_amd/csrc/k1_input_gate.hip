// k1: input LayerNorm + gated dual projection + pair mask -> a, b (channel-major).
//
// RFProteína architecture page, "Triangle multiplication on SM90" (K1: the input
// projection with the input LayerNorm, producing the gated operands) and "Dual-GEMM
// gates" (x_x form sigma(x W_g^T + b_g) * (x W_p^T + b_p); the input gate absorbs the
// pair mask and writes its output already laid out for the contraction).
//
// The k extent is a compile-time constant: the host pads c_z to exactly KMAX chunk groups.
// Work split (persistent): a tile is TP = 64 consecutive storage columns of one storage
// row r; for outgoing the z pairs are (r, s), for incoming (s, r), so both directions
// store a[b][ch][r][s] contiguously along s. A workgroup of 8 waves loops over tiles.
// Each wave owns UPW "units" (a unit = the gate and proj rows of 16 channels of a or b)
// and keeps their weights in registers for the whole kernel; the tile's normalised z
// (the MFMA A operand) is shared through LDS. The LayerNorm gamma is folded into the
// weights and beta / the bias into the accumulator's initial value (host side); the gate
// rows carry an extra -log2(e) so the epilogue is one exp2 and one reciprocal.
// The next tile's z is fetched into registers while the MFMAs of the current tile run.

#include "device_common.h"

namespace trimul {

constexpr int K1_TP = 64;
constexpr int K1_WAVES = 8;
constexpr int K1_THREADS = 64 * K1_WAVES;

template <class T, int KMAX, int UPW>
__global__ __launch_bounds__(K1_THREADS, 2) void k1_input_gate(
    const T* __restrict__ z, const T* __restrict__ mask, T* __restrict__ a_out,
    T* __restrict__ b_out, const T* __restrict__ w1, const float* __restrict__ t1, int n, int np,
    int cz, int czp, int c, int incoming, int mask_all, int total_tiles) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = Traits<T>::KG;
  constexpr int TP = K1_TP;
  constexpr int NCH = (KMAX * KG / E + 7) / 8;  // z chunks per thread (8 threads per pair)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int zstride = czp + E;
  // LDS: normalised z tiles [2][TP][zstride], masks [2][TP]
  T* const zbase = (T*)smem;
  float* const mvbuf = (float*)(zbase + 2 * TP * zstride);
  auto zbuf = [&](int b) { return zbase + b * TP * zstride; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cblocks = c / 16, units = 2 * cblocks;
  const int ntx = np / TP;

  // ---- this wave's units: weights and biases into registers ----
  chunk_t wgt[UPW][2][KMAX];
  float bias[UPW][2];
  int uch[UPW], uq[UPW];
  bool uok[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = blockIdx.y * (K1_WAVES * UPW) + wave + K1_WAVES * j;
    uok[j] = u < units;
    uq[j] = uok[j] ? u / cblocks : 0;
    uch[j] = uok[j] ? (u - uq[j] * cblocks) * 16 + (lane & 15) : 0;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const size_t row = (size_t)(2 * uq[j] + gp) * c + uch[j];
      bias[j][gp] = uok[j] ? t1[row] : 0.f;
#pragma unroll
      for (int ks = 0; ks < KMAX; ++ks)
        wgt[j][gp][ks] = uok[j] ? ld16(w1 + row * czp + ks * KG + (lane >> 4) * E)
                                : chunk_t{0u, 0u, 0u, 0u};
    }
  }

  // ---- tile staging: thread (t, part) handles chunks part, part+8, ... of pair t ----
  const int t = tid >> 3, part = tid & 7;
  const int czc = cz / E, cpr = czp / E;
  auto tile_coords = [&](int tile, int& bb, int& r, int& s0) {
    bb = tile / (np * ntx);
    const int rem = tile - bb * np * ntx;
    r = rem / ntx;
    s0 = (rem - r * ntx) * TP;
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
  auto fetch = [&](int tile, Pre& f) {
    int bb, r, s0;
    tile_coords(tile, bb, r, s0);
    const int s = s0 + t;
    const int p = incoming ? s : r, q = incoming ? r : s;
    f.valid = p < n && q < n;
    const size_t pair = f.valid ? ((size_t)bb * n + p) * n + q : 0;
    const T* src = z + pair * cz;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = part + 8 * i;
      f.v[i] = ld16(src + (ch < czc ? ch : 0) * E);
    }
    f.m = mask[mask_all ? 0 : pair];
  };
  auto stage = [&](int buf, Pre& f) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (!(f.valid && part + 8 * i < czc)) f.v[i] = chunk_t{0u, 0u, 0u, 0u};
    normalize_row<T, NCH>(f.v, part, czc, cz);
    T* row = zbuf(buf) + t * zstride;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = part + 8 * i;
      if (ch < cpr) st16(row + ch * E, f.v[i]);
    }
    if (part == 0) mvbuf[buf * TP + t] = f.valid ? to_f32(f.m) : 0.f;
  };

  int tile = blockIdx.x;  // the grid never exceeds the tile count
  {
    Pre f;
    fetch(tile, f);
    stage(0, f);
  }
  __syncthreads();

  for (int it = 0; tile < total_tiles; tile += gridDim.x, ++it) {
    const int cur = it & 1;
    const int next = tile + gridDim.x;
    Pre pre;
    fetch(next < total_tiles ? next : tile, pre);  // the last iteration refetches, unused

    int bb, r, s0;
    tile_coords(tile, bb, r, s0);
    const T* zs = zbuf(cur);
    const float* mv = mvbuf + cur * TP;
#pragma unroll
    for (int rt = 0; rt < TP / 16; ++rt) {
      f32x4 acc[UPW][2];
#pragma unroll
      for (int j = 0; j < UPW; ++j)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp)
          acc[j][gp] = f32x4{bias[j][gp], bias[j][gp], bias[j][gp], bias[j][gp]};
      const T* arow = zs + (rt * 16 + (lane & 15)) * zstride + (lane >> 4) * E;
#pragma unroll
      for (int ks = 0; ks < KMAX; ++ks) {
        const chunk_t af = ld16(arow + ks * KG);
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
          acc[j][0] = mma16(acc[j][0], af, wgt[j][0][ks], T());
          acc[j][1] = mma16(acc[j][1], af, wgt[j][1][ks], T());
        }
      }
      // accumulator register rr <-> pair rt*16 + 4*(lane/16) + rr, channel uch
      const int p0 = rt * 16 + 4 * (lane >> 4);
      const f32x4 m4 = ld16f(mv + p0);
#pragma unroll
      for (int j = 0; j < UPW; ++j) {
        if (!uok[j]) continue;
        float o[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[rr] = gate_mul(acc[j][1][rr] * m4[rr], acc[j][0][rr]);
        T* dst = (uq[j] ? b_out : a_out) + (((size_t)bb * c + uch[j]) * np + r) * np + s0 + p0;
        store4(dst, o[0], o[1], o[2], o[3]);
      }
    }
    stage(cur ^ 1, pre);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------

template <class T, int KMAX, int UPW>
static hipError_t launch_k1_t(const StageArgs& a, hipStream_t st) {
  constexpr int E = Traits<T>::E;
  const size_t lds = 2 * (size_t)K1_TP * (a.czp + E) * sizeof(T) + 2 * K1_TP * sizeof(float);
  auto fn = k1_input_gate<T, KMAX, UPW>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const int units = 2 * (a.c / 16);
  const int groups = (units + K1_WAVES * UPW - 1) / (K1_WAVES * UPW);
  const int total = a.batch * a.np * (a.np / K1_TP);
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, K1_THREADS, lds, occ, occ_lds);
  const int cap = a.num_cus * per_cu / groups > 0 ? a.num_cus * per_cu / groups : 1;
  const int blocks = total < cap ? total : cap;
  const int mask_all = a.mask == nullptr;
  hipLaunchKernelGGL(fn, dim3(blocks, groups), dim3(K1_THREADS), lds, st, (const T*)a.z,
                     (const T*)(mask_all ? a.one : a.mask), (T*)a.a, (T*)a.b, (const T*)a.w1, a.t1,
                     a.n, a.np, a.cz, a.czp, a.c, a.incoming, mask_all, total);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_k1_dispatch(const StageArgs& a, hipStream_t st) {
  switch (a.czp / Traits<T>::KG) {
    case 1: return launch_k1_t<T, 1, 2>(a, st);
    case 2: return launch_k1_t<T, 2, 2>(a, st);
    case 4: return launch_k1_t<T, 4, 2>(a, st);
    case 8: return launch_k1_t<T, 8, 1>(a, st);
    case 12: return launch_k1_t<T, 12, 1>(a, st);
    case 16: return launch_k1_t<T, 16, 1>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_k1(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  return bf16_storage ? launch_k1_dispatch<bf16>(a, st) : launch_k1_dispatch<float>(a, st);
}

}  // namespace trimul
