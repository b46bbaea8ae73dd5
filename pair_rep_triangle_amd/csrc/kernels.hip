// Device code of the triangle multiplicative update for gfx950 (CDNA4).
//
// Three kernels, one per stage of the chain the RFProteína architecture page
// describes for its fused path ("Triangle multiplication on SM90"), re-designed
// for 64-wide wavefronts, MFMA and LDS:
//   k1_input_gate   input LayerNorm (folded into the weights) + the four c_z->c
//                   projections on MFMA + sigmoid gate + pair mask; writes a and
//                   b channel-major [B][c][Np][Np], transposed for incoming
//                   ("Dual-GEMM gates": the input gate absorbs the mask and the
//                   layout change).
//   k2_contract     the contraction over the third residue: one NT GEMM per
//                   (batch, channel), x = A B^T, LDS double-buffered, MFMA with
//                   fp32 accumulation.
//   k3_output_gate  output LayerNorm (folded) + c->c_z projection + output gate
//                   from the re-normalised z (folded) + mask; writes out
//                   [B][N][N][c_z].
//
// LayerNorm folding: W (gamma (.) xhat + beta) + bias with xhat = (x - mu) r is
// computed as r (W' x - mu s) + t, where W' = W diag(gamma) (rounded to the
// storage type), s = row sums of the rounded W' and t = W beta + bias. The
// MFMAs therefore read the raw stored activations; the per-pair (mu, r) are
// applied in the epilogue. The host folds the weights in double precision.
//
// MFMA operand convention used throughout: every lane hands the instruction one
// 16-byte chunk per operand, holding consecutive k of its row (A) / column (B).
// For bf16 that is one v_mfma_*_bf16 (8 k per lane); for fp32 four v_mfma_*_f32
// (one k per lane each). A and B use the same lane -> k assignment, so the sum
// covers every k of the chunk group exactly once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "launch.h"

namespace trimul {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int chunk_t;  // 16 bytes

template <class T> struct Traits;
template <> struct Traits<bf16> { static constexpr int E = 8; };   // elements per chunk
template <> struct Traits<float> { static constexpr int E = 4; };

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ chunk_t ld16(const void* p) { return *(const chunk_t*)p; }
__device__ __forceinline__ void st16(void* p, chunk_t v) { *(chunk_t*)p = v; }

// 16x16 output tile; D[row][col] += sum_k A[row][k] B[col][k] over one chunk group
// (32 k for bf16, 16 k for fp32). Lane l: A row / B col = l % 16.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, chunk_t a, chunk_t b, bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, chunk_t a, chunk_t b, float) {
  f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
  return acc;
}
// 32x32 output tile over one chunk group (16 k for bf16, 8 k for fp32). Lane l: row/col = l % 32.
__device__ __forceinline__ f32x16 mma32(f32x16 acc, chunk_t a, chunk_t b, bf16) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(f32x16 acc, chunk_t a, chunk_t b, float) {
  f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float sigmoidf_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Four consecutive values of T packed for one 8-byte (bf16) / 16-byte (fp32) LDS store.
template <class T> struct Pack4;
template <> struct Pack4<bf16> {
  typedef __attribute__((ext_vector_type(2))) unsigned int type;
  __device__ static type make(float a, float b, float c, float d) {
    bf16 h[4] = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    return __builtin_bit_cast(type, h);
  }
};
template <> struct Pack4<float> {
  typedef f32x4 type;
  __device__ static type make(float a, float b, float c, float d) { return f32x4{a, b, c, d}; }
};

constexpr int TP = 64;        // pairs per tile in k1 / k3
constexpr int NTHREADS = 256; // 4 waves

// Per-pair LayerNorm statistics of TP rows held in LDS (row stride `stride`
// elements, `width` real channels): 4 threads per pair, two passes in fp32.
template <class T>
__device__ __forceinline__ void row_stats(const T* rows, int stride, int width, float* mu, float* rs) {
  const int tid = threadIdx.x;
  const int t = tid >> 2, part = tid & 3;
  const T* row = rows + t * stride;
  float sum = 0.f;
  for (int k = part; k < width; k += 4) sum += to_f32(row[k]);
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  const float mean = sum / (float)width;
  float sq = 0.f;
  for (int k = part; k < width; k += 4) {
    float d = to_f32(row[k]) - mean;
    sq += d * d;
  }
  sq += __shfl_xor(sq, 1);
  sq += __shfl_xor(sq, 2);
  if (part == 0) {
    mu[t] = mean;
    rs[t] = rsqrtf(sq / (float)width + TRI_MUL_LN_EPS_F);
  }
}

// ---------------------------------------------------------------------------------------
// k1: z tile of TP pairs along the storage row -> a, b channel-major.
// Grid (np / TP, np, batch). Storage row r, storage columns s0 .. s0+TP-1; the z pair at
// storage (r, s) is (r, s) for outgoing and (s, r) for incoming.
template <class T>
__global__ __launch_bounds__(NTHREADS) void k1_input_gate(
    const T* __restrict__ z, const T* __restrict__ mask, T* __restrict__ a_out,
    T* __restrict__ b_out, const T* __restrict__ w1, const float* __restrict__ s1,
    const float* __restrict__ t1, int n, int np, int cz, int czp, int c, int incoming) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = 4 * E;  // k per 16x16 MFMA chunk group
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int zstride = czp + E;
  T* zs = (T*)smem;
  float* mu = (float*)(smem + (size_t)TP * zstride * sizeof(T));
  float* rs = mu + TP;
  float* mv = rs + TP;
  T* stg = (T*)(mv + TP);  // [4 waves][16 channels][TP + E]
  const int sstride = TP + E;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bb = blockIdx.z, r = blockIdx.y, s0 = blockIdx.x * TP;

  // 1. z tile -> LDS (zero outside the n x n pairs and in the k padding)
  const int cpr = czp / E, czc = cz / E;
  for (int idx = tid; idx < TP * cpr; idx += NTHREADS) {
    const int t = idx / cpr, ch = idx - t * cpr;
    const int s = s0 + t;
    const int p = incoming ? s : r, q = incoming ? r : s;
    chunk_t v = {0u, 0u, 0u, 0u};
    if (ch < czc && p < n && q < n) v = ld16(z + (((size_t)bb * n + p) * n + q) * cz + ch * E);
    st16(zs + t * zstride + ch * E, v);
  }
  if (tid < TP) {
    const int s = s0 + tid;
    const int p = incoming ? s : r, q = incoming ? r : s;
    float m = 0.f;
    if (p < n && q < n) m = mask ? to_f32(mask[((size_t)bb * n + p) * n + q]) : 1.f;
    mv[tid] = m;
  }
  __syncthreads();
  row_stats(zs, zstride, cz, mu, rs);
  __syncthreads();

  // Per-lane statistics of the pairs this lane's accumulators hold:
  // row tile rt, register rr -> pair rt*16 + 4*(lane/16) + rr.
  float pmu[4][4], prs[4][4], pm[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = rt * 16 + 4 * (lane >> 4) + rr;
      pmu[rt][rr] = mu[t];
      prs[rt][rr] = rs[t];
      pm[rt][rr] = mv[t];
    }

  const int cblocks = c / 16;
  const int units = 2 * cblocks;  // (operand a|b) x (16-channel block)
  const int ksteps = czp / KG;
  T* stw = stg + wave * 16 * sstride;
  for (int u0 = 0; u0 < units; u0 += 4) {
    const int u = u0 + wave;
    if (u < units) {
      const int q = u / cblocks, cb = u - q * cblocks;
      const int ch = cb * 16 + (lane & 15);
      const T* wgr = w1 + ((size_t)(2 * q) * c + ch) * czp + (lane >> 4) * E;
      const T* wpr = w1 + ((size_t)(2 * q + 1) * c + ch) * czp + (lane >> 4) * E;
      f32x4 ag[4], ap[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) ag[rt] = ap[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < ksteps; ++ks) {
        const chunk_t bg = ld16(wgr + ks * KG), bp = ld16(wpr + ks * KG);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const chunk_t af = ld16(zs + (rt * 16 + (lane & 15)) * zstride + ks * KG + (lane >> 4) * E);
          ag[rt] = mma16(ag[rt], af, bg, T());
          ap[rt] = mma16(ap[rt], af, bp, T());
        }
      }
      const float sg = s1[(2 * q) * c + ch], tg = t1[(2 * q) * c + ch];
      const float sp = s1[(2 * q + 1) * c + ch], tp = t1[(2 * q + 1) * c + ch];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float g = prs[rt][rr] * (ag[rt][rr] - pmu[rt][rr] * sg) + tg;
          const float p = prs[rt][rr] * (ap[rt][rr] - pmu[rt][rr] * sp) + tp;
          v[rr] = pm[rt][rr] * p * sigmoidf_fast(g);
        }
        *(typename Pack4<T>::type*)(stw + (lane & 15) * sstride + rt * 16 + 4 * (lane >> 4)) =
            Pack4<T>::make(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
    // staged units -> global: 16 channel rows x TP pairs each, TP*sizeof(T) contiguous bytes
    const int nu = min(4, units - u0);
    const int cpt = TP / E;
    for (int idx = tid; idx < nu * 16 * cpt; idx += NTHREADS) {
      const int wv = idx / (16 * cpt), rem = idx - wv * 16 * cpt;
      const int row = rem / cpt, cc = rem - row * cpt;
      const int uu = u0 + wv, q = uu / cblocks, ch = (uu - q * cblocks) * 16 + row;
      T* dst = (q ? b_out : a_out) + (((size_t)bb * c + ch) * np + r) * np + s0 + cc * E;
      st16(dst, ld16(stg + (wv * 16 + row) * sstride + cc * E));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// k2: x[bc] = A[bc] B[bc]^T for every (batch, channel) bc; A, B, x are [np][np].
// 128 x 128 output tile per workgroup, 4 waves as 2 x 2, each 64 x 64 (2 x 2 MFMA
// 32x32 tiles). k advances 128 bytes per stage through a double-buffered LDS.
// Flat grid of (np/128)^2 * batch*c workgroups, remapped so that consecutive tiles
// of one channel land on the same XCD (workgroup ids are dealt round-robin over the
// 8 XCDs) and share its L2.
constexpr int K2_TILE = 128;

template <class T>
__global__ __launch_bounds__(NTHREADS) void k2_contract(const T* __restrict__ A,
                                                        const T* __restrict__ B,
                                                        T* __restrict__ X, int np) {
  constexpr int E = Traits<T>::E;
  constexpr int KT = 8 * E;        // k per stage (128 bytes per row)
  constexpr int LROW = KT + E;     // LDS row stride in elements (144 bytes)
  constexpr int STAGE = K2_TILE * LROW;
  __shared__ __attribute__((aligned(16))) T lds[2][2][STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int bid = blockIdx.x, total = gridDim.x;
  const int per = total >> 3;
  const int logical = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
  const int t1d = np / K2_TILE;
  const int tiles = t1d * t1d;
  const int bc = logical / tiles, tile = logical - bc * tiles;
  const int ti = tile / t1d, tj = tile - ti * t1d;

  const size_t mat = (size_t)np * np;
  const T* Ab = A + bc * mat + (size_t)ti * K2_TILE * np;
  const T* Bb = B + bc * mat + (size_t)tj * K2_TILE * np;

  chunk_t ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NTHREADS * q, row = idx >> 3, c16 = idx & 7;
      ra[q] = ld16(Ab + (size_t)row * np + k0 + c16 * E);
      rb[q] = ld16(Bb + (size_t)row * np + k0 + c16 * E);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NTHREADS * q, row = idx >> 3, c16 = idx & 7;
      st16(&lds[buf][0][row * LROW + c16 * E], ra[q]);
      st16(&lds[buf][1][row * LROW + c16 * E], rb[q]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nst = np / KT;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    if (s + 1 < nst) gload((s + 1) * KT);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int koff = (2 * kk + (lane >> 5)) * E;
      chunk_t fa[2], fb[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        fa[mt] = ld16(&lds[cur][0][(wm * 64 + mt * 32 + (lane & 31)) * LROW + koff]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        fb[nt] = ld16(&lds[cur][1][(wn * 64 + nt * 32 + (lane & 31)) * LROW + koff]);
      // operands swapped: the MFMA produces D[j][i] = x[i][j], so each lane ends up
      // with runs of 4 consecutive j of one row i.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32(acc[mt][nt], fb[nt], fa[mt], T());
    }
    if (s + 1 < nst) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: stage the 128 x 128 tile in LDS as [i][j], then 16-byte coalesced stores
  constexpr int XROW = K2_TILE + E;
  T* xs = &lds[0][0][0];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = wm * 64 + mt * 32 + (lane & 31);
        const int j = wn * 64 + nt * 32 + 8 * q + 4 * (lane >> 5);
        *(typename Pack4<T>::type*)(xs + i * XROW + j) =
            Pack4<T>::make(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2],
                           acc[mt][nt][4 * q + 3]);
      }
  __syncthreads();
  T* Xb = X + bc * mat + (size_t)ti * K2_TILE * np + tj * K2_TILE;
  constexpr int CPR = K2_TILE / E;
  for (int idx = tid; idx < K2_TILE * CPR; idx += NTHREADS) {
    const int row = idx / CPR, cc = idx - row * CPR;
    st16(Xb + (size_t)row * np + cc * E, ld16(xs + row * XROW + cc * E));
  }
}

// ---------------------------------------------------------------------------------------
// k3: x tile (all c channels of TP pairs of row i) + z tile -> out.
// Grid (ceil(n / TP), n, batch); pairs (i, j0 + t), t < TP.
template <class T>
__global__ __launch_bounds__(NTHREADS) void k3_output_gate(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ mask,
    T* __restrict__ out, const T* __restrict__ wo, const float* __restrict__ so,
    const float* __restrict__ to, const T* __restrict__ wg, const float* __restrict__ sg,
    const float* __restrict__ tg, int n, int np, int cz, int czp, int c, int cp) {
  constexpr int E = Traits<T>::E;
  constexpr int KG = 4 * E;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int xstride = cp + E, zstride = czp + E;
  const int ostride = 64 + E;  // staging: TP pairs x 64 output channels per round
  T* xs = (T*)smem;
  T* zs = xs + TP * xstride;
  T* os = zs + TP * zstride;
  float* mux = (float*)(os + TP * ostride);
  float* rsx = mux + TP;
  float* muz = rsx + TP;
  float* rsz = muz + TP;
  float* mv = rsz + TP;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bb = blockIdx.z, i = blockIdx.y, j0 = blockIdx.x * TP;

  // 1. x tile, transposed on the way in: x[bb][ch][i][j0 + t] -> xs[t][ch]. Each thread
  //    moves an E x E block (E channels x E pairs) through registers.
  {
    const int cbk = c / E, pbk = TP / E;
    for (int idx = tid; idx < cbk * pbk; idx += NTHREADS) {
      const int cb = idx / pbk, pb = idx - cb * pbk;
      T blk[E][E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const chunk_t v = ld16(x + (((size_t)bb * c + cb * E + e) * np + i) * np + j0 + pb * E);
        const T* pv = (const T*)&v;
#pragma unroll
        for (int f = 0; f < E; ++f) blk[e][f] = pv[f];
      }
#pragma unroll
      for (int f = 0; f < E; ++f) {
        T col[E];
#pragma unroll
        for (int e = 0; e < E; ++e) col[e] = blk[e][f];
        st16(xs + (pb * E + f) * xstride + cb * E, __builtin_bit_cast(chunk_t, col));
      }
    }
    // zero the k padding [c, cp)
    const int padc = (cp - c) / E;
    for (int idx = tid; idx < TP * padc; idx += NTHREADS) {
      const int t = idx / padc, k = idx - t * padc;
      st16(xs + t * xstride + c + k * E, chunk_t{0u, 0u, 0u, 0u});
    }
  }
  // 2. z tile and mask
  {
    const int cpr = czp / E, czc = cz / E;
    for (int idx = tid; idx < TP * cpr; idx += NTHREADS) {
      const int t = idx / cpr, ch = idx - t * cpr;
      const int j = j0 + t;
      chunk_t v = {0u, 0u, 0u, 0u};
      if (ch < czc && j < n) v = ld16(z + (((size_t)bb * n + i) * n + j) * cz + ch * E);
      st16(zs + t * zstride + ch * E, v);
    }
    if (tid < TP) {
      const int j = j0 + tid;
      float m = 0.f;
      if (j < n) m = mask ? to_f32(mask[((size_t)bb * n + i) * n + j]) : 1.f;
      mv[tid] = m;
    }
  }
  __syncthreads();
  row_stats(xs, xstride, c, mux, rsx);
  row_stats(zs, zstride, cz, muz, rsz);
  __syncthreads();

  // accumulator (pair tile pt, register rr): output channel u*16 + 4*(lane/16) + rr,
  // pair pt*16 + lane%16
  float lmx[4], lrx[4], lmz[4], lrz[4], lm[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int t = pt * 16 + (lane & 15);
    lmx[pt] = mux[t];
    lrx[pt] = rsx[t];
    lmz[pt] = muz[t];
    lrz[pt] = rsz[t];
    lm[pt] = mv[t];
  }

  const int units = cz / 16;
  const int kx = cp / KG, kz = czp / KG;
  for (int u0 = 0; u0 < units; u0 += 4) {
    const int u = u0 + wave;
    if (u < units) {
      const int orow = u * 16 + (lane & 15);
      const T* wor = wo + (size_t)orow * cp + (lane >> 4) * E;
      const T* wgr = wg + (size_t)orow * czp + (lane >> 4) * E;
      f32x4 ap[4], ag[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) ap[pt] = ag[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < kx; ++ks) {
        const chunk_t wa = ld16(wor + ks * KG);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const chunk_t xf = ld16(xs + (pt * 16 + (lane & 15)) * xstride + ks * KG + (lane >> 4) * E);
          ap[pt] = mma16(ap[pt], wa, xf, T());
        }
      }
      for (int ks = 0; ks < kz; ++ks) {
        const chunk_t wa = ld16(wgr + ks * KG);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const chunk_t zf = ld16(zs + (pt * 16 + (lane & 15)) * zstride + ks * KG + (lane >> 4) * E);
          ag[pt] = mma16(ag[pt], wa, zf, T());
        }
      }
      float cso[4], cto[4], csg[4], ctg[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int oc = u * 16 + 4 * (lane >> 4) + rr;
        cso[rr] = so[oc];
        cto[rr] = to[oc];
        csg[rr] = sg[oc];
        ctg[rr] = tg[oc];
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        float v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = lrx[pt] * (ap[pt][rr] - lmx[pt] * cso[rr]) + cto[rr];
          const float g = lrz[pt] * (ag[pt][rr] - lmz[pt] * csg[rr]) + ctg[rr];
          v[rr] = lm[pt] * p * sigmoidf_fast(g);
        }
        *(typename Pack4<T>::type*)(os + (pt * 16 + (lane & 15)) * ostride + wave * 16 + 4 * (lane >> 4)) =
            Pack4<T>::make(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
    // staged round -> out[bb][i][j0 + t][u0*16 .. u0*16 + nu*16)
    const int nu = min(4, units - u0);
    const int cpp = nu * 16 / E;  // chunks per pair
    for (int idx = tid; idx < TP * cpp; idx += NTHREADS) {
      const int t = idx / cpp, cc = idx - t * cpp;
      const int j = j0 + t;
      if (j < n)
        st16(out + (((size_t)bb * n + i) * n + j) * cz + u0 * 16 + cc * E,
             ld16(os + t * ostride + cc * E));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// launchers

template <class T>
static size_t k1_lds(int czp) {
  constexpr int E = Traits<T>::E;
  return (size_t)TP * (czp + E) * sizeof(T) + 3 * TP * sizeof(float) +
         (size_t)4 * 16 * (TP + E) * sizeof(T);
}
template <class T>
static size_t k3_lds(int czp, int cp) {
  constexpr int E = Traits<T>::E;
  return ((size_t)TP * (cp + E) + (size_t)TP * (czp + E) + (size_t)TP * (64 + E)) * sizeof(T) +
         5 * TP * sizeof(float);
}

// Raises a kernel's dynamic-LDS limit when a launch needs more than was granted so
// far (the limit is a per-function attribute; `granted` tracks it per instantiation).
static hipError_t ensure_lds(const void* fn, std::atomic<int>& granted, size_t need) {
  if ((int)need <= granted.load(std::memory_order_relaxed)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)need);
  if (e == hipSuccess) {
    int cur = granted.load();
    while ((int)need > cur && !granted.compare_exchange_weak(cur, (int)need)) {
    }
  }
  return e;
}

template <class T>
static hipError_t launch_stage_t(int stage, const StageArgs& a, hipStream_t st) {
  static std::atomic<int> k1_granted{0}, k3_granted{0};
  if (stage == 1) {
    const size_t lds = k1_lds<T>(a.czp);
    auto fn = k1_input_gate<T>;
    hipError_t e = ensure_lds((const void*)fn, k1_granted, lds);
    if (e != hipSuccess) return e;
    dim3 grid(a.np / TP, a.np, a.batch);
    hipLaunchKernelGGL(fn, grid, dim3(NTHREADS), lds, st, (const T*)a.z, (const T*)a.mask,
                       (T*)a.a, (T*)a.b, (const T*)a.w1, a.s1, a.t1, a.n, a.np, a.cz, a.czp, a.c,
                       a.incoming);
  } else if (stage == 2) {
    const size_t t1d = a.np / K2_TILE;
    dim3 grid((unsigned)(t1d * t1d * (size_t)a.batch * a.c));
    hipLaunchKernelGGL(k2_contract<T>, grid, dim3(NTHREADS), 0, st, (const T*)a.a, (const T*)a.b,
                       (T*)a.x, a.np);
  } else {
    const size_t lds = k3_lds<T>(a.czp, a.cp);
    auto fn = k3_output_gate<T>;
    hipError_t e = ensure_lds((const void*)fn, k3_granted, lds);
    if (e != hipSuccess) return e;
    dim3 grid((a.n + TP - 1) / TP, a.n, a.batch);
    hipLaunchKernelGGL(fn, grid, dim3(NTHREADS), lds, st, (const T*)a.x, (const T*)a.z,
                       (const T*)a.mask, (T*)a.out, (const T*)a.wo, a.so, a.to, (const T*)a.wg, a.sg,
                       a.tg, a.n, a.np, a.cz, a.czp, a.c, a.cp);
  }
  return hipGetLastError();
}

hipError_t launch_stage(int stage, bool bf16_storage, const StageArgs& a, hipStream_t st) {
  return bf16_storage ? launch_stage_t<bf16>(stage, a, st) : launch_stage_t<float>(stage, a, st);
}

size_t stage_lds_bytes(int stage, bool bf16_storage, int czp, int cp) {
  if (stage == 1) return bf16_storage ? k1_lds<bf16>(czp) : k1_lds<float>(czp);
  if (stage == 3) return bf16_storage ? k3_lds<bf16>(czp, cp) : k3_lds<float>(czp, cp);
  return bf16_storage ? sizeof(bf16) * 2 * 2 * K2_TILE * 72 : sizeof(float) * 2 * 2 * K2_TILE * 36;
}

}  // namespace trimul
