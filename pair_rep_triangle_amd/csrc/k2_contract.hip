// k2: the contraction over the third residue, one NT GEMM per (batch, channel):
//   x[bc][i][j] = sum_k A[bc][i][k] * B[bc][j][k]
// RFProteína architecture page, "Triangle multiplication on SM90": K2 performs the
// contraction itself, compiled per direction. Here the direction is absorbed by the
// input-gate kernel's store layout (it writes the incoming operands transposed), so one
// kernel serves both.

#include "device_common.h"

namespace trimul {

constexpr int NTHREADS = 256;

// k2: x[bc] = A[bc] B[bc]^T for every (batch, channel) bc; A, B, x are [np][np].
// 128 x 128 output tile per workgroup, 4 waves as 2 x 2, each 64 x 64 (2 x 2 MFMA
// 32x32 tiles). k advances 128 bytes per stage through a double-buffered LDS, with two
// stages of global loads in flight.
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

  // Global -> registers -> LDS, two stages in flight: the loads of stage s+2 are issued
  // before stage s is computed and land in LDS after it, so two stages of MFMA work cover
  // the memory latency. The two register sets alternate (the loop is unrolled by two so
  // that every register index is static).
  chunk_t ra[2][4], rb[2][4];
  auto gload = [&](int set, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NTHREADS * q, row = idx >> 3, c16 = idx & 7;
      ra[set][q] = ld16(Ab + (size_t)row * np + k0 + c16 * E);
      rb[set][q] = ld16(Bb + (size_t)row * np + k0 + c16 * E);
    }
  };
  auto lstore = [&](int buf, int set) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NTHREADS * q, row = idx >> 3, c16 = idx & 7;
      st16(&lds[buf][0][row * LROW + c16 * E], ra[set][q]);
      st16(&lds[buf][1][row * LROW + c16 * E], rb[set][q]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int cur) {
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
  };

  // stage s lives in LDS buffer s % 2 and (while in flight) register set s % 2
  const int nst = np / KT;  // even: np is a multiple of 128 and KT is 64 or 32
  gload(0, 0);
  gload(1, KT);
  lstore(0, 0);
  __syncthreads();
  for (int s = 0; s < nst; s += 2) {
    // even stage s: buffer 0 holds it, set 1 holds s+1, set 0 is free
    if (s + 2 < nst) gload(0, (s + 2) * KT);
    compute(0);
    lstore(1, 1);  // stage s+1 always exists (nst even)
    __syncthreads();
    // odd stage s+1: buffer 1 holds it, set 0 holds s+2 (if any), set 1 is free
    if (s + 3 < nst) gload(1, (s + 3) * KT);
    compute(1);
    if (s + 2 < nst) lstore(0, 0);
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
        store4(xs + i * XROW + j, acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1],
               acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
      }
  __syncthreads();
  T* Xb = X + bc * mat + (size_t)ti * K2_TILE * np + tj * K2_TILE;
  constexpr int CPR = K2_TILE / E;
  for (int idx = tid; idx < K2_TILE * CPR; idx += NTHREADS) {
    const int row = idx / CPR, cc = idx - row * CPR;
    st16(Xb + (size_t)row * np + cc * E, ld16(xs + row * XROW + cc * E));
  }
}


hipError_t launch_k2(bool bf16_storage, const StageArgs& a, hipStream_t st) {
  const size_t t1d = a.np / K2_TILE;
  dim3 grid((unsigned)(t1d * t1d * (size_t)a.batch * a.c));
  if (bf16_storage)
    hipLaunchKernelGGL(k2_contract<bf16>, grid, dim3(NTHREADS), 0, st, (const bf16*)a.a,
                       (const bf16*)a.b, (bf16*)a.x, a.np);
  else
    hipLaunchKernelGGL(k2_contract<float>, grid, dim3(NTHREADS), 0, st, (const float*)a.a,
                       (const float*)a.b, (float*)a.x, a.np);
  return hipGetLastError();
}

}  // namespace trimul
