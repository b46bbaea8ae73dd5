// k0: the mask extents of each batch item, the input of the contraction's work skipping.
//
// RFProteína architecture page, "Dual-GEMM gates": the input gate takes the left-aligned
// pair mask as per-row valid counts that are computed once per forward and reused by
// every pair update of that forward. For a pair mask that is the outer product of a
// left-aligned residue mask every valid row has the same count L, so one number per item
// carries it. Here that number is defined for any mask: L_b = 1 + the largest max(i, j)
// over the nonzero entries of item b (0 when there is none), the side of the smallest
// leading square that holds every nonzero pair. Outside that square a and b are zero, so
// the contraction over k stops at L_b and output tiles past it are zero.
//
// Grid (TRI_MUL_EXTENT_PARTS, batch): workgroup g of item b scans residue rows
// [n g / P, n (g + 1) / P) and writes its partial maximum to parts[b][g]; readers take the
// maximum of the P parts (one 64-lane load). No atomics, so nothing has to be cleared
// before the launch, and the buffer may be reused as is.

#include "device_common.h"
#include "tri_mul.h"

namespace trimul {

constexpr int K0_THREADS = 1024;
static_assert(TRI_MUL_EXTENT_PARTS == 64, "one part per lane of a wave");

template <class T>
__global__ __launch_bounds__(K0_THREADS) void k0_mask_extents(const T* __restrict__ mask, int n,
                                                              int* __restrict__ parts) {
  __shared__ int wmax[K0_THREADS / 64];
  const int g = blockIdx.x, bb = blockIdx.y;
  const int r0 = (int)((long long)n * g / TRI_MUL_EXTENT_PARTS);
  const int r1 = (int)((long long)n * (g + 1) / TRI_MUL_EXTENT_PARTS);
  // the rows' entries are one contiguous run: thread k takes entries e0 + k + 1024 m, eight
  // loads in flight before their compares
  // (an item has at most 2^30 entries: 32-bit indices)
  const T* const mb = mask + (size_t)bb * n * n;
  const unsigned int e0 = (unsigned int)r0 * n, e1 = (unsigned int)r1 * n;
  int ext = 0;
  for (unsigned int base = e0 + threadIdx.x; base < e1; base += 8 * K0_THREADS) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned int e = base + u * K0_THREADS;
      v[u] = e < e1 ? to_f32(mb[e]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (v[u] != 0.f) {
        const unsigned int e = base + u * K0_THREADS;
        const unsigned int i = e / (unsigned int)n, j = e - i * (unsigned int)n;
        ext = max(ext, (int)max(i, j) + 1);
      }
    }
  }
  ext = wave_max(ext);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = ext;
  __syncthreads();
  if (threadIdx.x < 64) {
    int v = threadIdx.x < K0_THREADS / 64 ? wmax[threadIdx.x] : 0;
    v = wave_max(v);
    if (threadIdx.x == 0) parts[bb * TRI_MUL_EXTENT_PARTS + g] = v;
  }
}

hipError_t launch_k0(bool bf16_storage, const void* mask, int batch, int n, int* parts,
                     hipStream_t st) {
  const dim3 grid(TRI_MUL_EXTENT_PARTS, batch);
  if (bf16_storage)
    hipLaunchKernelGGL(k0_mask_extents<bf16>, grid, dim3(K0_THREADS), 0, st, (const bf16*)mask, n,
                       parts);
  else
    hipLaunchKernelGGL(k0_mask_extents<float>, grid, dim3(K0_THREADS), 0, st, (const float*)mask,
                       n, parts);
  return hipGetLastError();
}

}  // namespace trimul
