// k3 (streamed weights): the output gate for wide pair tracks, bf16, c_z > 128.
//   out = m * sigmoid(W_g zhat + b_g) * (W_o LN_c(x) + b_o)      [+ z with the residual]
// RFProteína architecture page, "Triangle multiplication on SM90" (K3: the output gate and
// projection with both LayerNorms folded in) and "Dual-GEMM gates" (the x0_x1 form); the
// pair width of 384 is the generative trunk's ("Inside the velocity network").
//
// At c_z = 384 the output gate's weights (W_o 384 x 128 and W_g 384 x 384, 393 KB in
// bf16) do not fit one workgroup's LDS. Splitting the output channels over workgroups
// makes every group read x and z again. Here one workgroup produces all c_z channels of
// its pairs and streams the weights through LDS instead, one pair of output units (32
// channels: W_o and W_g rows, 32 (c + c_z) bf16 values each) per step, into one of two
// buffers by direct global-to-LDS loads while the waves compute on the other:
//   - a workgroup step gives each of its 8 waves 16 consecutive pairs of one row;
//   - x arrives channel-major (16-byte chunks of 8 pairs of one channel), is transposed
//     through a per-wave LDS staging tile into MFMA operand layout (lane (p, q) holds
//     chunk ks*4 + q of pair p) and layer-normalised in registers; z arrives in operand
//     layout and is normalised in place as the gate's B operand (with the residual, each
//     output chunk's raw z is read again just before it is stored);
//   - per output unit: W_o rows x xhat and W_g rows x zhat (A = weight rows, B = the
//     pairs), start values from LDS, m * p / (1 + 2^g) in registers. The rows of a unit
//     pair are stored so that lane (p, q) ends with channels 32k + 8q .. 32k + 8q + 7 of
//     pair p: one 16-byte store (with the residual, added to its own raw z chunk);
//   - the next step's x and mask loads go out at the start of the last weight step, its z
//     loads once the last MFMA has read the current z.
// Chunk c of a weight row r sits at position c ^ (r & 15) in LDS (the host stores it that
// way, so the copy is linear), which keeps the operand reads free of bank conflicts.
// One workgroup owns each pair from its reads to its store, so out may be z.

#include "device_common.h"

namespace trimul {

constexpr int K3S_WAVES = 8;
constexpr int K3S_THREADS = 64 * K3S_WAVES;

// 16 bytes per lane through a buffer resource straight into LDS (lane i writes
// lds_base + 16 i); counted by vmcnt.
__device__ __forceinline__ void k3s_lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned int voff,
                                              void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, (int)voff, 0, 0, 0);
}

template <int KXM, int KZM, bool RESID>
__global__ __launch_bounds__(K3S_THREADS) void k3_output_gate_stream(
    const bf16* __restrict__ x, ZIn<bf16, RESID> z, const bf16* __restrict__ mask,
    ZOut<bf16, RESID> out, const unsigned char* __restrict__ image, int n, int np, int cz, int c,
    int mask_all, int items) {
  using T = bf16;
  constexpr int E = 8, KG = 32;
  constexpr int CP = KXM * KG, CZP = KZM * KG;
  constexpr int GB = 64 * (CP + CZP);     // one step's weights: 32 rows of W_o and of W_g
  constexpr int WOB = 64 * CP;            // its W_o part
  static_assert(GB % (1024 * K3S_WAVES) == 0, "whole 1 KB blocks per wave");
  constexpr int BPW = GB / 1024 / K3S_WAVES;
  constexpr int STEPS = CZP / 32;         // unit pairs
  constexpr int SST = CP + E;             // x staging row stride (elements)
  constexpr int XCH = 16 * CP / E / 32;   // x chunks per lane of the 32 loading lanes (8)
  static_assert(XCH == 8 || XCH == 16, "an 8 x 8 transpose per chunk block");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* const wbuf = smem;                          // [2][GB]
  float* const tos = (float*)(smem + 2 * GB);               // [CZP] kernel row order
  float* const tgs = tos + CZP;                              // [CZP]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const stg = (T*)(tgs + CZP) + wave * 16 * SST;         // per-wave x staging [16][SST]
  const int p = lane & 15, q = lane >> 4;

  {
    const float* src = (const float*)(image + (size_t)STEPS * GB);
    for (int k = tid; k < 2 * CZP; k += K3S_THREADS) tos[k] = src[k];
  }
  const __amdgpu_buffer_rsrc_t rimg = buffer_rsrc(image, (size_t)STEPS * GB);
  auto issue = [&](int s) {
    const int g = s % STEPS;
    unsigned char* dst = wbuf + (s & 1) * GB;
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int blk = wave * BPW + k;
      k3s_lds_dma16(rimg, (unsigned int)((size_t)g * GB + blk * 1024 + lane * 16), dst + blk * 1024);
    }
  };

  // item = 16 consecutive pairs (i, j0 .. j0 + 15) of one row of one batch item
  const int nt = (n + 15) / 16;
  // x: the 32 loading lanes l take channel block cb = l % 16 (channels 8 cb .. of every
  // 128 channels) and pair half h = l / 16; chunk k is channel 8 cb + k % 8 + 128 (k / 8)
  const bool xl = lane < 32;
  const int xcb = lane & 15, xh = (lane >> 4) & 1;
  // x and the mask of an item go to `f`; its z goes straight into the operand registers
  // (raw, normalised in place when the item starts)
  struct Pre {
    chunk_t xv[XCH];
    T m;
  };
  chunk_t za[KZM];
  auto fetch_z = [&](int it) {
    const int itc = it < items ? it : items - 1;
    const int bb = itc / (n * nt), rem = itc - bb * n * nt, i = rem / nt;
    const int j0 = (rem - i * nt) * 16;
    const int live = it < items ? min(16, n - j0) : 0;
    const size_t pair0 = ((size_t)bb * n + i) * n + j0;
    const __amdgpu_buffer_rsrc_t rz =
        buffer_rsrc(z + pair0 * cz, (size_t)live * cz * sizeof(T));
    const unsigned int zoff = (unsigned int)((p * cz + q * E) * sizeof(T));
#pragma unroll
    for (int ks = 0; ks < KZM; ++ks)
      za[ks] = ks * KG + q * E < cz ? load16(rz, zoff + ks * KG * (unsigned int)sizeof(T), 0)
                                    : chunk_t{0u, 0u, 0u, 0u};
  };
  auto fetch = [&](int it, Pre& f) {
    const int itc = it < items ? it : items - 1;  // past the end: refetch the last item
    const int bb = itc / (n * nt), rem = itc - bb * n * nt, i = rem / nt;
    const int j0 = (rem - i * nt) * 16;
    const int live = it < items ? min(16, n - j0) : 0;  // real pairs of the item
    // x of this item's pairs: channel planes of one batch item (below 2 GiB at launch)
    const __amdgpu_buffer_rsrc_t rx =
        buffer_rsrc(x + (size_t)bb * c * np * np, (size_t)c * np * np * sizeof(T));
    const unsigned int xrow = (unsigned int)(((size_t)i * np + j0 + 8 * xh) * sizeof(T));
#pragma unroll
    for (int k = 0; k < XCH; ++k) {
      const int ch = 8 * xcb + k % 8 + 128 * (k / 8);
      const unsigned int off = (unsigned int)((size_t)(ch < c ? ch : 0) * np * np * sizeof(T)) + xrow;
      f.xv[k] = (xl && ch < c && live > 8 * xh) ? load16(rx, off, 0) : chunk_t{0u, 0u, 0u, 0u};
    }
    const size_t pair0 = ((size_t)bb * n + i) * n + j0;
    const __amdgpu_buffer_rsrc_t rm =
        buffer_rsrc(mask_all ? mask : mask + pair0, mask_all ? (live ? sizeof(T) : 0) : live * sizeof(T));
    f.m = load_elem(rm, mask_all ? 0u : (unsigned int)(p * sizeof(T)), 0, T());
  };

  const int wb = blockIdx.x, nwb = gridDim.x;
  const int steps_total = (items + K3S_WAVES - 1) / K3S_WAVES;  // workgroup steps
  Pre f;
  int s = 0;  // weight-stream step
  issue(0);
  fetch(wb * K3S_WAVES + wave, f);
  fetch_z(wb * K3S_WAVES + wave);
  for (int ws = wb; ws < steps_total; ws += nwb) {
    const int it = ws * K3S_WAVES + wave;
    const int itc = it < items ? it : items - 1;
    const int bb = itc / (n * nt), rem = itc - bb * n * nt, i = rem / nt;
    const int j0 = (rem - i * nt) * 16;
    const int live = it < items ? min(16, n - j0) : 0;

    // x: 8 x 8 blocks (8 channels x 8 pairs) transposed in registers into pair-major
    // staging rows, then read back in operand layout
    if (xl) {
#pragma unroll
      for (int kb = 0; kb < XCH / 8; ++kb) {
        T tb[8][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const T* pv = (const T*)&f.xv[8 * kb + e];
#pragma unroll
          for (int ff = 0; ff < 8; ++ff) tb[e][ff] = pv[ff];
        }
#pragma unroll
        for (int ff = 0; ff < 8; ++ff) {
          T col[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) col[e] = tb[e][ff];
          st16(stg + (8 * xh + ff) * SST + 8 * xcb + 128 * kb, __builtin_bit_cast(chunk_t, col));
        }
      }
    }
    chunk_t bx[KXM];
    const float mv = p < live ? to_f32(f.m) : 0.f;
    wave_lds_sync();
#pragma unroll
    for (int ks = 0; ks < KXM; ++ks) bx[ks] = ld16(stg + p * SST + (ks * 4 + q) * E);
    normalize_operand_row<KXM>(bx, c, lane, T());
    normalize_operand_row<KZM>(za, cz, lane, T());
    const size_t pair = ((size_t)bb * n + i) * n + j0 + p;  // this lane's pair

#pragma unroll 1
    for (int k = 0; k < STEPS; ++k, ++s) {
      // step s's weights are in LDS once this thread's loads are done and every wave is
      // past the barrier; every wave is then also done with the other buffer
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(s + 1);
      const int next = (ws + nwb) * K3S_WAVES + wave;  // this wave's item of the next step
      if (k == STEPS - 1) fetch(next, f);                // its x and mask
      // with the residual: the raw z chunk this lane's output of the step is added to (out
      // may be z: it is read before the store below, by the same lane)
      chunk_t zres = {0u, 0u, 0u, 0u};
      if constexpr (RESID)
        if (p < live && 32 * k + 8 * q < cz) zres = ld16(z + pair * cz + 32 * k + 8 * q);
      const unsigned char* gbuf = wbuf + (s & 1) * GB;
      const T* const wo = (const T*)gbuf;          // [32][CP], swizzled
      const T* const wg = (const T*)(gbuf + WOB);  // [32][CZP], swizzled
      float o[8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 16 * u + p;
        f32x4 ap = ld16f(tos + 32 * k + 16 * u + 4 * q);
        f32x4 ag = ld16f(tgs + 32 * k + 16 * u + 4 * q);
#pragma unroll
        for (int ks = 0; ks < KXM; ++ks)
          ap = mma16(ap, ld16(wo + row * CP + (((ks * 4 + q) ^ p) * E)), bx[ks], T());
#pragma unroll
        for (int ks = 0; ks < KZM; ++ks)
          ag = mma16(ag, ld16(wg + row * CZP + (((ks * 4 + q) ^ p) * E)), za[ks], T());
#pragma unroll
        for (int r = 0; r < 4; ++r) o[4 * u + r] = gate_mul(ap[r] * mv, ag[r]);
      }
      if (k == STEPS - 1) fetch_z(next);  // za is free: the next item's z
      // channels 32k + 8q .. + 7 of this lane's pair (real channels only: c_z is a
      // multiple of 16, so a chunk is all real or all padding)
      if (p < live && 32 * k + 8 * q < cz) {
        chunk_t v = pack(o, T());
        if constexpr (RESID) v = add_chunks(v, zres, T());
        __builtin_nontemporal_store(v, (chunk_t*)(out + pair * cz + 32 * k + 8 * q));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // the stream's one extra step lands before exit
}

// LDS of the streamed form: two weight steps, the start values, the x staging tiles
size_t k3_stream_lds(int cp, int czp) {
  return (size_t)2 * 64 * (cp + czp) + (size_t)2 * czp * 4 +
         (size_t)K3S_WAVES * 16 * (cp + 8) * 2;
}

template <int KXM, int KZM, bool RESID>
static hipError_t launch_k3s(const StageArgs& a, hipStream_t st) {
  const size_t lds = k3_stream_lds(a.cp, a.czp);
  auto fn = k3_output_gate_stream<KXM, KZM, RESID>;
  static std::atomic<int> granted{0};
  hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
  if (e != hipSuccess) return e;
  const long long items = (long long)a.batch * a.n * ((a.n + 15) / 16);
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  static std::atomic<int> occ{0};
  static std::atomic<size_t> occ_lds{0};
  const int per_cu = resident_blocks((const void*)fn, K3S_THREADS, lds, occ, occ_lds);
  const long long wsteps = (items + K3S_WAVES - 1) / K3S_WAVES;
  const long long cap = (long long)a.num_cus * per_cu;
  const int blocks = (int)(wsteps < cap ? wsteps : cap);
  const int mask_all = a.mask == nullptr;
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(K3S_THREADS), lds, st, (const bf16*)a.x,
                     (const bf16*)a.z, (const bf16*)(mask_all ? a.one : a.mask), (bf16*)a.out,
                     (const unsigned char*)a.k3s_image, a.n, a.np, a.cz, a.c, mask_all,
                     (int)items);
  return hipGetLastError();
}

// The streamed form if it is compiled for the padded widths and fits LDS: *done = false
// leaves the launch to the other forms.
hipError_t launch_k3_stream(const StageArgs& a, hipStream_t st, bool* done) {
  *done = false;
  if (!a.k3s_image) return hipSuccess;
  if ((size_t)a.c * a.np * a.np * 2 >= 0x80000000ull) return hipSuccess;  // 32-bit x offsets
  if (a.plan) {
    a.plan->k3_form = 2;
    a.plan->k3_groups = 1;
    *done = true;
    return hipSuccess;
  }
  *done = true;
  const int kx = a.cp / 32, kz = a.czp / 32;
#define TRIMUL_K3S(X_, Z_)                                                          \
  if (kx == X_ && kz == Z_)                                                         \
    return a.residual ? launch_k3s<X_, Z_, true>(a, st) : launch_k3s<X_, Z_, false>(a, st);
  TRIMUL_K3S_VARIANTS(TRIMUL_K3S)
#undef TRIMUL_K3S
  *done = false;
  return hipSuccess;
}

}  // namespace trimul
