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
// channels: W_o and W_g rows, 32 (c + c_z) bf16 values each) per step, by direct
// global-to-LDS loads into a ring of three buffers, two steps ahead of the compute:
//   - a workgroup step gives each of its 8 waves 16 consecutive pairs of one row;
//   - x arrives channel-major (16-byte chunks of 8 pairs of one channel), is transposed
//     through a per-wave LDS staging tile into MFMA operand layout (lane (p, q) holds
//     chunk ks*4 + q of pair p) and layer-normalised in registers; z arrives in operand
//     layout and is normalised in place as the gate's B operand (with the residual, each
//     output chunk's raw z is read again at the start of the step that stores it);
//   - per output unit: W_o rows x xhat and W_g rows x zhat (A = weight rows, B = the
//     pairs), start values from LDS, m * p / (1 + 2^g) in registers. The rows of a unit
//     pair are stored so that lane (p, q) ends with channels 32k + 8q .. 32k + 8q + 7 of
//     pair p: one 16-byte store (with the residual, added to its own raw z chunk);
//   - the next item's x and mask loads go out at the start of the current item's last
//     weight step, its z loads once that step's gate products have read the current z;
//   - every step issues exactly one store (chunks of padded pairs and channels fall outside
//     the buffer range and are dropped), so the wait for a step's weights can leave the
//     previous step's store in flight instead of waiting for it;
//   - the weight operands are read a few products ahead through a small register ring, at
//     per-lane LDS offsets fixed for the kernel plus the buffer base and immediates.
// Chunk c of a weight row r sits at position c ^ (r & 15) in LDS (the host stores it that
// way, so the copy is linear), which keeps the operand reads free of bank conflicts.
// One workgroup owns each pair from its reads to its store, so out may be z.

#include "device_common.h"

namespace trimul {

constexpr int K3S_WAVES = 8;
constexpr int K3S_BUFS = 3;  // weight steps in LDS: the one in use and two in flight
static_assert(K3S_BUFS == 3, "the loads two steps ahead refill the previous step's buffer");
constexpr int K3S_THREADS = 64 * K3S_WAVES;

// s_waitcnt operand: vmcnt(n) (6 bits, split over two fields), lgkmcnt(0), expcnt off
constexpr int k3s_waitcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

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
  static_assert(CP == 128, "x of an item: 128 channels x 16 pairs, four 1 KB loads");
  // the vector memory operations issued after a step's weight loads until the wait for
  // them (see the step loop): in steady state the next step's weight loads, two stores
  // and, with the residual, two z reads; in the first two steps of an item also the next
  // item's loads (four of x, the mask, KZM z chunks)
  constexpr int K3S_WAIT = k3s_waitcnt(BPW + 2 + (RESID ? 2 : 0));
  constexpr int K3S_WAIT_FIRST = k3s_waitcnt(BPW + 2 + (RESID ? 2 : 0) + 4 + 1 + KZM);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* const wbuf = smem;                          // [K3S_BUFS][GB]
  float* const tos = (float*)(smem + K3S_BUFS * GB);        // [CZP] kernel row order
  float* const tgs = tos + CZP;                              // [CZP]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* const stg = (T*)(tgs + CZP) + wave * 16 * SST;         // per-wave x staging [16][SST]
  unsigned char* const stgb = (unsigned char*)stg;
  const int p = lane & 15, q = lane >> 4;

  {
    const float* src = (const float*)(image + (size_t)STEPS * GB);
    for (int k = tid; k < 2 * CZP; k += K3S_THREADS) tos[k] = src[k];
  }
  const __amdgpu_buffer_rsrc_t rimg = buffer_rsrc(image, (size_t)STEPS * GB);
  // weight step g into buffer b: block k of this wave is bytes (wave * BPW + k) KB of the
  // step; the block's global offset rides in the scalar offset (the immediate offset of an
  // LDS load would move the LDS address as well)
  const unsigned int dma_off = (unsigned int)(wave * BPW * 1024 + lane * 16);
  auto issue = [&](int g, int b) {
    unsigned char* dst = wbuf + b * GB + wave * BPW * 1024;
#pragma unroll
    for (int k = 0; k < BPW; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rimg, (__attribute__((address_space(3))) void*)(dst + k * 1024), 16, (int)dma_off,
          g * GB + k * 1024, 0, 0);
  };

  // item = 16 consecutive pairs (i, j0 .. j0 + 15) of one row of one batch item
  const int nt = (n + 15) / 16;
  const unsigned int plane = (unsigned int)np * np * sizeof(T);  // one channel plane of x
  // x of the next item arrives by direct loads into this wave's staging tile, channel-major:
  // 256 chunks of 16 bytes (chunk m = 2 ch + h: channel ch, pairs 8h .. 8h + 7 of the
  // item), chunk m at slot 16 (m >> 4) + ((m & 15) ^ (m >> 4)) (the map is its own
  // inverse), which keeps the reads of the transpose below free of bank conflicts; load j,
  // lane l fills slot 64 j + l. Channels at or past c get an offset past every range check
  // (no memory access; the transpose zeroes them), so the loads need no branch.
  constexpr unsigned int OUT_OF_RANGE = 0x80000000u;
  const bool xl = lane < 32;
  const int xcb = lane & 15, xh = (lane >> 4) & 1;
  unsigned int xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = 64 * j + lane;
    const int m = 16 * (sl >> 4) + ((sl & 15) ^ (sl >> 4));
    xoff[j] = (m >> 1) < c ? (unsigned int)(m >> 1) * plane + 16u * (m & 1) : OUT_OF_RANGE;
  }
  // the mask of an item goes to fm; its z goes straight into the operand registers (raw,
  // normalised in place when the item starts)
  T fm;
  chunk_t za[KZM];
  // the next item's raw z, loaded a whole item ahead where the registers allow it
  constexpr bool PF_Z = KZM <= 12;
  chunk_t zn[PF_Z ? KZM : 1];
  auto item_of = [&](int it, int& bb, int& i, int& j0, int& live) {
    const int itc = it < items ? it : items - 1;  // past the end: the last item, no pairs
    bb = itc / (n * nt);
    const int rem = itc - bb * n * nt;
    i = rem / nt;
    j0 = (rem - i * nt) * 16;
    live = it < items ? min(16, n - j0) : 0;
  };
  // lane (p, q) holds chunks 4 ks + q of pair p, channels 32 ks + 8 q .. + 7; c_z is a
  // multiple of 16, so a chunk is all real or all padding: the first klim chunks of the
  // lane are real (the same offsets serve the output chunks of the weight steps)
  const unsigned int ooff = (unsigned int)((p * cz + 8 * q) * sizeof(T));
  const int klim = (cz - 8 * q + 31) / 32;
  auto fetch_z = [&](int it, chunk_t (&dst)[KZM]) {
    int bb, i, j0, live;
    item_of(it, bb, i, j0, live);
    const size_t pair0 = ((size_t)bb * n + i) * n + j0;
    const __amdgpu_buffer_rsrc_t rz =
        buffer_rsrc(z + pair0 * cz, (size_t)live * cz * sizeof(T));
#pragma unroll
    for (int ks = 0; ks < KZM; ++ks)
      dst[ks] = load16(rz, ks < klim ? ooff : OUT_OF_RANGE, ks * KG * (int)sizeof(T));
  };
  auto fetch = [&](int it) {
    int bb, i, j0, live;
    item_of(it, bb, i, j0, live);
    // x from pair (i, j0) of channel 0 of this batch item on (below 2 GiB at launch);
    // pairs past the item's end are still inside row i of the padded planes
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(
        x + ((size_t)bb * c * np + i) * np + j0, (size_t)c * plane);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(stgb + j * 1024), 16, (int)xoff[j], 0, 0, 0);
    const size_t pair0 = ((size_t)bb * n + i) * n + j0;
    const __amdgpu_buffer_rsrc_t rm =
        buffer_rsrc(mask_all ? mask : mask + pair0, mask_all ? (live ? sizeof(T) : 0) : live * sizeof(T));
    fm = load_elem(rm, mask_all ? 0u : (unsigned int)(p * sizeof(T)), 0, T());
  };

  // per-lane LDS offsets of the weight operands: chunk ks = 4a + b of row 16u + p sits at
  // byte 256a + 16((4b + q) ^ p) of its row (p < 16), so four offsets per matrix serve
  // every chunk and the rest is an immediate
  unsigned int lo[4], lg[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const unsigned int sw = 16u * ((4 * b + q) ^ p);
    lo[b] = (unsigned int)(p * CP * 2) + sw;
    lg[b] = (unsigned int)(WOB + p * CZP * 2) + sw;
  }

  const int wb = blockIdx.x, nwb = gridDim.x;
  const int steps_total = (items + K3S_WAVES - 1) / K3S_WAVES;  // workgroup steps
  int buf = 0;  // the buffer of the current weight step
  issue(0, 0);
  issue(1, 1);
  fetch(wb * K3S_WAVES + wave);
  if constexpr (PF_Z) fetch_z(wb * K3S_WAVES + wave, zn);
  else fetch_z(wb * K3S_WAVES + wave, za);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the first item is in
  for (int ws = wb; ws < steps_total; ws += nwb) {
    const int it = ws * K3S_WAVES + wave;
    int bb, i, j0, live;
    item_of(it, bb, i, j0, live);
    const size_t pair0 = ((size_t)bb * n + i) * n + j0;

    // x: lane (cb, h) < 32 takes channels 8 cb .. 8 cb + 7 of pairs 8h .. 8h + 7 (chunks
    // m = 16 cb + 2k + h) and transposes the 8 x 8 block in registers into pair-major
    // staging rows, which are read back in operand layout
    chunk_t xv[8];
    if (xl) {
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = ld16(stgb + 16 * (16 * xcb + ((2 * k + xh) ^ xcb)));
    }
    const float mv = p < live ? to_f32(fm) : 0.f;
    wave_lds_sync();
    if (xl) {
      T tb[8][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const chunk_t v = 8 * xcb < c ? xv[e] : chunk_t{0u, 0u, 0u, 0u};
        const T* pv = (const T*)&v;
#pragma unroll
        for (int ff = 0; ff < 8; ++ff) tb[e][ff] = pv[ff];
      }
#pragma unroll
      for (int ff = 0; ff < 8; ++ff) {
        T col[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) col[e] = tb[e][ff];
        st16(stg + (8 * xh + ff) * SST + 8 * xcb, __builtin_bit_cast(chunk_t, col));
      }
    }
    chunk_t bx[KXM];
    if constexpr (PF_Z) {
#pragma unroll
      for (int ks = 0; ks < KZM; ++ks) za[ks] = zn[ks];
    }
    wave_lds_sync();
#pragma unroll
    for (int ks = 0; ks < KXM; ++ks) bx[ks] = ld16(stg + p * SST + (ks * 4 + q) * E);
    // the next item's x (into the tile, once the reads above are done), mask (and z) go
    // out now: the waits of this item's first two weight steps leave them in flight
    wave_lds_sync();
    const int next = (ws + nwb) * K3S_WAVES + wave;  // this wave's item of the next step
    fetch(next);
    if constexpr (PF_Z) fetch_z(next, zn);
    asm volatile("" ::: "memory");
    normalize_operand_row<KXM>(bx, c, lane, T());
    normalize_operand_row<KZM>(za, cz, lane, T());
    // this item's output (and raw z) over its real pairs only: the chunks of padded pairs
    // fall outside the range check, so every step issues exactly one store
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(out + pair0 * cz, (size_t)live * cz * sizeof(T));
    const __amdgpu_buffer_rsrc_t rzr = buffer_rsrc(z + pair0 * cz, (size_t)live * cz * sizeof(T));

    // weight step k of the item; the buffers take the steps of all items in turn
#pragma unroll 1
    for (int k = 0; k < STEPS; ++k, buf = buf == K3S_BUFS - 1 ? 0 : buf + 1) {
      // this lane's output chunk of the step (the whole offset per lane: a store's data
      // registers are guarded against the next write only without a scalar offset)
      const unsigned int voff = k < klim ? ooff + 64u * (unsigned int)k : OUT_OF_RANGE;
      // with the residual: the raw z chunk this lane's output of the step is added to (out
      // may be z: it is read before the store below, by the same lane), issued before the
      // wait so that it overlaps the barrier
      chunk_t zres = {0u, 0u, 0u, 0u};
      if constexpr (RESID) zres = load16(rzr, voff, 0);
      asm volatile("" ::: "memory");
      // This step's weights are in LDS once this thread's loads of them are done and every
      // wave is past the barrier; every wave is then also done reading the previous step's
      // buffer, which the loads issued below refill. Vector memory operations complete in
      // issue order, and since the loads of this step (issued two steps back) every wave
      // has issued the BPW loads of the next step, the stores of the two steps between,
      // with the residual two z reads, and in the first two steps of an item the next
      // item's loads: that many may still be outstanding.
      if (k < 2) __builtin_amdgcn_s_waitcnt(K3S_WAIT_FIRST);
      else __builtin_amdgcn_s_waitcnt(K3S_WAIT);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(k + 2 < STEPS ? k + 2 : k + 2 - STEPS, buf == 0 ? K3S_BUFS - 1 : buf - 1);
      const bool last = k == STEPS - 1;
      const unsigned char* const gbuf = wbuf + buf * GB;
      const float* const tk = tos + 32 * k + 4 * q;
      f32x4 ap0 = ld16f(tk), ap1 = ld16f(tk + 16);
      f32x4 ag0 = ld16f(tk + CZP), ag1 = ld16f(tk + CZP + 16);
      // the gate first, chunk by chunk for both units, so that on the item's last step each
      // z chunk is free for the next item's load right after its second product; the
      // weight operands come through a ring of D registers, read D products ahead
      constexpr int NG = 2 * KZM, NM = NG + 2 * KXM, D = 4;
      auto wsrc = [&](int t) -> const unsigned char* {
        if (t < NG) {
          const int ks = t >> 1;
          return gbuf + lg[ks & 3] + 256 * (ks >> 2) + (t & 1) * (16 * CZP * 2);
        }
        const int ks = (t - NG) >> 1;
        return gbuf + lo[ks & 3] + 256 * (ks >> 2) + (t & 1) * (16 * CP * 2);
      };
      chunk_t ring[D];
#pragma unroll
      for (int t = 0; t < D; ++t) ring[t] = ld16(wsrc(t));
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const chunk_t wa = ring[t % D];
        if (t + D < NM) ring[t % D] = ld16(wsrc(t + D));
        if (t < NG) {
          if (t & 1) ag1 = mma16(ag1, wa, za[t >> 1], T());
          else ag0 = mma16(ag0, wa, za[t >> 1], T());
        } else {
          if (t & 1) ap1 = mma16(ap1, wa, bx[(t - NG) >> 1], T());
          else ap0 = mma16(ap0, wa, bx[(t - NG) >> 1], T());
        }
        if (!PF_Z && t == NG - 1 && last) fetch_z(next, za);  // za is free: the next z
      }
      float o[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = gate_mul(ap0[r] * mv, ag0[r]);
        o[4 + r] = gate_mul(ap1[r] * mv, ag1[r]);
      }
      chunk_t v = pack(o, T());
      if constexpr (RESID) v = add_chunks(v, zres, T());
      // default cache policy: a pair's 128-byte line is written in two halves one step
      // apart, which L2 joins before it writes the line back (non-temporal stores reached
      // HBM as half lines: 1.2x the output's bytes)
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)voff, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // the stream's one extra step lands before exit
}

// LDS of the streamed form: the weight step buffers, the start values, the x staging tiles
size_t k3_stream_lds(int cp, int czp) {
  return (size_t)K3S_BUFS * 64 * (cp + czp) + (size_t)2 * czp * 4 +
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
