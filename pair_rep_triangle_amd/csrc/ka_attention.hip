// Triangular attention (starting and ending node), two kernels:
//   ka_project: LayerNorm of z and every projection (q, k, gate, v, per-head pair bias)
//               with MFMAs, written in stored coordinates;
//   ka_core:    per stored row, flash attention for every head over 32-key tiles, the
//               gate, and the output projection, written to out.
// Definition and sources: include/tri_attention.h (yage.ai summary of the
// biomolecular-software report: triangular attention as a pair operation of cubic cost
// with a fused kernel; OpenFold-TRT summary: triangular attention among the pair
// kernels). Stored coordinates (r, c) are (i, j) around the starting node and (j, i)
// around the ending node: both nodes then attend along a stored row, keys indexed by the
// stored column, and the pair bias of query column qc and key column kc is the bias of
// stored pair (qc, kc).

#include <type_traits>

#include "attention_launch.h"
#include "device_common.h"

namespace trimul {

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int KA_WAVES = 8;                  // projection kernel
constexpr int KA_THREADS = 64 * KA_WAVES;
constexpr int KA_TW = 32;                    // pairs per projection wave tile
constexpr int KC_WAVES = 4;                  // attention kernel
constexpr int KC_THREADS = 64 * KC_WAVES;
constexpr int KC_QB = 4;                     // 16-query blocks per attention tile
constexpr int KC_KB = 2;                     // 16-key blocks per attention step (2 or 4)
constexpr int KC_MIN_SPLIT = 4;              // workgroups per stored row, at least

// The bias planes and the v^T planes are stored in tiles of 16 rows x 32 columns (1 KB in
// bf16, row-major inside the tile): element (row, col) of a plane with np columns sits at
// tile_off(row, col, np). A wave's 16 rows x 32 keys of a key step are then one 1 KB run.
__device__ __forceinline__ size_t tile_off(int row, int col, int np) {
  return ((size_t)(row >> 4) * (np >> 5) + (col >> 5)) * 512 + (row & 15) * 32 + (col & 31);
}

// ---------------------------------------------------------------------------------------
// ka_project. A wave tile is 32 consecutive stored columns (two 16-pair subtiles) of one
// stored row; row p of subtile st is the tile's pair 8 (p / 4) + 4 st + p % 4. z arrives
// in MFMA operand layout (lane (p, q): chunk ks*4 + q of that pair), is normalised in
// registers and is the B operand of the q, k and gate heads (W rows as A, stored
// permuted per head: lane (p, q) ends with channels 8q..8q+7 of its pair) and the A
// operand of the v and bias units (W rows as B: lane (p, q) ends with stored columns
// 8q..8q+7 of output p). Every result leaves as one 16-byte store per lane.
// The weights (LDS image, rows padded by 16 bytes) are loaded once per workgroup.
template <int KZ>
__global__ __launch_bounds__(KA_THREADS) void ka_project(
    const bf16* __restrict__ z, const bf16* __restrict__ mask, const chunk_t* __restrict__ image,
    int image_chunks, bf16* __restrict__ qo, bf16* __restrict__ ko, bf16* __restrict__ go,
    bf16* __restrict__ vto, bf16* __restrict__ bo, unsigned int* __restrict__ mwo, int batch, int n,
    int np, int heads, int ending, int mask_all) {
  constexpr int E = 8, KG = 32, CZ = KZ * KG, RS = CZ + 8;  // LDS row stride (elements)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int hd = heads * ATT_D;
  const int rows = 4 * hd + 16;
  const bf16* const wl = (const bf16*)smem;
  const float* const tl = (const float*)(smem + (size_t)rows * RS * 2);  // start values

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;
  const int ctiles = np / KA_TW;
  const int tiles = batch * np * ctiles;
  const int gw = blockIdx.x * KA_WAVES + wave, nw = gridDim.x * KA_WAVES;
  // stored (r, c) -> z pair (x, y); consecutive stored columns are 1 (starting) or n
  // (ending) z pairs apart
  const size_t pstride = ending ? (size_t)n : 1;

  struct Pre {
    chunk_t zv[2][KZ];
    bf16 m[2];
  };
  auto coords = [&](int t, int& b, int& r, int& c0) {
    b = t / (np * ctiles);
    const int rem = t - b * np * ctiles;
    r = rem / ctiles;
    c0 = (rem - r * ctiles) * KA_TW;
  };
  // Row p of subtile st is the tile's pair pp(st) = 8 (p / 4) + 4 st + p % 4, so that the
  // v^T and bias units end with eight consecutive pairs per lane. Pairs outside n x n read
  // as zero (the resource extent ends at the last real pair of the tile's run; rows past
  // n get an empty extent).
  auto pair_of = [&](int st) { return 8 * (p >> 2) + 4 * st + (p & 3); };
  auto fetch = [&](int t, Pre& f) {
    int b, r, c0;
    coords(t < tiles ? t : tiles - 1, b, r, c0);
    const bool ok = r < n && c0 < n;
    const size_t x = ending ? (size_t)c0 : (size_t)r, y = ending ? (size_t)r : (size_t)c0;
    const size_t p0 = ok ? ((size_t)b * n + x) * n + y : 0;
    // pairs from the tile's first to the last real one of its run
    const size_t span = ok ? (size_t)(n - 1 - c0) * pstride + 1 : 0;
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(z + p0 * CZ, span * CZ * 2);
    const __amdgpu_buffer_rsrc_t rm =
        mask_all ? buffer_rsrc(mask, 2) : buffer_rsrc(mask + p0, span * 2);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const unsigned int zoff = (unsigned int)(((size_t)pair_of(st) * pstride * CZ + q * E) * 2);
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) f.zv[st][ks] = load16(rz, zoff + ks * KG * 2, 0);
      f.m[st] = load_elem(rm, mask_all ? 0u : (unsigned int)(pair_of(st) * pstride * 2), 0,
                          bf16());
    }
  };

  Pre f;
  copy_image<KA_THREADS>(image, (chunk_t*)smem, image_chunks, tid, [&]() { fetch(gw, f); });
  __syncthreads();

  for (int t = gw; t < tiles; t += nw) {
    int b, r, c0;
    coords(t, b, r, c0);
    chunk_t za[2][KZ];
    float mv[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      mv[st] = (r < n && c0 + pair_of(st) < n) ? to_f32(f.m[st]) : 0.f;
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) za[st][ks] = f.zv[st][ks];
      normalize_operand_row<KZ>(za[st], CZ, lane, bf16());
    }
    fetch(t + nw, f);  // the next tile's loads have this tile's MFMAs to land

    const size_t rowbase = ((size_t)b * np + r) * heads;  // [b][r][h] of q, k, g, v^T
    int opaque;  // keeps the loop-invariant LDS reads inside the tile loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque));

    // q, k and gate: one head (two 16-row halves, W rows as A) at a time. The handle
    // stores a head's 32 rows permuted: row 4q + rr of half hf is channel 8q + 4 hf + rr,
    // so after both halves lane (p, q) holds channels 8q .. 8q + 7 of the head for pair
    // c0 + 16 st + p, and one 16-byte store per lane writes the pair's whole 64-byte row.
    auto head_a = [&](int row0, int which, bf16* dst) {
      const int h = (row0 - which * hd) / ATT_D;
      f32x4 acc[2][2];  // [half][st]
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16* const wrow = wl + (row0 + 16 * hf + p) * RS + q * E + opaque;
        chunk_t wa[KZ];
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) wa[ks] = ld16(wrow + ks * KG);
        const f32x4 t0 = ld16f(tl + row0 + 16 * hf + 4 * q + opaque);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          acc[hf][st] = t0;
#pragma unroll
          for (int ks = 0; ks < KZ; ++ks) acc[hf][st] = mma16(acc[hf][st], wa[ks], za[st][ks], bf16());
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = acc[e >> 2][st][e & 3];
          // gate: rows scaled by -log2(e), sigmoid = 1 / (1 + 2^acc)
          if (which == 2) v[e] = __builtin_amdgcn_rcpf(1.f + exp2f(v[e]));
        }
        const int c = c0 + pair_of(st);
        st16(dst + ((rowbase + h) * np + c) * ATT_D + 8 * q, pack(v, bf16()));
      }
    };
    // v and bias units: W rows as B. Lane (p, q): pairs c0 + 8q + 4 st .. +3 (rows 4q .. 4q
    // + 3 of subtile st), output 16u' + p of the block; the two subtiles leave as one
    // 16-byte store of pairs c0 + 8q .. c0 + 8q + 7.
    auto unit_b = [&](int row0, bool bias) {
      const bf16* const wrow = wl + (row0 + p) * RS + q * E + opaque;
      chunk_t wb[KZ];
#pragma unroll
      for (int ks = 0; ks < KZ; ++ks) wb[ks] = ld16(wrow + ks * KG);
      const float t0 = tl[row0 + p + opaque];
      const int o = bias ? p : row0 - 3 * hd + p;
      const int h = o / ATT_D, dd = o - h * ATT_D;
      float v[8];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 acc = {t0, t0, t0, t0};
#pragma unroll
        for (int ks = 0; ks < KZ; ++ks) acc = mma16(acc, za[st][ks], wb[ks], bf16());
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * st + e] = acc[e];
      }
      const int c = c0 + 8 * q;
      if (bias) {
        if (p < heads)
          st16(bo + ((size_t)b * heads + p) * np * np + tile_off(r, c, np), pack(v, bf16()));
      } else {
        st16(vto + (rowbase + h) * ATT_D * np + tile_off(dd, c, np), pack(v, bf16()));
      }
    };
#pragma unroll 1
    for (int hh = 0; hh < heads; ++hh) head_a(ATT_D * hh, 0, qo);
#pragma unroll 1
    for (int hh = 0; hh < heads; ++hh) head_a(hd + ATT_D * hh, 1, ko);
#pragma unroll 1
    for (int hh = 0; hh < heads; ++hh) head_a(2 * hd + ATT_D * hh, 2, go);
#pragma unroll 1
    for (int u = 0; u < hd / 16; ++u) unit_b(3 * hd + 16 * u, false);
    unit_b(4 * hd, true);
    // key-valid bits in stored coordinates (0 on padding): bit k of word c0 / 32 of
    // stored row r is column c0 + k (nonzero mask value); lanes q = 0 hold the tile's
    // 32 values
    // (lane p of subtile st holds pair 8 (p / 4) + 4 st + p % 4: nibble g of a ballot
    // goes to bits 8g + 4 st)
    const unsigned long long v0 = __ballot(q == 0 && mv[0] != 0.f);
    const unsigned long long v1 = __ballot(q == 0 && mv[1] != 0.f);
    unsigned int word = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      word |= (unsigned int)((v0 >> (4 * g)) & 0xfu) << (8 * g) |
              (unsigned int)((v1 >> (4 * g)) & 0xfu) << (8 * g + 4);
    if (lane == 0) mwo[((size_t)b * np + r) * (np / 32) + c0 / 32] = word;
  }
}

// ---------------------------------------------------------------------------------------
// ka_core. Stored row r is shared by `split` workgroups (query tiles share, share +
// split, ...); the four waves of a workgroup take the heads (wave w: heads
// w, w + 4). Per tile of 16 QB query columns and head, a wave runs the keys in steps of
// 16 KB, with the step's keys permuted so that lane q owns 4 KB consecutive ones:
//   S^T = K Q^T (key rows, query columns) with the pair bias as the accumulator start:
//     lane (p, q) of block kb holds keys 4 KB q + 4 kb + e (e < 4) of query 16 qb + p
//     (the K operand's row p is key 4 KB (p / 4) + 4 kb + p % 4);
//   online softmax per query in base 2 (log2(e) / sqrt(d) is folded into W_q and
//     log2(e) into the bias rows), masked keys left out; the four lanes p, p^16, p^32,
//     p^48 hold all keys of a query, so the running maximum is reduced across them and
//     the sum is kept per lane until the end;
//   O^T += V^T P^T: each run of eight of the lane's probabilities of a query ARE its
//     B-operand chunk once V^T's A chunk holds the same eight keys, one 16-byte run of
//     the transposed v.
// Then o = O^T / l * gate goes to LDS as [query][h*d + channel]; after a barrier the
// waves split the output channels: out^T = W_o o^T + b_o with W_o rows from LDS as A.
template <int KZ, int QB, int KB>
__global__ __launch_bounds__(KC_THREADS) void ka_core(
    const bf16* __restrict__ qi, const bf16* __restrict__ ki, const bf16* __restrict__ gi,
    const bf16* __restrict__ vti, const bf16* __restrict__ bi, const unsigned int* __restrict__ mwi,
    const chunk_t* __restrict__ image, int image_chunks, bf16* __restrict__ out, int n, int np,
    int heads, int ending, int rows, int split) {
  constexpr int CZ = KZ * 32;
  constexpr int QT = 16 * QB;  // queries per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int hd = heads * ATT_D, os_stride = hd + 8;
  const bf16* const wo = (const bf16*)smem;                                 // [CZ][hd + 8]
  const float* const bo = (const float*)(smem + (size_t)CZ * os_stride * 2);  // [CZ]
  bf16* const os = (bf16*)(smem + (size_t)CZ * os_stride * 2 + CZ * 4);       // [64][hd + 8]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 15, q = lane >> 4;
  // XCD-aware order: workgroup ids are dealt to the eight XCDs in turn. The `split`
  // workgroups of stored row `row` get ids equal mod 8 and within 8 * split of each other,
  // so they run together on one XCD and read the row's K and V^T through its L2 once.
  const int grp = blockIdx.x / (8 * split), w8 = blockIdx.x - grp * 8 * split;
  const int share = w8 >> 3, row = grp * 8 + (w8 & 7);
  if (row >= rows) return;  // the last group of eight may be partial (whole workgroup)
  const int b = row / n, r = row - b * n;
  copy_image<KC_THREADS>(image, (chunk_t*)smem, image_chunks, tid, []() {});
  __syncthreads();

  constexpr int KT = 16 * KB;  // keys per step
  const int ksteps = (n + KT - 1) / KT;  // key steps past n would be all masked
  const unsigned int* const mwrow = mwi + ((size_t)b * np + r) * (np / 32);
  // a row without any valid key (a padded residue) adds nothing: its queries get a zero
  // attention output without running the key steps
  unsigned int anyv = 0;
  for (int t = lane; t < np / 32; t += 64) anyv |= mwrow[t];
  const int kend = __any(anyv != 0u) ? ksteps : 0;
  const float NEG = -__builtin_huge_valf();

  for (int qt = share; qt < np / QT; qt += split) {
    const int qc0 = qt * QT;
    for (int h = wave; h < heads; h += KC_WAVES) {
      const size_t rh = ((size_t)b * np + r) * heads + h;
      const bf16* const qrow = qi + rh * np * ATT_D;
      const bf16* const krow = ki + rh * np * ATT_D;
      const bf16* const vrow = vti + rh * ATT_D * np;
      const bf16* const brow = bi + ((size_t)b * heads + h) * np * np;
      chunk_t qf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qf[qb] = ld16(qrow + (size_t)(qc0 + 16 * qb + p) * ATT_D + 8 * q);
      f32x4 o[2][QB];
      float mrun[QB], lsum[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mrun[qb] = NEG;
        lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < 2; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // One key step's operands (KB blocks of 16 keys): K chunks, the bias tiles (the
      // accumulator start of S^T), the key-valid bits and V^T chunks. Each is reloaded for
      // the next step right after its last use in this one (bias, K and the bits after the
      // S^T MFMAs, V^T after the O^T MFMAs), so the loads run a step ahead with no copies.
      // Key order: lane q of a step owns the 4 KB consecutive keys 4 KB q .. 4 KB q + 4 KB - 1
      // (row 4q + e of S^T block kb is key 4 KB q + 4 kb + e), so its bias values and its
      // V^T chunks are whole 16-byte runs.
      chunk_t kf[KB], vf[KB / 2][2];
      chunk_t sb[KB / 2][QB];  // eight bf16 bias values per chunk and lane
      unsigned long long mw;  // the step's key-valid bits (bit k: key k0 + k), wave-uniform
      auto load_kbm = [&](int ks) {
        const int k0 = (ks < ksteps ? ks : ksteps - 1) * KT;
        if constexpr (KB == 2) {
          mw = __builtin_amdgcn_readfirstlane(mwrow[k0 / 32]);
        } else {
          const u32x2 w2 = *(const u32x2*)(mwrow + k0 / 32);
          mw = (unsigned long long)__builtin_amdgcn_readfirstlane(w2[0]) |
               ((unsigned long long)__builtin_amdgcn_readfirstlane(w2[1]) << 32);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          // A row p of block kb: key 4 KB (p / 4) + 4 kb + p % 4
          kf[kb] = ld16(krow + (size_t)(k0 + 4 * KB * (p >> 2) + 4 * kb + (p & 3)) * ATT_D + 8 * q);
        }
#pragma unroll
        for (int j = 0; j < KB / 2; ++j)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sb[j][qb] = ld16(brow + tile_off(qc0 + 16 * qb + p, k0 + 4 * KB * q + 8 * j, np));
      };
      // V^T row p of block db is channel 8 (p / 4) + 4 db + p % 4, so that O^T lane (p, q)
      // ends with channels 8q .. 8q + 7 of its query across the two blocks (one 16-byte
      // gate load and one 16-byte staging store); half kh of the step: keys 4 KB q + 8 kh
      // .. + 7 (the keys of the lane's probabilities pv[8 kh .. 8 kh + 7])
      auto load_v = [&](int ks) {
        const int k0 = (ks < ksteps ? ks : ksteps - 1) * KT;
#pragma unroll
        for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
          for (int db = 0; db < 2; ++db)
            vf[kh][db] = ld16(vrow + tile_off(8 * (p >> 2) + 4 * db + (p & 3),
                                              k0 + 4 * KB * q + 8 * kh, np));
      };
      load_kbm(0);
      load_v(0);
#pragma unroll 1
      for (int ks = 0; ks < kend; ++ks) {
        const unsigned long long w = mw;
        f32x4 s[KB][QB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const unsigned int b01 = sb[kb >> 1][qb][2 * (kb & 1)];
            const unsigned int b23 = sb[kb >> 1][qb][2 * (kb & 1) + 1];
            const f32x4 b0 = {__uint_as_float(b01 << 16), __uint_as_float(b01 & 0xffff0000u),
                              __uint_as_float(b23 << 16), __uint_as_float(b23 & 0xffff0000u)};
            s[kb][qb] = mma16(b0, kf[kb], qf[qb], bf16());
          }
        bool valid[KB][4];  // keys 4 KB q + 4 kb + e (read on the masked path only)
        const unsigned long long wl = w >> (4 * KB * q);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) valid[kb][e] = (wl >> (4 * kb + e)) & 1u;
        load_kbm(ks + 1);  // the last step reloads itself (unused)
        // The common case (every key of the step valid) runs without selects; the
        // probabilities use the raw base-2 exponential (results below 2^-126 flush to 0).
        chunk_t pb[KB / 2][QB];
        auto softmax_step = [&](auto masked) {
          constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float tmax = (!MASKED || valid[0][0]) ? s[0][qb][0] : NEG;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (kb + e > 0) tmax = fmaxf(tmax, (!MASKED || valid[kb][e]) ? s[kb][qb][e] : NEG);
            tmax = fmaxf(tmax, lane_value(tmax, lane ^ 16));
            tmax = fmaxf(tmax, lane_value(tmax, lane ^ 32));
            const float mnew = fmaxf(mrun[qb], tmax);
            const float msafe = mnew == NEG ? 0.f : mnew;  // no valid key yet: every p is 0
            // the accumulated sums follow the new maximum: 2^(old - new), 1 when it did not
            // grow, 0 before the first valid key (old = -inf); no branch, no copies
            const float scale = __builtin_amdgcn_exp2f(mrun[qb] - msafe);
            lsum[qb] *= scale;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int e = 0; e < 4; ++e) o[db][qb][e] *= scale;
            mrun[qb] = mnew;
            float pv[4 * KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float ex = __builtin_amdgcn_exp2f(s[kb][qb][e] - msafe);
                pv[4 * kb + e] = (!MASKED || valid[kb][e]) ? ex : 0.f;
              }
            float ps = pv[0];
#pragma unroll
            for (int e = 1; e < 4 * KB; ++e) ps += pv[e];
            lsum[qb] += ps;
#pragma unroll
            for (int kh = 0; kh < KB / 2; ++kh) pb[kh][qb] = pack(pv + 8 * kh, bf16());
          }
        };
        if (w == (KB == 2 ? 0xffffffffull : ~0ull))
          softmax_step(std::false_type());
        else
          softmax_step(std::true_type());
#pragma unroll
        for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < 2; ++db)
              o[db][qb] = mma16(o[db][qb], vf[kh][db], pb[kh][qb], bf16());
        load_v(ks + 1);
      }
      // normalise, gate, stage: o^T lane (p, q) reg e of block db = channel 8q + 4 db + e
      // of query 16 qb + p
      const bf16* const grow = gi + rh * np * ATT_D;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float l = lsum[qb];
        l += lane_value(l, lane ^ 16);
        l += lane_value(l, lane ^ 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int qc = qc0 + 16 * qb + p;
        float gv[8], ov[8];
        unpack(ld16(grow + (size_t)qc * ATT_D + 8 * q), gv, bf16());
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = o[e >> 2][qb][e & 3] * inv * gv[e];
        st16(os + (16 * qb + p) * os_stride + h * ATT_D + 8 * q, pack(ov, bf16()));
      }
    }
    __syncthreads();
    // out^T = W_o o^T + b_o per group of 32 output channels, as two 16-row halves. The
    // handle stores W_o's rows (and b_o) permuted per group: row 4q + rr of half hf is
    // channel 8q + 4 hf + rr, so lane (p, q) ends with channels 32g + 8q .. + 7 of query
    // 16 qb + p and writes them as one 16-byte store.
    for (int g = wave; g < CZ / 32; g += KC_WAVES) {
#pragma unroll 1
      for (int qb = 0; qb < QB; ++qb) {  // one query block at a time: few live registers
        f32x4 acc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int u = 2 * g + hf;
          acc[hf] = ld16f(bo + 16 * u + 4 * q);
          for (int kk = 0; kk < hd / 32; ++kk)
            acc[hf] = mma16(acc[hf], ld16(wo + (16 * u + p) * os_stride + 32 * kk + 8 * q),
                            ld16(os + (16 * qb + p) * os_stride + 32 * kk + 8 * q), bf16());
        }
        const int qc = qc0 + 16 * qb + p;
        if (qc < n) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[e >> 2][e & 3];
          const size_t x = ending ? (size_t)qc : (size_t)r, y = ending ? (size_t)r : (size_t)qc;
          // non-temporal: the output is not read again here and would only displace
          // K, V^T and the bias from the caches (ka_core 235 -> 229 us)
          __builtin_nontemporal_store(
              pack(v, bf16()), (chunk_t*)(out + (((size_t)b * n + x) * n + y) * CZ + 32 * g + 8 * q));
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------

template <int KZ>
static hipError_t launch_attention_kz(const AttnArgs& a, int stages, hipStream_t st) {
  const int np = att_np(a.n);
  const AttnWorkspace L = att_workspace(a.batch, a.n, a.heads);
  unsigned char* ws = (unsigned char*)a.ws;
  bf16* q = (bf16*)(ws + L.q);
  bf16* k = (bf16*)(ws + L.k);
  bf16* g = (bf16*)(ws + L.g);
  bf16* vt = (bf16*)(ws + L.vt);
  bf16* bias = (bf16*)(ws + L.bias);
  unsigned int* mw = (unsigned int*)(ws + L.ms);

  // projection: persistent waves over 32-pair tiles of the padded stored grid
  if (stages & 1) {
    const size_t lds = att_proj_image_bytes(a.cz, a.heads);
    if (lds % 16) return hipErrorInvalidValue;
    auto fn = ka_project<KZ>;
    static std::atomic<int> granted{0};
    hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
    if (e != hipSuccess) return e;
    static std::atomic<int> occ{0};
    static std::atomic<size_t> occ_lds{0};
    const int per_cu = resident_blocks((const void*)fn, KA_THREADS, lds, occ, occ_lds);
    const long long tiles = (long long)a.batch * np * (np / KA_TW);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    const long long need = (tiles + KA_WAVES - 1) / KA_WAVES;
    const long long cap = (long long)a.num_cus * per_cu;
    const int blocks = (int)(need < cap ? need : cap);
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(KA_THREADS), lds, st, (const bf16*)a.z,
                       (const bf16*)a.mask, (const chunk_t*)a.proj_image, (int)(lds / 16), q, k,
                       g, vt, bias, mw, a.batch, a.n, np, a.heads, a.node, a.mask_all);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // attention: one workgroup per stored row
  if (stages & 2) {
    const size_t img = att_out_image_bytes(a.cz, a.heads);
    const size_t lds = att_core_lds_bytes(a.cz, a.heads);
    if (img % 16) return hipErrorInvalidValue;
    constexpr int QB = KC_QB;
    static_assert(KC_KB == 2 || KC_KB == 4, "a step is 32 or 64 keys");
    auto fn = ka_core<KZ, QB, KC_KB>;
    static std::atomic<int> granted{0};
    hipError_t e = ensure_dynamic_lds((const void*)fn, granted, lds);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.batch * a.n;
    if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
    // a row's query tiles are shared by `split` workgroups on one XCD: at least
    // KC_MIN_SPLIT (they share the row's K and V^T through L2), enough for four per CU
    const int qtiles = np / (16 * QB);
    const long long rows8 = (rows + 7) / 8 * 8;
    long long split = ((long long)a.num_cus * 4 + rows - 1) / rows;
    if (split < KC_MIN_SPLIT) split = KC_MIN_SPLIT;
    if (split > qtiles) split = qtiles;
    while (split > 1 && rows8 * split > 0x7fffffffLL) --split;
    if (rows8 * split > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned int)(rows8 * split)), dim3(KC_THREADS), lds, st, q, k,
                       g, vt, bias, mw, (const chunk_t*)a.out_image, (int)(img / 16),
                       (bf16*)a.out, a.n, np, a.heads, a.node, (int)rows, (int)split);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, int stages, hipStream_t st) {
  switch (a.cz / 32) {
    case 1: return launch_attention_kz<1>(a, stages, st);
    case 2: return launch_attention_kz<2>(a, stages, st);
    case 3: return launch_attention_kz<3>(a, stages, st);
    case 4: return launch_attention_kz<4>(a, stages, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace trimul
