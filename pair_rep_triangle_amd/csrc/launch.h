// Internal interface between the C-ABI host code and the device code.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

#define TRI_MUL_LN_EPS_F 1e-5f

namespace trimul {

// Which form of the input and output kernels a call takes (filled by a launcher instead of
// launching when StageArgs::plan is set).
struct KernelPlan {
  int k1_form;    // 0 = wave-independent, weights in LDS; 1 = tile-shared, weights in registers
  int k3_form;    // same two forms for the output kernel
  int k3_groups;  // output-channel groups the output kernel splits c_z into (grid y)
};

// Everything one stage launch needs. Pointers are device memory; the element type
// (bf16 or fp32) is chosen by the launcher's `bf16_storage`.
struct StageArgs {
  const void* z;     // [batch][n][n][cz]
  const void* mask;  // [batch][n][n] or nullptr (all ones)
  void* out;         // [batch][n][n][cz]
  void* a;           // [batch][c][np][np]
  void* b;           // [batch][c][np][np]
  void* x;           // [batch][c][np][np]
  const void* w1;    // [4][c][czp]  a_gate, a_proj, b_gate, b_proj: W diag(gamma_in);
                     //              gate rows times -log2(e)
  const float* t1;   // [4][c]       W beta_in + bias (gate rows times -log2(e))
  const void* wo;    // [cz][cp]     W_o diag(gamma_out)
  const float* to;   // [cz]         W_o beta_out + b_o
  const void* wg;    // [cz][czp]    W_g diag(gamma_in) times -log2(e)
  const float* tg;   // [cz]         (W_g beta_in + b_g) times -log2(e)
  const void* one;   // one element of value 1 in the storage type (stands in for no mask)
  const void* k1w_image;  // the wave-independent input gate's weights, one LDS image per
                          // unit group (k1w_layout.h), or nullptr when that form is unused
  int batch, n, np, cz, czp, c, cp, incoming, num_cus;
  int residual;      // stage 3 writes z + update instead of the update (out may be z)
  KernelPlan* plan;  // when set, the k1 / k3 launchers record their choice and launch nothing
  const int* extents;  // [batch][64] partial mask extents (k0) or nullptr: the contraction
                       // then covers the whole padded side
  const void* k3s_image;  // the streamed output gate's weights (k3_stream.hip), or nullptr
};

// k extent of one 16x16 MFMA chunk group: 32 (bf16) or 16 (fp32).
inline int k_group(bool bf16_storage) { return bf16_storage ? 32 : 16; }
inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
// With mask extents and at most this many batch items, the persistent projection kernels
// hand out only the tiles inside each item's extent (every wave reads all items' extents);
// with more items they keep the full tile list and skip the tiles outside.
constexpr int COMPACT_MAX_ITEMS = 32;
constexpr int N_PAD = 64;  // side padding of a, b, x (whole 64-pair input tiles)
constexpr size_t LDS_PER_CU = 160 * 1024;  // gfx950 LDS per CU (the most one workgroup may use)

// The projection kernels keep their weights in registers, sized at compile time by the
// number of chunk groups along k. The output kernel is compiled for these (KX, KZ) pairs
// (KX for c, KZ for c_z); the input kernel for every KZ that appears. A handle pads c and
// c_z with zeros up to the cheapest pair that covers both.
#define TRIMUL_K3_VARIANTS(X) \
  X(1, 1) X(2, 2) X(4, 4) X(8, 8) X(12, 12) X(16, 16) X(4, 12) X(4, 16) X(8, 12) X(8, 16) \
  X(12, 16) X(2, 4) X(4, 8) X(4, 2) X(8, 4)
inline bool padded_ksteps(int c, int cz, bool bf16_storage, int* kx, int* kz) {
  const int kg = k_group(bf16_storage);
  const int kx0 = (c + kg - 1) / kg, kz0 = (cz + kg - 1) / kg;
  int best = -1;
#define TRIMUL_PICK(X_, Z_) \
  if (X_ >= kx0 && Z_ >= kz0 && (best < 0 || X_ + Z_ < best)) { best = X_ + Z_; *kx = X_; *kz = Z_; }
  TRIMUL_K3_VARIANTS(TRIMUL_PICK)
#undef TRIMUL_PICK
  return best > 0;
}

// Raises a kernel's dynamic-LDS limit when a launch needs more than was granted so far.
inline hipError_t ensure_dynamic_lds(const void* fn, std::atomic<int>& granted, size_t need) {
  if ((int)need <= granted.load(std::memory_order_relaxed)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)need);
  if (e == hipSuccess) {
    int cur = granted.load();
    while ((int)need > cur && !granted.compare_exchange_weak(cur, (int)need)) {
    }
  }
  return e;
}

// Resident workgroups per CU for a persistent kernel (queried once per instantiation and
// LDS size; at least 1).
inline int resident_blocks(const void* fn, int threads, size_t lds, std::atomic<int>& cache,
                           std::atomic<size_t>& cache_lds) {
  int v = cache.load(std::memory_order_relaxed);
  if (v > 0 && cache_lds.load(std::memory_order_relaxed) == lds) return v;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds) != hipSuccess || nb < 1)
    nb = 1;
  cache_lds.store(lds);
  cache.store(nb);
  return nb;
}

hipError_t launch_k0(bool bf16_storage, const void* mask, int batch, int n, int* parts,
                     hipStream_t st);
hipError_t launch_k1(bool bf16_storage, const StageArgs& a, hipStream_t st);
hipError_t launch_k2(bool bf16_storage, const StageArgs& a, hipStream_t st);
size_t k2_grid(int np, int batch, int c);  // contraction workgroups per launch
hipError_t launch_k3(bool bf16_storage, const StageArgs& a, hipStream_t st);

// The output gate with its weights streamed through LDS (bf16, c_z above 128), compiled
// for these padded (KX, KZ) chunk-group pairs; its weight image per unit pair k of 32
// output rows: W_o rows [32][cp] then W_g rows [32][czp] (row R of the kernel is channel
// 32 (R / 32) + 8 ((R % 16) / 4) + 4 ((R % 32) / 16) + R % 4; chunk c of row r at position
// c ^ (r & 15)), then the start values of W_o and W_g [czp] each, in kernel row order.
#define TRIMUL_K3S_VARIANTS(X) X(4, 8) X(4, 12) X(4, 16)
size_t k3_stream_lds(int cp, int czp);
inline bool k3_stream_variant(int kx, int kz) {
#define TRIMUL_K3S_IS(X_, Z_) if (kx == X_ && kz == Z_) return true;
  TRIMUL_K3S_VARIANTS(TRIMUL_K3S_IS)
#undef TRIMUL_K3S_IS
  return false;
}
inline int k3_stream_channel(int R) {
  return 32 * (R / 32) + 8 * ((R % 16) / 4) + 4 * ((R % 32) / 16) + R % 4;
}
hipError_t launch_k3_stream(const StageArgs& a, hipStream_t st, bool* done);

}  // namespace trimul
