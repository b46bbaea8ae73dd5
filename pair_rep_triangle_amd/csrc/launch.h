// Internal interface between the C-ABI host code and the device code.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#define TRI_MUL_LN_EPS_F 1e-5f

namespace trimul {

// Everything one stage launch needs. Pointers are device memory; the element
// type (bf16 or fp32) is chosen by launch_stage's `bf16_storage`.
struct StageArgs {
  const void* z;     // [batch][n][n][cz]
  const void* mask;  // [batch][n][n] or nullptr (all ones)
  void* out;         // [batch][n][n][cz]
  void* a;           // [batch][c][np][np]
  void* b;           // [batch][c][np][np]
  void* x;           // [batch][c][np][np]
  const void* w1;    // [4][c][czp]  a_gate, a_proj, b_gate, b_proj with gamma_in folded
  const float* s1;   // [4][c]       row sums of the stored w1
  const float* t1;   // [4][c]       W beta_in + bias
  const void* wo;    // [cz][cp]     output projection with gamma_out folded
  const float* so;   // [cz]
  const float* to;   // [cz]
  const void* wg;    // [cz][czp]    output gate with gamma_in folded
  const float* sg;   // [cz]
  const float* tg;   // [cz]
  int batch, n, np, cz, czp, c, cp, incoming;
};

// Padded widths: the k extent of every MFMA chunk group (32 for bf16, 16 for fp32).
inline int k_group(bool bf16_storage) { return bf16_storage ? 32 : 16; }
inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
constexpr int N_PAD = 128;  // a, b, x side padding (the contraction tile)

hipError_t launch_stage(int stage, bool bf16_storage, const StageArgs& a, hipStream_t st);
size_t stage_lds_bytes(int stage, bool bf16_storage, int czp, int cp);

}  // namespace trimul
