// Launch interface of the triangular-attention kernels (host code in tri_attention.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace trimul {

constexpr int ATT_D = 32;      // head width the kernels are compiled for
constexpr int ATT_PAD = 64;    // the stored pair grid is padded to a multiple of this

// Storage of the projections ("stored coordinates" (r, c): (i, j) around the starting
// node, (j, i) around the ending node, so both nodes attend along stored rows):
//   q, k, g  [B][Np][H][Np][d]   bf16   (g already through the sigmoid)
//   vt       [B][Np][H][d][Np]   bf16   (v transposed: keys contiguous)
//   bias     [B][H][Np][Np]      bf16   (the pair bias of stored pair (r, c), base 2)
//   (the vt planes [d][Np] and the bias planes [Np][Np] in tiles of 16 rows x 32 columns,
//   row-major inside the tile, tiles row-major: one 1 KB run per tile)
//   ms       [B][Np][Np / 32]    u32    (key-valid bits of the stored row: bit k of word w is
//                                        stored column 32 w + k; 0 on padding)
struct AttnWorkspace {
  size_t q, k, g, vt, bias, ms, total;
};
inline size_t att_align(size_t v) { return (v + 255) / 256 * 256; }
inline int att_np(int n) { return (n + ATT_PAD - 1) / ATT_PAD * ATT_PAD; }
inline AttnWorkspace att_workspace(int batch, int n, int heads) {
  const size_t np = (size_t)att_np(n);
  const size_t plane = (size_t)batch * np * np;
  AttnWorkspace w;
  const size_t qkv = att_align(plane * heads * ATT_D * 2);
  w.q = 0;
  w.k = w.q + qkv;
  w.g = w.k + qkv;
  w.vt = w.g + qkv;
  w.bias = w.vt + qkv;
  w.ms = w.bias + att_align(plane * heads * 2);
  w.total = w.ms + att_align(plane / 8);
  return w;
}

// Projection weights as the projection kernel's LDS images: rows [q | k | g | v] (H*d each)
// then 16 bias rows (H used), each c_z + 8 bf16 (one 16-byte chunk of padding), and the
// fp32 start value of every row (W beta, plus b_g for the gate rows). The rows are cut
// into parts that each fit one workgroup's LDS (one part up to c_z = 128 at 4 heads); a
// part is a contiguous row range [lo, hi) of whole heads of q, k and g (32 rows) and whole
// 16-row units of v and the bias, stored as its rows then its start values, and the
// projection kernel runs once per part (each run reads z again).
inline int att_proj_rows(int heads) { return 4 * heads * ATT_D + 16; }
constexpr size_t ATT_LDS_MAX = 160 * 1024;
inline size_t att_part_bytes(int cz, int rows) {
  return ((size_t)rows * (cz + 8) * 2 + (size_t)rows * 4 + 15) / 16 * 16;
}
// The parts' row boundaries, lo of part i at bounds[i] (bounds[count] = all rows); count 0
// when a single block does not fit.
struct AttnParts {
  int count;
  int bounds[64];
};
inline AttnParts att_proj_parts(int cz, int heads) {
  AttnParts pt{};
  const int hd = heads * ATT_D, rows = att_proj_rows(heads);
  int lo = 0, at = 0;
  pt.bounds[0] = 0;
  while (at < rows) {
    const int block = at < 3 * hd ? 32 : 16;  // a q, k or gate head; a v unit or the bias
    if (att_part_bytes(cz, at + block - lo) > ATT_LDS_MAX) {
      if (at == lo || pt.count + 1 >= 63) return AttnParts{};
      pt.bounds[++pt.count] = at;
      lo = at;
      continue;
    }
    at += block;
  }
  pt.bounds[++pt.count] = rows;
  return pt;
}
inline size_t att_proj_image_bytes(int cz, int heads) {
  const AttnParts pt = att_proj_parts(cz, heads);
  size_t total = 0;
  for (int i = 0; i < pt.count; ++i) total += att_part_bytes(cz, pt.bounds[i + 1] - pt.bounds[i]);
  return total;
}
// Output weights as the attention kernel's image: W_o [c_z][H*d + 8] bf16, then b_o
// [c_z] fp32. The kernel holds at most ATT_WO_ROWS rows of it (and their b_o) in LDS at a
// time (all of it up to c_z = 128, copied once), followed by its staging rows
// [64][H*d + 8] bf16.
constexpr int ATT_WO_ROWS = 128;
inline size_t att_out_image_bytes(int cz, int heads) {
  return (size_t)cz * (heads * ATT_D + 8) * 2 + (size_t)cz * 4;
}
inline size_t att_core_lds_bytes(int cz, int heads) {
  const size_t rows = cz < ATT_WO_ROWS ? (size_t)cz : (size_t)ATT_WO_ROWS;
  return rows * (heads * ATT_D + 8) * 2 + rows * 4 + (size_t)64 * (heads * ATT_D + 8) * 2;
}

struct AttnArgs {
  const void* z;      // [B][N][N][c_z] bf16
  const void* mask;   // [B][N][N] bf16, or the one-element `one` when there is no mask
  void* out;          // [B][N][N][c_z] bf16
  void* ws;           // workspace base (att_workspace layout)
  const void* proj_image;
  const void* out_image;
  int batch, n, cz, heads, node, mask_all, num_cus;
};

inline bool attention_supported(int cz, int heads, int d) {
  if (d != ATT_D || heads < 1 || heads > 8) return false;
  if (cz % 32 || cz < 32 || cz > 384) return false;
  return att_proj_parts(cz, heads).count > 0 && att_core_lds_bytes(cz, heads) <= ATT_LDS_MAX;
}

// stages: 1 = projection, 2 = attention and output, 3 = both
hipError_t launch_attention(const AttnArgs& a, int stages, hipStream_t st);

}  // namespace trimul
