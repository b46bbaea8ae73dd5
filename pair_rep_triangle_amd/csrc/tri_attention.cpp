// Host side of the C ABI declared in include/tri_attention.h: validation, folding of the
// LayerNorm and the softmax scale into the weights, the kernels' LDS images, launch.

#include "tri_attention.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "attention_launch.h"
#include "host_common.h"

struct tri_attn_handle {
  int c_z, heads, d, device, num_cus;
  void* block;  // projection image | output image | one
  const void *proj_image, *out_image, *one;
};

namespace {

using namespace trimul_host;

constexpr double kLog2e = 1.4426950408889634;

// Row `row` of the projection image: dst[k] = scale * W[k] * gamma[k] (k < c_z, bf16),
// start value scale * (W . beta + bias).
void fold_row(const float* W, const float* gamma, const float* beta, double bias, int c_z,
              double scale, unsigned char* dst, float* start) {
  double t = bias;
  for (int k = 0; k < c_z; ++k) {
    const double w = W[k];
    store_elem(dst + (size_t)k * 2, (float)(scale * w * (gamma ? (double)gamma[k] : 1.0)), true);
    if (beta) t += w * (double)beta[k];
  }
  *start = (float)(scale * t);
}

}  // namespace

extern "C" {

int tri_attn_create(const tri_attn_weights* w, int c_z, int heads, int head_dim, int dtype,
                    tri_attn_handle** out) {
  if (!out) return TRI_MUL_ERR_INVALID_ARG;
  *out = nullptr;
  if (!w || !w->w_q || !w->w_k || !w->w_v || !w->w_b || !w->w_g || !w->w_o)
    return TRI_MUL_ERR_INVALID_ARG;
  if (c_z < 1 || heads < 1 || head_dim < 1) return TRI_MUL_ERR_INVALID_ARG;
  if (dtype != TRI_MUL_BF16) return TRI_MUL_ERR_UNSUPPORTED;
  if (!trimul::attention_supported(c_z, heads, head_dim)) return TRI_MUL_ERR_UNSUPPORTED;
  // the host image first (no device needed), then the device
  const int hd = heads * head_dim;
  const size_t rs = (size_t)c_z + 8, ors = (size_t)hd + 8;  // row strides (bf16 elements)
  const trimul::AttnParts parts = trimul::att_proj_parts(c_z, heads);
  const size_t pimg = trimul::att_proj_image_bytes(c_z, heads);
  const size_t oimg = trimul::att_out_image_bytes(c_z, heads);
  const size_t total = align256(pimg) + align256(oimg) + 256;
  std::vector<unsigned char> host(total, 0);
  unsigned char* hp = host.data();
  // projection row o and its start value, in the image of the part that holds it: the
  // part's rows, then its start values
  auto prow = [&](int o) {
    size_t base = 0;
    int i = 0;
    while (o >= parts.bounds[i + 1]) {
      base += trimul::att_part_bytes(c_z, parts.bounds[i + 1] - parts.bounds[i]);
      ++i;
    }
    return hp + base + (size_t)(o - parts.bounds[i]) * rs * 2;
  };
  auto pstart = [&](int o) {
    size_t base = 0;
    int i = 0;
    while (o >= parts.bounds[i + 1]) {
      base += trimul::att_part_bytes(c_z, parts.bounds[i + 1] - parts.bounds[i]);
      ++i;
    }
    const size_t prows = (size_t)(parts.bounds[i + 1] - parts.bounds[i]);
    return (float*)(hp + base + prows * rs * 2) + (o - parts.bounds[i]);
  };
  unsigned char* ho = hp + align256(pimg);
  float* hob = (float*)(ho + (size_t)c_z * ors * 2);  // b_o
  unsigned char* hone = ho + align256(oimg);
  store_elem(hone, 1.0f, true);

  // projection rows: q (scaled by log2(e) / sqrt(d): the softmax runs in base 2), k,
  // gate (scaled by -log2(e): sigmoid = 1 / (1 + 2^t)), v, then the per-head bias rows
  // (scaled by log2(e)); bias rows past `heads` stay zero
  const double qs = kLog2e / sqrt((double)head_dim);
  for (int o = 0; o < hd; ++o) {
    // q, k and gate rows per head in the projection kernel's order: image row 16 hf + i
    // of a head (half hf, MFMA row i = 4q + rr) is channel 8q + 4 hf + rr of the head
    const int i = o % 16, hf = (o / 16) % 2;
    const int src = o / head_dim * head_dim + 8 * (i >> 2) + 4 * hf + (i & 3);
    const size_t W = (size_t)src * c_z;
    fold_row(w->w_q + W, w->ln_gamma, w->ln_beta, 0.0, c_z, qs, prow(o), pstart(o));
    fold_row(w->w_k + W, w->ln_gamma, w->ln_beta, 0.0, c_z, 1.0, prow(hd + o), pstart(hd + o));
    fold_row(w->w_g + W, w->ln_gamma, w->ln_beta, w->b_g ? (double)w->b_g[src] : 0.0, c_z,
             -kLog2e, prow(2 * hd + o), pstart(2 * hd + o));
    // v rows in channel order (the v^T unit stores one channel per lane)
    fold_row(w->w_v + (size_t)o * c_z, w->ln_gamma, w->ln_beta, 0.0, c_z, 1.0, prow(3 * hd + o),
             pstart(3 * hd + o));
  }
  for (int h = 0; h < heads; ++h)
    fold_row(w->w_b + (size_t)h * c_z, w->ln_gamma, w->ln_beta, 0.0, c_z, kLog2e,
             prow(4 * hd + h), pstart(4 * hd + h));
  // output image: W_o [c_z][hd] rows and b_o, permuted per group of 32 output channels
  // as the attention kernel's output projection reads them: image row 16 hf + i of a
  // group (half hf, MFMA row i = 4q + rr) is channel 8q + 4 hf + rr of the group
  for (int c = 0; c < c_z; ++c) {
    const int i = c % 16, hf = (c / 16) % 2;
    const int src = c / 32 * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
    for (int k = 0; k < hd; ++k)
      store_elem(ho + ((size_t)c * ors + k) * 2, w->w_o[(size_t)src * hd + k], true);
    hob[c] = w->b_o ? w->b_o[src] : 0.f;
  }

  int dev = -1, cus = 0;
  const int rc = check_device(&dev, &cus);
  if (rc != TRI_MUL_OK) return rc;
  tri_attn_handle* h = new (std::nothrow) tri_attn_handle();
  if (!h) return TRI_MUL_ERR_OUT_OF_MEMORY;
  void* dptr = nullptr;
  hipError_t e = hipMalloc(&dptr, total);
  if (e != hipSuccess) {
    delete h;
    if (e == hipErrorOutOfMemory) return TRI_MUL_ERR_OUT_OF_MEMORY;
    return hip_fail(e, "hipMalloc(attention weights)");
  }
  e = hipMemcpy(dptr, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dptr);
    delete h;
    return hip_fail(e, "hipMemcpy(attention weights)");
  }
  unsigned char* d = (unsigned char*)dptr;
  h->c_z = c_z;
  h->heads = heads;
  h->d = head_dim;
  h->device = dev;
  h->num_cus = cus;
  h->block = dptr;
  h->proj_image = d;
  h->out_image = d + align256(pimg);
  h->one = d + align256(pimg) + align256(oimg);
  *out = h;
  return TRI_MUL_OK;
}

int tri_attn_workspace_bytes(const tri_attn_handle* h, int batch, int n, size_t* bytes) {
  if (!h || !bytes || batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N)
    return TRI_MUL_ERR_INVALID_ARG;
  *bytes = trimul::att_workspace(batch, n, h->heads).total;
  return TRI_MUL_OK;
}

}  // extern "C"

namespace {

int attn_forward(tri_attn_handle* h, int stages, const void* z, const void* pair_mask,
                 void* out, int batch, int n, int node, void* workspace, size_t ws_bytes,
                 void* stream) {
  if (!h || !z || !out || !workspace) return TRI_MUL_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N) return TRI_MUL_ERR_INVALID_ARG;
  if (node != TRI_ATTN_STARTING && node != TRI_ATTN_ENDING) return TRI_MUL_ERR_INVALID_ARG;
  if (((uintptr_t)z | (uintptr_t)out | (uintptr_t)workspace) & 15u) return TRI_MUL_ERR_ALIGNMENT;
  if (pair_mask && ((uintptr_t)pair_mask & 1u)) return TRI_MUL_ERR_ALIGNMENT;
  const size_t pairs = (size_t)batch * n * n;
  const size_t zb = pairs * h->c_z * 2, mb = pairs * 2;
  const size_t need = trimul::att_workspace(batch, n, h->heads).total;
  if (ws_bytes < need) return TRI_MUL_ERR_WORKSPACE_TOO_SMALL;
  if (overlaps(out, zb, z, zb) || overlaps(out, zb, pair_mask, mb) ||
      overlaps(out, zb, workspace, need) || overlaps(workspace, need, z, zb) ||
      overlaps(workspace, need, pair_mask, mb))
    return TRI_MUL_ERR_ALIAS;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  trimul::AttnArgs a;
  a.z = z;
  a.mask = pair_mask ? pair_mask : h->one;
  a.out = out;
  a.ws = workspace;
  a.proj_image = h->proj_image;
  a.out_image = h->out_image;
  a.batch = batch;
  a.n = n;
  a.cz = h->c_z;
  a.heads = h->heads;
  a.node = node;
  a.mask_all = pair_mask ? 0 : 1;
  a.num_cus = h->num_cus;
  e = trimul::launch_attention(a, stages, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launch triangular attention");
  return TRI_MUL_OK;
}

}  // namespace

extern "C" {

int tri_attn_forward(tri_attn_handle* h, const void* z, const void* pair_mask, void* out,
                     int batch, int n, int node, void* workspace, size_t ws_bytes,
                     void* stream) {
  return attn_forward(h, 3, z, pair_mask, out, batch, n, node, workspace, ws_bytes, stream);
}

int tri_attn_forward_stage(tri_attn_handle* h, int stage, const void* z, const void* pair_mask,
                           void* out, int batch, int n, int node, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (stage != 1 && stage != 2) return TRI_MUL_ERR_INVALID_ARG;
  return attn_forward(h, stage, z, pair_mask, out, batch, n, node, workspace, ws_bytes, stream);
}

void tri_attn_destroy(tri_attn_handle* h) {
  if (!h) return;
  if (h->block) (void)hipFree(h->block);
  delete h;
}

}  // extern "C"
