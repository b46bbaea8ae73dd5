// Host side of the C ABI declared in include/pair_transition.h: validation, LayerNorm
// folding, the kernel's weight order, launch.

#include "pair_transition.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "host_common.h"
#include "transition_launch.h"

struct pair_transition_handle {
  int c_z, hidden, hp, dtype, device, num_cus;
  bool bf16, wide;
  int czp;  // wide form: padded c_z
  void* block;  // LDS image of the weights | one
  const void *image, *one;
  size_t image_bytes;
};

namespace {

using namespace trimul_host;

// Output channel held by accumulator row R of the second GEMM. bf16: row 16v + 4q + r of
// output unit v is element 4 (v % 2) + r of the lane's z chunk v / 2, i.e. channel
// 32 (v / 2) + 8q + 4 (v % 2) + r; fp32: the natural order.
int out_channel(int R, bool bf16) {
  if (!bf16) return R;
  const int v = R / 16, q = (R % 16) / 4, r = R % 4;
  return 32 * (v / 2) + 8 * q + 4 * (v % 2) + r;
}

// Hidden unit in k slot s of the second GEMM. bf16: slots 8q..8q+3 of a 32-wide group
// hold rows 4q..4q+3 of the group's first 16-row unit, slots 8q+4..8q+7 those of its
// second; fp32: the natural order.
int hidden_of_slot(int s, bool bf16) {
  if (!bf16) return s;
  const int g = s / 32, w = s % 32, q = w / 8, j = w % 8;
  return 32 * g + (j < 4 ? 4 * q + j : 16 + 4 * q + (j - 4));
}

// Uploads the image and fills the handle; frees nothing on success.
int upload(const std::vector<unsigned char>& host, pair_transition_handle* h, size_t image,
           void** dptr) {
  hipError_t e = hipMalloc(dptr, host.size());
  if (e != hipSuccess) {
    if (e == hipErrorOutOfMemory) return TRI_MUL_ERR_OUT_OF_MEMORY;
    return hip_fail(e, "hipMalloc(transition weights)");
  }
  e = hipMemcpy(*dptr, host.data(), host.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(*dptr);
    return hip_fail(e, "hipMemcpy(transition weights)");
  }
  unsigned char* d = (unsigned char*)*dptr;
  h->block = *dptr;
  h->image = d;
  h->image_bytes = image;
  h->one = d + align256(image);
  return TRI_MUL_OK;
}

// The wide form's image (bf16): per hidden group g of 32 units, W_1' rows 32g..32g+31
// ([32][czp], chunk c of row r at position c ^ (r & 15)) and W_2's columns of the group
// ([czp][32] in the kernel's row and slot order, chunk q of row R at q ^ ((R >> 2) & 3));
// then b_1' [hp] and b_2 [czp] (kernel row order); then the one-element mask `one`.
int create_wide(const pair_transition_weights* w, int c_z, int hidden, int hp,
                pair_transition_handle** out) {
  const int czp = trimul::transition_wide_czp(c_z), groups = hp / 32;
  const size_t gb = (size_t)128 * czp;
  const size_t image = (size_t)groups * gb + ((size_t)hp + czp) * 4;
  std::vector<unsigned char> host(align256(image) + 256, 0);
  unsigned char* const base = host.data();
  float* hb1 = (float*)(base + (size_t)groups * gb);
  float* hb2 = hb1 + hp;
  store_elem(base + align256(image), 1.0f, true);
  for (int hu = 0; hu < hidden; ++hu) {
    double t = w->b1 ? (double)w->b1[hu] : 0.0;
    const int g = hu / 32, r = hu % 32;
    unsigned char* row = base + (size_t)g * gb + (size_t)r * czp * 2;
    for (int k = 0; k < c_z; ++k) {
      const double wk = w->w1[(size_t)hu * c_z + k];
      const int c = k / 8, e = k % 8, pos = c ^ (r & 15);
      store_elem(row + ((size_t)pos * 8 + e) * 2,
                 (float)(wk * (w->ln_gamma ? (double)w->ln_gamma[k] : 1.0)), true);
      if (w->ln_beta) t += wk * (double)w->ln_beta[k];
    }
    hb1[hu] = (float)t;
  }
  for (int R = 0; R < czp; ++R) {
    const int ch = out_channel(R, true);
    if (ch >= c_z) continue;  // padded output rows stay zero
    hb2[R] = w->b2 ? w->b2[ch] : 0.f;
    for (int s = 0; s < hp; ++s) {
      const int hu = hidden_of_slot(s, true);
      if (hu >= hidden) continue;
      const int g = s / 32, slot = s % 32, qq = slot / 8, e = slot % 8;
      const int pos = qq ^ ((R >> 2) & 3);
      unsigned char* w2g = base + (size_t)g * gb + (size_t)64 * czp;
      store_elem(w2g + ((size_t)R * 32 + pos * 8 + e) * 2, w->w2[(size_t)ch * hidden + hu], true);
    }
  }
  int dev = -1, cus = 0;
  const int rc = check_device(&dev, &cus);
  if (rc != TRI_MUL_OK) return rc;
  pair_transition_handle* h = new (std::nothrow) pair_transition_handle();
  if (!h) return TRI_MUL_ERR_OUT_OF_MEMORY;
  void* dptr = nullptr;
  const int urc = upload(host, h, image, &dptr);
  if (urc != TRI_MUL_OK) {
    delete h;
    return urc;
  }
  h->c_z = c_z;
  h->hidden = hidden;
  h->hp = hp;
  h->dtype = TRI_MUL_BF16;
  h->device = dev;
  h->num_cus = cus;
  h->bf16 = true;
  h->wide = true;
  h->czp = czp;
  *out = h;
  return TRI_MUL_OK;
}

}  // namespace

extern "C" {

int pair_transition_create(const pair_transition_weights* w, int c_z, int hidden, int dtype,
                           pair_transition_handle** out) {
  if (!out) return TRI_MUL_ERR_INVALID_ARG;
  *out = nullptr;
  if (!w || !w->w1 || !w->w2 || c_z < 1 || hidden < 1) return TRI_MUL_ERR_INVALID_ARG;
  if (dtype != TRI_MUL_FP32 && dtype != TRI_MUL_BF16) return TRI_MUL_ERR_UNSUPPORTED;
  const bool bf16 = dtype == TRI_MUL_BF16;
  const int kg = bf16 ? 32 : 16;
  if (hidden > 1 << 20) return TRI_MUL_ERR_UNSUPPORTED;
  const int hp = (hidden + kg - 1) / kg * kg;
  // the weights in one workgroup's LDS if they fit, else streamed through it (bf16)
  const bool wide = !trimul::transition_supported(bf16, c_z, hp);
  if (wide && !trimul::transition_wide_supported(bf16, c_z, hp)) return TRI_MUL_ERR_UNSUPPORTED;
  // the host image first (no device needed), then the device
  if (wide) return create_wide(w, c_z, hidden, hp, out);

  // the kernel's LDS image: W_1' [hp][c_z + pad] | W_2 [c_z][hp + pad] | b_1' [hp] | b_2 [c_z]
  // (pad: one 16-byte chunk of zeros per row), then the one-element mask `one`
  const size_t esz = bf16 ? 2 : 4;
  const size_t pad = 16 / esz;
  const size_t rs1 = (size_t)c_z + pad, rs2 = (size_t)hp + pad;
  const size_t image = trimul::transition_lds_bytes(c_z, hp, esz);
  const size_t total = align256(image) + 256;
  std::vector<unsigned char> host(total, 0);
  unsigned char* hw1 = host.data();
  unsigned char* hw2 = hw1 + (size_t)hp * rs1 * esz;
  float* hb1 = (float*)(hw2 + (size_t)c_z * rs2 * esz);
  float* hb2 = hb1 + hp;
  unsigned char* hone = host.data() + align256(image);
  store_elem(hone, 1.0f, bf16);

  // W_1' = W_1 diag(gamma), b_1' = W_1 beta + b_1 (sums in double); padded units stay 0
  for (int h = 0; h < hidden; ++h) {
    double t = w->b1 ? (double)w->b1[h] : 0.0;
    for (int k = 0; k < c_z; ++k) {
      const double wk = w->w1[(size_t)h * c_z + k];
      store_elem(hw1 + ((size_t)h * rs1 + k) * esz,
                 (float)(wk * (w->ln_gamma ? (double)w->ln_gamma[k] : 1.0)), bf16);
      if (w->ln_beta) t += wk * (double)w->ln_beta[k];
    }
    hb1[h] = (float)t;
  }
  // W_2 and b_2 in the kernel's row and column order
  for (int R = 0; R < c_z; ++R) {
    const int ch = out_channel(R, bf16);
    hb2[R] = w->b2 ? w->b2[ch] : 0.f;
    for (int s = 0; s < hp; ++s) {
      const int hu = hidden_of_slot(s, bf16);
      const float v = hu < hidden ? w->w2[(size_t)ch * hidden + hu] : 0.f;
      store_elem(hw2 + ((size_t)R * rs2 + s) * esz, v, bf16);
    }
  }

  int dev = -1, cus = 0;
  const int rc = check_device(&dev, &cus);
  if (rc != TRI_MUL_OK) return rc;
  pair_transition_handle* h = new (std::nothrow) pair_transition_handle();
  if (!h) return TRI_MUL_ERR_OUT_OF_MEMORY;
  void* dptr = nullptr;
  hipError_t e = hipMalloc(&dptr, total);
  if (e != hipSuccess) {
    delete h;
    if (e == hipErrorOutOfMemory) return TRI_MUL_ERR_OUT_OF_MEMORY;
    return hip_fail(e, "hipMalloc(transition weights)");
  }
  e = hipMemcpy(dptr, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dptr);
    delete h;
    return hip_fail(e, "hipMemcpy(transition weights)");
  }
  unsigned char* d = (unsigned char*)dptr;
  h->c_z = c_z;
  h->hidden = hidden;
  h->hp = hp;
  h->dtype = dtype;
  h->device = dev;
  h->num_cus = cus;
  h->bf16 = bf16;
  h->wide = false;
  h->czp = c_z;
  h->block = dptr;
  h->image = d;
  h->image_bytes = image;
  h->one = d + align256(image);
  *out = h;
  return TRI_MUL_OK;
}

int pair_transition_forward(pair_transition_handle* h, const void* z, const void* pair_mask,
                            void* out, int batch, int n, void* stream) {
  if (!h || !z || !out) return TRI_MUL_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N) return TRI_MUL_ERR_INVALID_ARG;
  const size_t esz = h->bf16 ? 2 : 4;
  if (((uintptr_t)z | (uintptr_t)out) & 15u) return TRI_MUL_ERR_ALIGNMENT;
  if (pair_mask && ((uintptr_t)pair_mask & (uintptr_t)(esz - 1))) return TRI_MUL_ERR_ALIGNMENT;
  const size_t pairs = (size_t)batch * n * n;
  if (pairs > (size_t)32 * 0x7fffffff) return TRI_MUL_ERR_UNSUPPORTED;  // 32-bit tile indices
  const size_t zb = pairs * h->c_z * esz, mb = pairs * esz;
  if ((out != z && overlaps(out, zb, z, zb)) || overlaps(out, zb, pair_mask, mb))
    return TRI_MUL_ERR_ALIAS;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  trimul::TransitionArgs a;
  a.z = z;
  a.mask = pair_mask ? pair_mask : h->one;
  a.out = out;
  a.image = h->image;
  a.image_bytes = h->image_bytes;
  a.pairs = (long long)pairs;
  a.cz = h->c_z;
  a.hp = h->hp;
  a.mask_all = pair_mask ? 0 : 1;
  a.num_cus = h->num_cus;
  a.wide = h->wide ? 1 : 0;
  a.czp = h->czp;
  e = trimul::launch_transition(h->bf16, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launch pair_transition");
  return TRI_MUL_OK;
}

void pair_transition_destroy(pair_transition_handle* h) {
  if (!h) return;
  if (h->block) (void)hipFree(h->block);
  delete h;
}

}  // extern "C"
