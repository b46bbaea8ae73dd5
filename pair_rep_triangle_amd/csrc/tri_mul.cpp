// Host side of the C ABI declared in include/tri_mul.h: argument validation,
// LayerNorm folding and weight packing, workspace layout, stage launches.

#include "tri_mul.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <new>
#include <vector>

#include "host_common.h"
#include "k1w_layout.h"
#include "launch.h"

struct tri_mul_handle {
  int c_z, c, czp, cp, dtype, device, num_cus;
  bool bf16;
  void* block;  // the one device allocation holding every packed weight
  trimul::StageArgs w;  // weight pointers into `block` (activation fields unused)
};

namespace {

using namespace trimul_host;

// Folds y = scale * (W (gamma (.) xhat + beta) + bias) into the stored matrix
// W' = scale * W diag(gamma) (rounded to the storage type, zero-padded from `cols` to
// `colsp`) and the accumulator start t = scale * (W beta + bias). Sums in double.
void fold(const float* W, const float* gamma, const float* beta, const float* bias, int rows,
          int cols, int colsp, bool bf16, double scale, unsigned char* wdst, float* t) {
  for (int r = 0; r < rows; ++r) {
    double trow = bias ? (double)bias[r] : 0.0;
    for (int k = 0; k < colsp; ++k) {
      double v = 0.0;
      if (k < cols) {
        const double wk = W[(size_t)r * cols + k];
        v = scale * wk * (gamma ? (double)gamma[k] : 1.0);
        if (beta) trow += wk * (double)beta[k];
      }
      const float vf = (float)v;
      if (bf16) {
        const uint16_t h = f32_to_bf16_rne(vf);
        memcpy(wdst + ((size_t)r * colsp + k) * 2, &h, 2);
      } else {
        memcpy(wdst + ((size_t)r * colsp + k) * 4, &vf, 4);
      }
    }
    t[r] = (float)(scale * trow);
  }
}

// The wave-independent input gate's weights as its LDS images, one per group of ug units
// (k1w_layout.h): image row lr = 32 uu + 16 gp + r of group g is the stored row
// (2 uq + gp) c + 16 cb + r of unit u = g ug + uu (uq = u / (c / 16): a or b; cb = its
// 16-channel block; gp: gate or projection row), its 16-byte chunk k at position
// k ^ (lr & 15); the rows' start values follow the rows. w1 rows are 256 bytes here.
void build_k1w_images(const unsigned char* w1, const float* t1, int c, int ug, int groups,
                      int esz, unsigned char* dst) {
  if (ug == 0) return;
  const int cblocks = c / 16, rows = ug * 32;
  const size_t rb = trimul::K1W_ROW_BYTES;
  for (int g = 0; g < groups; ++g) {
    unsigned char* img = dst + (size_t)g * trimul::k1w_image_bytes(ug);
    float* timg = (float*)(img + (size_t)rows * rb);
    for (int lr = 0; lr < rows; ++lr) {
      const int uu = lr >> 5, gp = (lr >> 4) & 1, r = lr & 15;
      const int u = g * ug + uu, uq = u / cblocks, cb = u - uq * cblocks;
      const size_t dr = (size_t)(2 * uq + gp) * c + cb * 16 + r;
      for (int k = 0; k < 16; ++k)
        memcpy(img + lr * rb + (size_t)(k ^ (lr & 15)) * 16, w1 + dr * rb + (size_t)k * 16, 16);
      timg[lr] = t1[dr];
    }
  }
  (void)esz;
}

// The streamed output gate's weight image (launch.h): per unit pair k, W_o rows then W_g
// rows of kernel rows 32k .. 32k + 31, chunk c of row r at position c ^ (r & 15); then the
// start values in kernel row order. wo [c_z][cp] and wg [c_z][czp] are the folded bf16
// matrices in channel order; rows of padding channels stay zero.
void build_k3s_image(const unsigned char* wo, const unsigned char* wg, const float* to,
                     const float* tg, int c_z, int cp, int czp, unsigned char* dst) {
  const int steps = czp / 32;
  const size_t gb = (size_t)64 * (cp + czp);
  float* tos = (float*)(dst + (size_t)steps * gb);
  float* tgs = tos + czp;
  for (int R = 0; R < czp; ++R) {
    const int ch = trimul::k3_stream_channel(R);
    const int k = R / 32, r = R % 32;
    unsigned char* blk = dst + (size_t)k * gb;
    if (ch >= c_z) continue;
    tos[R] = to[ch];
    tgs[R] = tg[ch];
    for (int cc = 0; cc < cp / 8; ++cc)
      memcpy(blk + ((size_t)r * cp + (size_t)(cc ^ (r & 15)) * 8) * 2, wo + ((size_t)ch * cp + cc * 8) * 2, 16);
    unsigned char* gblk = blk + (size_t)64 * cp;
    for (int cc = 0; cc < czp / 8; ++cc)
      memcpy(gblk + ((size_t)r * czp + (size_t)(cc ^ (r & 15)) * 8) * 2, wg + ((size_t)ch * czp + cc * 8) * 2, 16);
  }
}

struct Layout {
  size_t a, b, x, total;
  int np, esz;
};

Layout layout_of(const tri_mul_handle* h, int batch, int n) {
  Layout L;
  L.np = trimul::round_up(n, trimul::N_PAD);
  L.esz = h->bf16 ? 2 : 4;
  const size_t one = align256((size_t)batch * h->c * L.np * L.np * L.esz);
  L.a = 0;
  L.b = one;
  L.x = 2 * one;
  L.total = 3 * one;
  return L;
}

int validate_call(const tri_mul_handle* h, int stage, const void* z, const void* mask,
                  const void* out, int batch, int n, int direction, const void* ws,
                  size_t ws_bytes, bool residual) {
  if (!h) return TRI_MUL_ERR_INVALID_ARG;
  if (stage < 0 || stage > 3) return TRI_MUL_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N) return TRI_MUL_ERR_INVALID_ARG;
  if (direction != TRI_MUL_OUTGOING && direction != TRI_MUL_INCOMING) return TRI_MUL_ERR_INVALID_ARG;
  if (!z || !out || !ws) return TRI_MUL_ERR_INVALID_ARG;
  const Layout L = layout_of(h, batch, n);
  if (trimul::k2_grid(L.np, batch, h->c) > 0x7fffffffu) return TRI_MUL_ERR_INVALID_ARG;
  if (((uintptr_t)z | (uintptr_t)out | (uintptr_t)ws) & 15u) return TRI_MUL_ERR_ALIGNMENT;
  if (mask && ((uintptr_t)mask & (uintptr_t)(L.esz - 1))) return TRI_MUL_ERR_ALIGNMENT;
  if (ws_bytes < L.total) return TRI_MUL_ERR_WORKSPACE_TOO_SMALL;
  const size_t pairs = (size_t)batch * n * n;
  const size_t zb = pairs * h->c_z * L.esz, mb = pairs * L.esz;
  // with the residual add, out may be z itself (in place) but not overlap it otherwise
  const bool in_place = residual && out == z;
  if ((!in_place && overlaps(out, zb, z, zb)) || overlaps(out, zb, mask, mb) ||
      overlaps(out, zb, ws, L.total) ||
      overlaps(ws, L.total, z, zb) || overlaps(ws, L.total, mask, mb))
    return TRI_MUL_ERR_ALIAS;
  return TRI_MUL_OK;
}

// The stage arguments of a call (activation pointers may be null for a plan query).
trimul::StageArgs stage_args(const tri_mul_handle* h, const void* z, const void* mask, void* out,
                             int batch, int n, int direction, void* ws, bool residual) {
  const Layout L = layout_of(h, batch, n);
  trimul::StageArgs a = h->w;
  a.z = z;
  a.mask = mask;
  a.out = out;
  a.a = ws ? (unsigned char*)ws + L.a : nullptr;
  a.b = ws ? (unsigned char*)ws + L.b : nullptr;
  a.x = ws ? (unsigned char*)ws + L.x : nullptr;
  a.batch = batch;
  a.n = n;
  a.np = L.np;
  a.incoming = direction == TRI_MUL_INCOMING;
  a.num_cus = h->num_cus;
  a.residual = residual ? 1 : 0;
  a.plan = nullptr;
  a.extents = nullptr;
  return a;
}

// The kernel forms a call of (batch, n) takes.
trimul::KernelPlan plan_of(const tri_mul_handle* h, int batch, int n) {
  trimul::KernelPlan p{};
  trimul::StageArgs a = stage_args(h, nullptr, nullptr, nullptr, batch, n, TRI_MUL_OUTGOING,
                                   nullptr, false);
  a.plan = &p;
  (void)trimul::launch_k1(h->bf16, a, nullptr);
  (void)trimul::launch_k3(h->bf16, a, nullptr);
  return p;
}

int run(tri_mul_handle* h, int stage, const void* z, const void* mask, void* out, int batch, int n,
        int direction, void* ws, size_t ws_bytes, void* stream, bool residual = false,
        const int* extents = nullptr) {
  int rc = validate_call(h, stage, z, mask, out, batch, n, direction, ws, ws_bytes, residual);
  if (rc != TRI_MUL_OK) return rc;
  if (extents) {
    // read by the contraction after the input kernel has written the workspace, and never
    // written by the update
    const size_t eb = (size_t)batch * TRI_MUL_EXTENT_PARTS * sizeof(int);
    const size_t zb = (size_t)batch * n * n * h->c_z * (h->bf16 ? 2 : 4);
    if ((uintptr_t)extents & 3u) return TRI_MUL_ERR_ALIGNMENT;
    if (overlaps(extents, eb, ws, layout_of(h, batch, n).total) || overlaps(extents, eb, out, zb))
      return TRI_MUL_ERR_ALIAS;
  }
  // In place, each pair of z must be read (all c_z channels, for the gate's LayerNorm)
  // before any of it is overwritten. That holds only while one workgroup produces all
  // output channels of a pair; with several channel groups another group may already
  // have stored its slice.
  if (residual && out == z && plan_of(h, batch, n).k3_groups > 1) return TRI_MUL_ERR_ALIAS;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  trimul::StageArgs a = stage_args(h, z, mask, out, batch, n, direction, ws, residual);
  a.extents = extents;
  hipStream_t st = (hipStream_t)stream;
  if (stage == 0 || stage == 1) {
    e = trimul::launch_k1(h->bf16, a, st);
    if (e != hipSuccess) return hip_fail(e, "launch k1_input_gate");
  }
  if (stage == 0 || stage == 2) {
    e = trimul::launch_k2(h->bf16, a, st);
    if (e != hipSuccess) return hip_fail(e, "launch k2_contract");
  }
  if (stage == 0 || stage == 3) {
    e = trimul::launch_k3(h->bf16, a, st);
    if (e != hipSuccess) return hip_fail(e, "launch k3_output_gate");
  }
  return TRI_MUL_OK;
}

}  // namespace

extern "C" {

int tri_mul_create(const tri_mul_weights* w, int c_z, int c, int dtype, tri_mul_handle** out) {
  if (!out) return TRI_MUL_ERR_INVALID_ARG;
  *out = nullptr;
  if (!w || !w->w_a_gate || !w->w_a_proj || !w->w_b_gate || !w->w_b_proj || !w->w_out ||
      !w->w_gate)
    return TRI_MUL_ERR_INVALID_ARG;
  if (c_z < 1 || c < 1) return TRI_MUL_ERR_INVALID_ARG;
  if (dtype != TRI_MUL_FP32 && dtype != TRI_MUL_BF16) return TRI_MUL_ERR_UNSUPPORTED;
  const bool bf16 = dtype == TRI_MUL_BF16;
  if (c_z % 16 || c % 16) return TRI_MUL_ERR_UNSUPPORTED;
  if (bf16 ? (c_z > TRI_MUL_MAX_WIDTH || c > TRI_MUL_MAX_WIDTH)
           : (c_z > TRI_MUL_MAX_WIDTH_FP32_CZ || c > TRI_MUL_MAX_WIDTH_FP32_C))
    return TRI_MUL_ERR_UNSUPPORTED;
  // the host image first (no device needed), then the device
  const int kg = trimul::k_group(bf16);
  int kx = 0, kz = 0;
  if (!trimul::padded_ksteps(c, c_z, bf16, &kx, &kz)) return TRI_MUL_ERR_UNSUPPORTED;
  const int czp = kg * kz, cp = kg * kx;
  const int esz = bf16 ? 2 : 4;
  const double ng = -1.4426950408889634;  // -log2(e): gate rows feed exp2 directly
  // block: w1 | wo | wg | t1 | to | tg
  const size_t w1b = align256((size_t)4 * c * czp * esz);
  const size_t wob = align256((size_t)c_z * cp * esz);
  const size_t wgb = align256((size_t)c_z * czp * esz);
  const size_t t1b = align256((size_t)4 * c * sizeof(float));
  const size_t tob = align256((size_t)c_z * sizeof(float));
  const size_t oneb = 256;
  // the wave-independent input gate (four chunk groups along c_z) reads its weights as one
  // LDS image per unit group
  const int k1w_ug = czp == 4 * kg ? trimul::k1w_group_units(c) : 0;
  const int k1w_groups = k1w_ug ? 2 * (c / 16) / k1w_ug : 0;
  const size_t k1wb = align256((size_t)k1w_groups * (k1w_ug ? trimul::k1w_image_bytes(k1w_ug) : 0));
  // the streamed output gate (bf16, c_z above 128) reads its weights as a stream of unit
  // pairs (launch.h)
  const bool k3s = bf16 && czp > 128 && trimul::k3_stream_variant(kx, kz) &&
                   trimul::k3_stream_lds(cp, czp) <= trimul::LDS_PER_CU;
  const size_t k3sb = k3s ? align256((size_t)(czp / 32) * 64 * (cp + czp) + (size_t)2 * czp * 4) : 0;
  const size_t total = w1b + wob + wgb + t1b + 2 * tob + oneb + k1wb + k3sb;
  std::vector<unsigned char> host(total, 0);
  unsigned char* hw1 = host.data();
  unsigned char* hwo = hw1 + w1b;
  unsigned char* hwg = hwo + wob;
  float* ht1 = (float*)(hwg + wgb);
  float* hto = (float*)((unsigned char*)ht1 + t1b);
  float* htg = (float*)((unsigned char*)hto + tob);
  unsigned char* hone = (unsigned char*)htg + tob;
  if (bf16) {
    const uint16_t one = 0x3f80;  // 1.0 in bf16
    memcpy(hone, &one, 2);
  } else {
    const float one = 1.0f;
    memcpy(hone, &one, 4);
  }
  const float* mats[4] = {w->w_a_gate, w->w_a_proj, w->w_b_gate, w->w_b_proj};
  const float* biases[4] = {w->b_a_gate, w->b_a_proj, w->b_b_gate, w->b_b_proj};
  for (int q = 0; q < 4; ++q)
    fold(mats[q], w->ln_in_gamma, w->ln_in_beta, biases[q], c, c_z, czp, bf16,
         (q % 2 == 0) ? ng : 1.0, hw1 + (size_t)q * c * czp * esz, ht1 + q * c);
  fold(w->w_out, w->ln_out_gamma, w->ln_out_beta, w->b_out, c_z, c, cp, bf16, 1.0, hwo, hto);
  fold(w->w_gate, w->ln_in_gamma, w->ln_in_beta, w->b_gate, c_z, c_z, czp, bf16, ng, hwg, htg);
  unsigned char* himg = hone + oneb;
  build_k1w_images(hw1, ht1, c, k1w_ug, k1w_groups, esz, himg);  // rows of czp * esz = 256 bytes
  unsigned char* hk3s = himg + k1wb;
  if (k3s) build_k3s_image(hwo, hwg, hto, htg, c_z, cp, czp, hk3s);

  int dev = -1, cus = 0;
  int rc = check_device(&dev, &cus);
  if (rc != TRI_MUL_OK) return rc;
  // set-up of the allocation-free entry point on this device: the lookup's result is kept
  // per device and a failure is reported by tri_mul_forward_static itself
  void* static_ws = nullptr;
  (void)static_workspace(dev, &static_ws);

  tri_mul_handle* h = new (std::nothrow) tri_mul_handle();
  if (!h) return TRI_MUL_ERR_OUT_OF_MEMORY;
  void* dptr = nullptr;
  hipError_t e = hipMalloc(&dptr, total);
  if (e != hipSuccess) {
    delete h;
    if (e == hipErrorOutOfMemory) return TRI_MUL_ERR_OUT_OF_MEMORY;
    return hip_fail(e, "hipMalloc(weights)");
  }
  e = hipMemcpy(dptr, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dptr);
    delete h;
    return hip_fail(e, "hipMemcpy(weights)");
  }
  unsigned char* d = (unsigned char*)dptr;
  h->c_z = c_z;
  h->c = c;
  h->czp = czp;
  h->cp = cp;
  h->dtype = dtype;
  h->device = dev;
  h->num_cus = cus;
  h->bf16 = bf16;
  h->block = dptr;
  trimul::StageArgs& a = h->w;
  memset(&a, 0, sizeof(a));
  a.w1 = d;
  a.wo = d + w1b;
  a.wg = d + w1b + wob;
  a.t1 = (const float*)(d + ((unsigned char*)ht1 - hw1));
  a.to = (const float*)(d + ((unsigned char*)hto - hw1));
  a.tg = (const float*)(d + ((unsigned char*)htg - hw1));
  a.one = d + (hone - hw1);
  a.k1w_image = k1w_ug ? d + (himg - hw1) : nullptr;
  a.k3s_image = k3s ? d + (hk3s - hw1) : nullptr;
  a.cz = c_z;
  a.czp = czp;
  a.c = c;
  a.cp = cp;
  *out = h;
  return TRI_MUL_OK;
}

int tri_mul_workspace_bytes(const tri_mul_handle* h, int batch, int n, size_t* bytes) {
  if (!h || !bytes || batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N)
    return TRI_MUL_ERR_INVALID_ARG;
  *bytes = layout_of(h, batch, n).total;
  return TRI_MUL_OK;
}

int tri_mul_workspace_layout(const tri_mul_handle* h, int batch, int n, tri_mul_layout* out) {
  if (!h || !out || batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N)
    return TRI_MUL_ERR_INVALID_ARG;
  const Layout L = layout_of(h, batch, n);
  out->a_offset = L.a;
  out->b_offset = L.b;
  out->x_offset = L.x;
  out->total_bytes = L.total;
  out->n_pad = L.np;
  out->elem_bytes = L.esz;
  return TRI_MUL_OK;
}

int tri_mul_query_plan(const tri_mul_handle* h, int batch, int n, tri_mul_plan* out) {
  if (!h || !out || batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N)
    return TRI_MUL_ERR_INVALID_ARG;
  const trimul::KernelPlan p = plan_of(h, batch, n);
  out->input_form = p.k1_form;
  out->output_form = p.k3_form;
  out->output_groups = p.k3_groups;
  out->in_place_ok = p.k3_groups == 1;
  out->n_pad = layout_of(h, batch, n).np;
  return TRI_MUL_OK;
}

int tri_mul_forward(tri_mul_handle* h, const void* z, const void* pair_mask, void* out, int batch,
                    int n, int direction, void* workspace, size_t workspace_bytes, void* stream) {
  return run(h, 0, z, pair_mask, out, batch, n, direction, workspace, workspace_bytes, stream);
}

int tri_mul_forward_residual(tri_mul_handle* h, const void* z, const void* pair_mask, void* z_out,
                             int batch, int n, int direction, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return run(h, 0, z, pair_mask, z_out, batch, n, direction, workspace, workspace_bytes, stream,
             true);
}

int tri_mul_mask_extents(int dtype, const void* pair_mask, int batch, int n, int* extents,
                         void* stream) {
  if (dtype != TRI_MUL_FP32 && dtype != TRI_MUL_BF16) return TRI_MUL_ERR_UNSUPPORTED;
  if (!pair_mask || !extents || batch < 1 || batch > 65535 || n < 1 || n > TRI_MUL_MAX_N)
    return TRI_MUL_ERR_INVALID_ARG;
  const size_t esz = dtype == TRI_MUL_BF16 ? 2 : 4;
  if (((uintptr_t)pair_mask & (esz - 1)) || ((uintptr_t)extents & 3u)) return TRI_MUL_ERR_ALIGNMENT;
  if (overlaps(extents, (size_t)batch * TRI_MUL_EXTENT_PARTS * sizeof(int), pair_mask,
               (size_t)batch * n * n * esz))
    return TRI_MUL_ERR_ALIAS;
  // the current device's architecture, checked once per device (this call runs once per
  // model forward, next to launches that take microseconds)
  static std::atomic<int> checked[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  if (checked[dev].load() == 0) {
    int d = -1, cus = 0;
    const int rc = check_device(&d, &cus);
    if (rc != TRI_MUL_OK && rc != TRI_MUL_ERR_UNSUPPORTED_DEVICE) return rc;
    checked[dev].store(rc == TRI_MUL_OK ? 1 : -1);
  }
  if (checked[dev].load() < 0) return TRI_MUL_ERR_UNSUPPORTED_DEVICE;
  e = trimul::launch_k0(dtype == TRI_MUL_BF16, pair_mask, batch, n, extents,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launch k0_mask_extents");
  return TRI_MUL_OK;
}

int tri_mul_forward_extents(tri_mul_handle* h, const void* z, const void* pair_mask,
                            const int* extents, void* out, int batch, int n, int direction,
                            int residual, void* workspace, size_t workspace_bytes, void* stream) {
  if (!extents || !pair_mask || (residual != 0 && residual != 1)) return TRI_MUL_ERR_INVALID_ARG;
  return run(h, 0, z, pair_mask, out, batch, n, direction, workspace, workspace_bytes, stream,
             residual == 1, extents);
}

int tri_mul_forward_stage(tri_mul_handle* h, int stage, const void* z, const void* pair_mask,
                          void* out, int batch, int n, int direction, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 3) return TRI_MUL_ERR_INVALID_ARG;
  return run(h, stage, z, pair_mask, out, batch, n, direction, workspace, workspace_bytes, stream);
}

void tri_mul_destroy(tri_mul_handle* h) {
  if (!h) return;
  if (h->block) (void)hipFree(h->block);
  delete h;
}

const char* tri_mul_strerror(int code) {
  switch (code) {
    case TRI_MUL_OK: return "ok";
    case TRI_MUL_ERR_INVALID_ARG: return "invalid argument (NULL pointer, size out of range or bad enum)";
    case TRI_MUL_ERR_UNSUPPORTED: return "unsupported configuration (c_z and c multiples of 16; at most 512 for bf16, c_z 256 / c 128 for fp32; dtype fp32 or bf16)";
    case TRI_MUL_ERR_UNSUPPORTED_DEVICE: return "unsupported device (needs gfx950, the device the handle was created on)";
    case TRI_MUL_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case TRI_MUL_ERR_ALIAS: return "output or workspace overlaps another buffer";
    case TRI_MUL_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than tri_mul_workspace_bytes()";
    case TRI_MUL_ERR_HIP: return "HIP runtime error (see tri_mul_last_hip_error)";
    case TRI_MUL_ERR_OUT_OF_MEMORY: return "out of device memory";
    default: return "unknown error code";
  }
}

const char* tri_mul_last_hip_error(void) { return trimul_host::g_hip_err; }

}  // extern "C"
