/* Pair transition on MI355X (gfx950): C ABI of libtrimul.so.
 *
 * Applied as a masked residual on the pair representation z [B][N][N][c_z]:
 *
 *   out_bij = z_bij + m_bij * (W_2 relu(W_1 LN(z_bij) + b_1) + b_2)
 *
 * RFProteína architecture page: "Inside the velocity network" (each pair update ends
 * with a pair transition, applied as a masked residual) and, under "Kernel support",
 * the pair-transition paragraph of "Dispatch and fallback" (both linears, the ReLU,
 * the mask and the residual in one launch, the hidden activation kept on chip; the
 * released pair width uses an
 * expansion of 2, hidden = 2 c_z). The LayerNorm over c_z (biased variance, epsilon
 * TRI_MUL_LN_EPS) is the pre-norm the pages run as a separate norm kernel; here it is
 * folded into W_1 and b_1.
 *
 * Conventions as in tri_mul.h: error codes TRI_MUL_OK / TRI_MUL_ERR_* (text from
 * tri_mul_strerror, HIP details from tri_mul_last_hip_error), dtypes TRI_MUL_FP32 /
 * TRI_MUL_BF16 (storage type of z, mask and out; fp32 accumulation), device pointers
 * 16-byte aligned, nothing allocated or synchronised by the forward call.
 */
#ifndef PAIR_TRANSITION_H
#define PAIR_TRANSITION_H

#include <stddef.h>

#include "tri_mul.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Host fp32 weights, nn.Linear orientation ([out][in], row-major). NULL ln_gamma means
 * ones; NULL ln_beta, b1 or b2 mean zeros. Copied by pair_transition_create. */
typedef struct pair_transition_weights {
  const float* ln_gamma; /* [c_z]           */
  const float* ln_beta;  /* [c_z]           */
  const float* w1;       /* [hidden][c_z]   */
  const float* b1;       /* [hidden]        */
  const float* w2;       /* [c_z][hidden]   */
  const float* b2;       /* [c_z]           */
} pair_transition_weights;

typedef struct pair_transition_handle pair_transition_handle;

/* Build a handle on the current device (must be gfx950): folds the LayerNorm into W_1
 * and b_1, rounds the weights to `dtype` and stores them on the device in the kernel's
 * order. Supported, with hidden >= 1 padded with zero units to a multiple of 32 (bf16)
 * or 16 (fp32):
 *   - weights resident in LDS: c_z a multiple of 32 up to 128 (bf16) or of 16 up to 64
 *     (fp32), when the padded weights of both layers (16 bytes of padding per row) and
 *     the fp32 biases fit one workgroup's 160 KB of LDS (bf16 c_z = 128: hidden <= 288);
 *   - otherwise, bf16 only, weights streamed through LDS one group of 32 hidden units at
 *     a time: c_z a multiple of 32 up to 512 (padded with zero channels to 128, 256, 384
 *     or 512) and hidden with 256 c_z_padded + 4 (hidden_padded + c_z_padded) bytes
 *     within 160 KB (c_z = 384: hidden <= 15744), which covers the released pair width
 *     384 with hidden 768.
 * Returns TRI_MUL_ERR_UNSUPPORTED for other shapes, TRI_MUL_ERR_INVALID_ARG for NULL
 * w / w1 / w2 / out or non-positive sizes. On error *out is NULL. */
int pair_transition_create(const pair_transition_weights* w, int c_z, int hidden, int dtype,
                           pair_transition_handle** out);

/* out = z + m * transition(z) for all B x N x N pairs, enqueued on `stream` (a
 * hipStream_t; NULL = default stream). z, out: [batch][n][n][c_z] in the handle's dtype;
 * pair_mask: [batch][n][n] in the same dtype, or NULL for all ones. out may be z itself
 * (in place); any other overlap of out with z or the mask is TRI_MUL_ERR_ALIAS. The
 * caller keeps ownership of every buffer. Errors: INVALID_ARG (NULL handle / z / out,
 * batch or n out of range), ALIGNMENT (z or out not 16-byte aligned, mask not aligned
 * to its element), ALIAS, UNSUPPORTED (more than 32 * (2^31 - 1) pairs),
 * UNSUPPORTED_DEVICE (not the handle's device), HIP. */
int pair_transition_forward(pair_transition_handle* h, const void* z, const void* pair_mask,
                            void* out, int batch, int n, void* stream);

/* Release the handle's device weights (NULL is ignored). */
void pair_transition_destroy(pair_transition_handle* h);

#ifdef __cplusplus
}
#endif

#endif /* PAIR_TRANSITION_H */
