/* Triangular attention on MI355X (gfx950): C ABI of libtrimul.so.
 *
 * Attention over the third residue k of every pair (i, j) of z [B][N][N][c_z], H heads
 * of width d, around the starting node (keys: the pairs (i, k) of the row, pair bias
 * from (j, k)) or the ending node (keys: the pairs (k, j) of the column, bias from
 * (k, i)):
 *
 *   zhat = LayerNorm_cz(z)                                  eps TRI_MUL_LN_EPS, biased var
 *   q, k, v, per head: W_q zhat, W_k zhat, W_v zhat; beta = w_b . zhat (per head)
 *   g = sigmoid(W_g zhat + b_g)
 *   starting: o_ij = g_ij * sum_k softmax_k(q_ij . k_ik / sqrt(d) + beta_jk) v_ik
 *   ending:   o_ij = g_ij * sum_k softmax_k(q_ij . k_kj / sqrt(d) + beta_ki) v_kj
 *   out_ij = W_o concat_heads(o_ij) + b_o
 *
 * Key pairs with mask 0 are left out of the softmax; a query whose row (starting) or
 * column (ending) has no valid key pair gets a zero attention output. The output is not
 * masked and has no residual.
 *
 * Sources: the yage.ai summary of the biomolecular-software report (triangular
 * attention and the triangular multiplicative update as the pair operations of cubic
 * cost; a fused kernel for triangular attention) and the OpenFold-TRT summary
 * (triangular attention among the accelerated pair kernels). The pages print no
 * equations; the definition above is the reading this library implements.
 *
 * Conventions as in tri_mul.h: error codes TRI_MUL_OK / TRI_MUL_ERR_* (text from
 * tri_mul_strerror, HIP details from tri_mul_last_hip_error), device pointers 16-byte
 * aligned, forward calls only enqueue work (no allocation, no synchronisation).
 */
#ifndef TRI_ATTENTION_H
#define TRI_ATTENTION_H

#include <stddef.h>

#include "tri_mul.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TRI_ATTN_STARTING = 0, TRI_ATTN_ENDING = 1 } tri_attn_node;

/* Host fp32 weights, nn.Linear orientation ([out][in], row-major); the H heads are
 * stacked along the output rows (rows h*d .. h*d + d - 1 belong to head h). NULL gamma
 * means ones, NULL beta / b_g / b_o mean zeros; the matrices are required. */
typedef struct tri_attn_weights {
  const float *ln_gamma, *ln_beta;  /* [c_z]                          */
  const float *w_q, *w_k, *w_v;     /* [H*d][c_z] each                */
  const float* w_b;                 /* [H][c_z]   pair bias per head  */
  const float *w_g, *b_g;           /* [H*d][c_z], [H*d]  gate        */
  const float *w_o, *b_o;           /* [c_z][H*d], [c_z]  output      */
} tri_attn_weights;

typedef struct tri_attn_handle tri_attn_handle;

/* Build a handle on the current device (must be gfx950): folds the LayerNorm into the
 * projections, the 1/sqrt(d) scale and log2(e) into W_q and log2(e) into w_b (the
 * softmax runs in base 2), and stores the weights on the device in the kernels' order.
 * Supported: dtype TRI_MUL_BF16 (storage of z, out and the intermediates; fp32
 * accumulation and softmax); c_z a multiple of 32 up to 384; head width d = 32;
 * heads 1..8. Projection weights that do not fit one workgroup's LDS are split into
 * parts, and the projection runs once per part; the output projection's weights pass
 * through LDS 128 rows at a time. The weights are copied: the host arrays may be freed on
 * return.
 * Errors: INVALID_ARG (NULL w / matrix / out, sizes < 1), UNSUPPORTED (other shapes or
 * dtype), UNSUPPORTED_DEVICE, OUT_OF_MEMORY, HIP. On error *out is NULL. */
int tri_attn_create(const tri_attn_weights* w, int c_z, int heads, int head_dim, int dtype,
                    tri_attn_handle** out);

/* Bytes of the caller-owned workspace a forward call over batch x n x n needs: the
 * per-head q, k, gate and transposed v, the pair bias and the mask, each over the
 * pair grid padded to a multiple of 64 per side. */
int tri_attn_workspace_bytes(const tri_attn_handle* h, int batch, int n, size_t* bytes);

/* out = triangular attention of z around `node` (tri_attn_node), enqueued on `stream`
 * (a hipStream_t; NULL = default stream). z, out: [batch][n][n][c_z] bf16; pair_mask:
 * [batch][n][n] bf16 (values 0 / 1) or NULL for all ones; workspace: ws_bytes >=
 * tri_attn_workspace_bytes. The caller owns every buffer. Errors: INVALID_ARG (NULL
 * handle / z / out / workspace, batch or n out of range, unknown node), ALIGNMENT,
 * ALIAS (out overlaps z, the mask or the workspace), WORKSPACE_TOO_SMALL,
 * UNSUPPORTED_DEVICE, HIP. */
int tri_attn_forward(tri_attn_handle* h, const void* z, const void* pair_mask, void* out,
                     int batch, int n, int node, void* workspace, size_t ws_bytes,
                     void* stream);

/* One of the two kernels of tri_attn_forward alone, with the same arguments: stage 1 =
 * the projection (LayerNorm, q, k, gate, v, pair bias and mask into the workspace),
 * stage 2 = the attention and output projection (reads the workspace stage 1 wrote for
 * the same z, mask and node). For tests and per-kernel timing. Errors as
 * tri_attn_forward, INVALID_ARG for another stage. */
int tri_attn_forward_stage(tri_attn_handle* h, int stage, const void* z, const void* pair_mask,
                           void* out, int batch, int n, int node, void* workspace,
                           size_t ws_bytes, void* stream);

/* Release the handle's device weights (NULL is ignored). */
void tri_attn_destroy(tri_attn_handle* h);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTENTION_H */
