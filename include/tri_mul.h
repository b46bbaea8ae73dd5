/*
 * tri_mul.h -- C ABI of the MI355X (gfx950) triangle multiplicative update.
 *
 * The operator (per batch item b and residue pair (i, j)):
 *   zhat = LayerNorm_cz(z_bij; gamma_in, beta_in)            eps 1e-5, biased var
 *   a_bij = m_bij * sigmoid(W_ag zhat + b_ag) * (W_ap zhat + b_ap)     [c]
 *   b_bij = m_bij * sigmoid(W_bg zhat + b_bg) * (W_bp zhat + b_bp)     [c]
 *   outgoing: x_bij = sum_k a_bik * b_bjk     incoming: x_bij = sum_k a_bki * b_bkj
 *   out_bij = m_bij * sigmoid(W_g zhat + b_g) * (W_o LayerNorm_c(x_bij; gamma_out, beta_out) + b_o)
 * Sources: RFProteína architecture page (BioNeMo Inference Runtime docs),
 * "Triangle multiplication on SM90" (the K1 -> K2 -> K3 chain: input projection
 * with the input LayerNorm folded in, the contraction compiled per direction,
 * output gate and projection with both LayerNorms folded in) and "Dual-GEMM
 * gates" (the x_x form sigma(x W_g^T + b_g) * (x W_p^T + b_p) for the input
 * gate, which absorbs the pair mask and emits its output transposed for the
 * contraction; the x0_x1 form for the output gate, x0 = normalized input pair
 * tensor, x1 = contracted hidden tensor). The index pattern of the two
 * directions and the zero output on padded pairs are readings, not printed on
 * the pages.
 *
 * Conventions
 *   - Every function returns TRI_MUL_OK (0) or a negative TRI_MUL_ERR_* code;
 *     tri_mul_strerror() names it. There is no fallback path: an unsupported
 *     request is rejected, never silently run another way.
 *   - Device pointers are HIP device memory on the device that was current at
 *     tri_mul_create(); that device must be current at every forward call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Forward calls only enqueue work: they never allocate, never synchronise
 *     and return before the GPU has finished.
 */
#ifndef TRI_MUL_H
#define TRI_MUL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_MUL_OK 0
#define TRI_MUL_ERR_INVALID_ARG -1        /* NULL pointer, size out of range, bad enum   */
#define TRI_MUL_ERR_UNSUPPORTED -2        /* width not a multiple of 16 / too large, dtype */
#define TRI_MUL_ERR_UNSUPPORTED_DEVICE -3 /* current device is not gfx950 / wrong device */
#define TRI_MUL_ERR_ALIGNMENT -4          /* a device pointer not 16-byte aligned         */
#define TRI_MUL_ERR_ALIAS -5              /* out or workspace overlaps another buffer     */
#define TRI_MUL_ERR_WORKSPACE_TOO_SMALL -6
#define TRI_MUL_ERR_HIP -7                /* a HIP runtime call or launch failed          */
#define TRI_MUL_ERR_OUT_OF_MEMORY -8      /* tri_mul_create could not allocate weights    */

#define TRI_MUL_MAX_N 32768               /* residues per side                            */
#define TRI_MUL_MAX_WIDTH 512             /* largest c_z and c, bf16                      */
#define TRI_MUL_MAX_WIDTH_FP32_CZ 256     /* largest c_z, fp32                            */
#define TRI_MUL_MAX_WIDTH_FP32_C 128      /* largest c, fp32                              */
#define TRI_MUL_LN_EPS 1e-5f              /* epsilon of both LayerNorms                   */
/* size of the library's own workspace for tri_mul_forward_static (256 MiB per GPU) */
#define TRI_MUL_STATIC_WORKSPACE_BYTES (256ull * 1024ull * 1024ull)

typedef enum { TRI_MUL_FP32 = 0, TRI_MUL_BF16 = 1 } tri_mul_dtype;
typedef enum { TRI_MUL_OUTGOING = 0, TRI_MUL_INCOMING = 1 } tri_mul_direction;

/* Host fp32 weights, nn.Linear orientation: a matrix is [out][in], row-major.
 * NULL gamma means all ones; NULL beta and NULL bias mean zeros; the weight
 * matrices themselves are required. The arrays are read during
 * tri_mul_create() only and may be freed when it returns. */
typedef struct tri_mul_weights {
  const float *ln_in_gamma, *ln_in_beta;                  /* [c_z]               */
  const float *w_a_gate, *b_a_gate, *w_a_proj, *b_a_proj; /* [c][c_z], [c]       */
  const float *w_b_gate, *b_b_gate, *w_b_proj, *b_b_proj; /* [c][c_z], [c]       */
  const float *ln_out_gamma, *ln_out_beta;                /* [c]                 */
  const float *w_out, *b_out;                             /* [c_z][c], [c_z]     */
  const float *w_gate, *b_gate;                           /* [c_z][c_z], [c_z]   */
} tri_mul_weights;

typedef struct tri_mul_handle tri_mul_handle;

/* Where the intermediates live inside a workspace (byte offsets from its
 * start). a, b and x are each [batch][c][n_pad][n_pad] in the handle's dtype,
 * n_pad = n rounded up to a multiple of 64, entries outside n x n are zero
 * for a and b. For outgoing, a[b][ch][i][k] = a_bik; for incoming the input
 * kernel stores the operands transposed, a[b][ch][i][k] = a_bki (same for b),
 * so the contraction is x[b][ch][i][j] = sum_k a[..][i][k] * b[..][j][k] in
 * both directions. */
typedef struct tri_mul_layout {
  size_t a_offset, b_offset, x_offset; /* bytes                         */
  size_t total_bytes;                  /* = tri_mul_workspace_bytes()   */
  int n_pad;                           /* padded side of a, b and x     */
  int elem_bytes;                      /* 2 (bf16) or 4 (fp32)          */
} tri_mul_layout;

/* Which kernel forms a call of (batch, n) takes (tri_mul_query_plan). The input and the
 * output kernel each come in a wave-independent form (weights in LDS, every wave runs its
 * own tiles) and a tile-shared form (weights in registers, tiles shared through LDS); the
 * output kernel also in a streamed form for wide pair tracks (bf16, c_z above 128: its
 * weights stream through LDS, one workgroup produces every channel of its pairs). The
 * choice depends on the widths and on the size of one batch item's operands. */
typedef struct tri_mul_plan {
  int input_form;    /* 0 wave-independent, 1 tile-shared                        */
  int output_form;   /* 0 wave-independent, 1 tile-shared, 2 streamed weights    */
  int output_groups; /* output-channel groups the output kernel splits c_z into  */
  int in_place_ok;   /* 1 when tri_mul_forward_residual may take z_out == z      */
  int n_pad;         /* padded side of the workspace planes                      */
} tri_mul_plan;

/* Build a handle: checks c_z, c (multiples of 16; at most TRI_MUL_MAX_WIDTH for
 * bf16, TRI_MUL_MAX_WIDTH_FP32_CZ / _C for fp32) and dtype, checks that the current
 * device is gfx950, folds both LayerNorm
 * affines into the projection weights (in double precision), converts them to
 * `dtype` and copies them to the current device. The only call that allocates.
 * On error *out is set to NULL. */
int tri_mul_create(const tri_mul_weights* weights, int c_z, int c, int dtype,
                   tri_mul_handle** out);

/* Bytes of workspace a forward call needs for (batch, n). */
int tri_mul_workspace_bytes(const tri_mul_handle* h, int batch, int n, size_t* bytes);

/* Offsets of a, b and x inside the workspace (see tri_mul_layout). */
int tri_mul_workspace_layout(const tri_mul_handle* h, int batch, int n, tri_mul_layout* out);

/* The kernel forms a forward call of (batch, n) takes (see tri_mul_plan). Enqueues nothing.
 * Errors: INVALID_ARG for a NULL handle or output, batch or n out of range. */
int tri_mul_query_plan(const tri_mul_handle* h, int batch, int n, tri_mul_plan* out);

/* The whole update for one direction: enqueues the three kernels on `stream`.
 *   z          [batch][n][n][c_z]  contiguous, handle dtype, 16-byte aligned
 *   pair_mask  [batch][n][n]       contiguous, handle dtype (0/1); NULL = all ones
 *   out        [batch][n][n][c_z]  contiguous, handle dtype; must not overlap
 *                                  z, pair_mask or the workspace
 *   workspace  >= tri_mul_workspace_bytes(h, batch, n) bytes, 16-byte aligned,
 *              must not overlap z, pair_mask or out; contents on entry ignored.
 * Several streams may share a handle if each call has its own workspace. */
int tri_mul_forward(tri_mul_handle* h, const void* z, const void* pair_mask, void* out,
                    int batch, int n, int direction, void* workspace, size_t workspace_bytes,
                    void* stream);

/* The update followed by its residual add, in one pass over the output:
 *   z_out = z + out,  out as in tri_mul_forward (so z_out = z on pairs with mask 0).
 * The masked residual add of a pair-update step, fused into the last kernel (the
 * kernel table on the RFProteína architecture page lists it as the separate "masked
 * residual" kernel after each pair operation). Running it for the outgoing direction
 * and then, on its result, for the incoming direction is the pair update's order
 * ("Inside the velocity network": outgoing, then incoming triangle multiplication).
 *   z_out  [batch][n][n][c_z], handle dtype, 16-byte aligned; either z itself (in
 *          place) or a buffer that does not overlap z, pair_mask or the workspace.
 *          In place needs the output kernel to produce every channel of a pair in one
 *          workgroup (tri_mul_plan.in_place_ok: always for bf16 c_z <= 128 and
 *          fp32 c_z <= 64, for wider shapes only where the plan says so); otherwise z_out == z returns
 *          TRI_MUL_ERR_ALIAS, because one channel group could overwrite z before
 *          another has read it.
 * The sum is taken in fp32 and rounded once to the handle dtype. Other arguments and
 * errors as for tri_mul_forward. */
int tri_mul_forward_residual(tri_mul_handle* h, const void* z, const void* pair_mask,
                             void* z_out, int batch, int n, int direction, void* workspace,
                             size_t workspace_bytes, void* stream);

/* tri_mul_forward for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the a | b | x workspace is a file-scope device array of
 * TRI_MUL_STATIC_WORKSPACE_BYTES inside this library, one per GPU, held until the
 * process ends. The call allocates nothing and enqueues the same three kernels as
 * tri_mul_forward.
 *   - Calls whose tri_mul_workspace_bytes(h, batch, n) exceeds the array return
 *     TRI_MUL_ERR_WORKSPACE_TOO_SMALL before any launch (bf16, c = 128: batch * n_pad^2
 *     up to 349525, e.g. batch 1 with n <= 576).
 *   - Every call on one GPU shares that GPU's array, whatever the handle: calls that may
 *     overlap on one GPU (several streams, several host threads) race on it and must be
 *     ordered by the caller. Nothing needs the array cleared between calls.
 *   - The array's device address is looked up once per device (at tri_mul_create on the
 *     handle's device, else at the first call); a failed lookup returns TRI_MUL_ERR_HIP.
 * Other arguments and errors as for tri_mul_forward. */
int tri_mul_forward_static(tri_mul_handle* h, const void* z, const void* pair_mask, void* out,
                           int batch, int n, int direction, void* stream);

/* Mask extents, computed once per model forward and reused by every update that shares the
 * mask (the RFProteína architecture page, "Dual-GEMM gates": the input gate takes the
 * left-aligned pair mask as per-row valid counts computed once per forward and reused by
 * all pair updates). For batch item b the extent is
 *   L_b = 1 + max{ max(i, j) : pair_mask[b][i][j] != 0 },   0 if the item has no nonzero,
 * the side of the smallest leading square holding every nonzero pair; for the outer
 * product of a left-aligned residue mask it is the item's valid length.
 *   pair_mask  [batch][n][n], dtype TRI_MUL_BF16 or TRI_MUL_FP32 (element-aligned)
 *   extents    [batch][TRI_MUL_EXTENT_PARTS] int32 device memory, 4-byte aligned, must not
 *              overlap the mask; receives partial maxima (L_b is the largest of its item's
 *              entries). Fully written by the call: no clearing needed, reusable as is.
 * Enqueues one small kernel on `stream`. Errors: INVALID_ARG (NULL, sizes), UNSUPPORTED
 * (dtype), ALIGNMENT, ALIAS, UNSUPPORTED_DEVICE, HIP. */
#define TRI_MUL_EXTENT_PARTS 64
int tri_mul_mask_extents(int dtype, const void* pair_mask, int batch, int n, int* extents,
                         void* stream);

/* tri_mul_forward (residual = 0) or tri_mul_forward_residual (residual = 1) with work
 * skipping: the contraction of item b runs over k < L_b only (rounded up to its 32-element
 * stage), and output tiles wholly past L_b run no contraction (their x is zero). The
 * results equal the plain call's exactly when `extents` are tri_mul_mask_extents of this
 * pair_mask: outside the leading L_b x L_b square both operands are zero. The input and
 * output kernels skip the tiles outside that square without reading them, and (as in the
 * plain call) run no MFMA for tiles whose mask is all zero.
 *   extents  as written by tri_mul_mask_extents for (pair_mask, batch, n); read only, may
 *            not overlap out or the workspace (ALIAS); 4-byte aligned.
 * Other arguments, in-place rules and errors as for tri_mul_forward / _residual, except
 * that pair_mask is required; INVALID_ARG also for a NULL pair_mask or extents and for
 * residual outside {0, 1}. With extents, the workspace's a and b are not written outside
 * each item's leading L_b x L_b square. */
int tri_mul_forward_extents(tri_mul_handle* h, const void* z, const void* pair_mask,
                            const int* extents, void* out, int batch, int n, int direction,
                            int residual, void* workspace, size_t workspace_bytes, void* stream);

/* One kernel of the chain, same arguments as tri_mul_forward:
 *   stage 1: input LayerNorm + gated dual projection + mask -> a, b (workspace)
 *   stage 2: contraction over k -> x (workspace)
 *   stage 3: output LayerNorm + projection + output gate + mask -> out
 * Running stages 1, 2, 3 in order equals tri_mul_forward. For inspection of the
 * intermediates and for per-kernel timing. */
int tri_mul_forward_stage(tri_mul_handle* h, int stage, const void* z, const void* pair_mask,
                          void* out, int batch, int n, int direction, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Releases the device weights. NULL is a no-op. Must not race a forward call. */
void tri_mul_destroy(tri_mul_handle* h);

/* Static text for an error code (never NULL). */
const char* tri_mul_strerror(int code);

/* Details of the last TRI_MUL_ERR_HIP on the calling thread (static text). */
const char* tri_mul_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TRI_MUL_H */
