"""fp64 CPU oracle for the triangle multiplicative update (outgoing and incoming).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain definition that the
HIP path is checked against. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
It shares no code, table or constant generator with the HIP library and it
imports nothing from it; the product path never calls it.

What is computed (per batch item b and residue pair (i, j); every step in
float64 NumPy):

1. Input LayerNorm over the c_z channels of z_bij, biased variance, eps = 1e-5,
   with affine gamma_in / beta_in.
   [RFProteína architecture page, "Triangle multiplication on SM90": K1 applies
   the input projection after the input LayerNorm; "Dual-GEMM gates": both
   input-gate projections read the normalized pair tensor.]
2. Gated dual projection, one weight set per operand:
   a = m_bij * sigmoid(zhat W_ag^T + b_ag) * (zhat W_ap^T + b_ap), same for b
   with the W_b* set.  [RFProteína architecture, "Dual-GEMM gates", the x_x
   form sigma(x W_g^T + b_g) * (x W_p^T + b_p); the input gate consumes the pair
   mask, "absorbing masking".]
3. Contraction over the third residue k (a plain sum, no normalisation):
   outgoing  x_bij = sum_k a_bik * b_bjk
   incoming  x_bij = sum_k a_bki * b_bkj
   [RFProteína architecture, "Inside the velocity network": a pair update runs
   outgoing then incoming triangle multiplication; yage.ai summary of the
   biomolecular-software report: every pair is checked against every third
   residue, cubic cost. The pages name the two directions but print no index
   pattern; the reading above is the one used throughout: outgoing pairs the
   edges leaving i and j, incoming the edges arriving at i and j.]
4. Output LayerNorm over the c channels of x_bij (gamma_out / beta_out).
   [RFProteína architecture, "Triangle multiplication on SM90": K3 carries the
   second LayerNorm.]
5. p = xhat W_o^T + b_o;  g = sigmoid(zhat W_g^T + b_g), zhat from step 1.
   [RFProteína architecture, "Dual-GEMM gates", the x0_x1 form: x0 is the
   normalized input pair tensor, x1 the contracted hidden tensor.]
6. out_bij = m_bij * g * p  (reading: padded pairs are defined as 0; the
   residual add is a separate op, the "Masked residual" row of the kernel
   table on the RFProteína architecture page).

Weights are the fp32 host arrays in nn.Linear orientation ([out][in]).
``mask`` None means all ones.

Parity pins (in the test suite, none of them reuses this code): brute-force
pure-Python loops on tiny inputs, an independent composition of torch library
routines (layer_norm / linear / sigmoid / einsum) in float64, the transpose
identity incoming(z, m; W_a, W_b) = outgoing(z^T, m^T; W_b, W_a)^T, the crop
invariant for padded residues, constant-z and N=1 closed forms, permutation
equivariance, and a planted-mistake check that each pin is sharp.
"""

import numpy as np

EPS = 1e-5  # LayerNorm epsilon for both norms (PyTorch LayerNorm default)

WEIGHT_FIELDS = (
    "ln_in_gamma", "ln_in_beta",
    "w_a_gate", "b_a_gate", "w_a_proj", "b_a_proj",
    "w_b_gate", "b_b_gate", "w_b_proj", "b_b_proj",
    "ln_out_gamma", "ln_out_beta",
    "w_out", "b_out",
    "w_gate", "b_gate",
)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def layer_norm(x, gamma, beta, eps=EPS):
    """LayerNorm over the last axis: biased variance, eps inside the root."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def sigmoid(t):
    return 1.0 / (1.0 + np.exp(-_f64(t)))


def linear(x, w, b):
    """nn.Linear orientation: x [..., in], w [out, in], b [out]."""
    return _f64(x) @ _f64(w).T + _f64(b)


def gated_projection(zhat, w_gate, b_gate, w_proj, b_proj):
    """sigmoid(zhat W_g^T + b_g) * (zhat W_p^T + b_p)."""
    return sigmoid(linear(zhat, w_gate, b_gate)) * linear(zhat, w_proj, b_proj)


def input_operands(z, mask, w, eps=EPS):
    """Steps 1-2: zhat, a and b for every pair. Shapes [..., c_z] / [..., c]."""
    zhat = layer_norm(z, w["ln_in_gamma"], w["ln_in_beta"], eps)
    m = _f64(mask)[..., None]
    a = m * gated_projection(zhat, w["w_a_gate"], w["b_a_gate"], w["w_a_proj"], w["b_a_proj"])
    b = m * gated_projection(zhat, w["w_b_gate"], w["b_b_gate"], w["w_b_proj"], w["b_b_proj"])
    return zhat, a, b


def contract(a, b, direction):
    """Step 3 on [B, N, N, c] operands, one matmul per (batch, channel)."""
    # channel-major copies so that every per-channel product is a BLAS matmul
    A = np.ascontiguousarray(np.moveaxis(_f64(a), -1, 1))  # [B, c, N, N]
    Bm = np.ascontiguousarray(np.moveaxis(_f64(b), -1, 1))
    if direction == "outgoing":
        X = np.matmul(A, np.swapaxes(Bm, -1, -2))  # x_ij = sum_k a_ik b_jk
    elif direction == "incoming":
        X = np.matmul(np.swapaxes(A, -1, -2), Bm)  # x_ij = sum_k a_ki b_kj
    else:
        raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
    return np.moveaxis(X, 1, -1)  # [B, N, N, c]


def output_stage(x, zhat, mask, w, eps=EPS):
    """Steps 4-6 on matching [..., c] / [..., c_z] pair tensors."""
    xhat = layer_norm(x, w["ln_out_gamma"], w["ln_out_beta"], eps)
    p = linear(xhat, w["w_out"], w["b_out"])
    g = sigmoid(linear(zhat, w["w_gate"], w["b_gate"]))
    return _f64(mask)[..., None] * g * p


def _prep(z, mask, weights):
    z = _f64(z)
    if z.ndim != 4:
        raise ValueError("z must be [B, N, N, c_z]")
    B, N, N2, _ = z.shape
    if N != N2:
        raise ValueError("z must be square in its two residue axes")
    mask = np.ones((B, N, N)) if mask is None else _f64(mask)
    if mask.shape != (B, N, N):
        raise ValueError("mask must be [B, N, N]")
    w = {k: _f64(weights[k]) for k in WEIGHT_FIELDS}
    return z, mask, w


def tri_mul_intermediates(z, mask, weights, direction, eps=EPS):
    """Full op returning every intermediate (zhat, a, b, x, out), all float64."""
    z, mask, w = _prep(z, mask, weights)
    zhat, a, b = input_operands(z, mask, w, eps)
    x = contract(a, b, direction)
    out = output_stage(x, zhat, mask, w, eps)
    return {"zhat": zhat, "a": a, "b": b, "x": x, "out": out}


def tri_mul_ref(z, mask, weights, direction, eps=EPS):
    """The triangle multiplicative update. z [B,N,N,c_z] -> out [B,N,N,c_z] float64."""
    return tri_mul_intermediates(z, mask, weights, direction, eps)["out"]


def tri_mul_ref_pairs(z, mask, weights, direction, bidx, iidx, jidx, eps=EPS):
    """The same op evaluated only at the listed pairs (b, i, j).

    For large N: each output needs the operand row/column of its two residues
    only (2N pairs through steps 1-2), so memory stays O(N c_z) per sample.
    Returns [S, c_z] float64.
    """
    z = np.asarray(z)
    B, N = z.shape[0], z.shape[1]
    w = {k: _f64(weights[k]) for k in WEIGHT_FIELDS}
    bidx, iidx, jidx = (np.asarray(v, dtype=np.int64).ravel() for v in (bidx, iidx, jidx))
    out = np.empty((bidx.size, z.shape[-1]))
    for s, (bb, i, j) in enumerate(zip(bidx, iidx, jidx)):
        mrow = np.ones(N) if mask is None else None
        if direction == "outgoing":
            # a over pairs (i, k), b over pairs (j, k)
            za, zb = z[bb, i, :, :], z[bb, j, :, :]
            ma = mrow if mask is None else np.asarray(mask)[bb, i, :]
            mb = mrow if mask is None else np.asarray(mask)[bb, j, :]
        elif direction == "incoming":
            # a over pairs (k, i), b over pairs (k, j)
            za, zb = z[bb, :, i, :], z[bb, :, j, :]
            ma = mrow if mask is None else np.asarray(mask)[bb, :, i]
            mb = mrow if mask is None else np.asarray(mask)[bb, :, j]
        else:
            raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
        _, a_rows, _ = input_operands(za, ma, w, eps)
        _, _, b_rows = input_operands(zb, mb, w, eps)
        x = (a_rows * b_rows).sum(axis=0)  # sum over the third residue k
        zhat_ij = layer_norm(z[bb, i, j, :], w["ln_in_gamma"], w["ln_in_beta"], eps)
        mij = 1.0 if mask is None else float(np.asarray(mask)[bb, i, j])
        out[s] = output_stage(x, zhat_ij, np.float64(mij), w, eps)
    return out


def line_operands(z, mask, weights, bidx, eps=EPS, chunk=8, workers=None):
    """Steps 1-2 for every pair of batch item `bidx`, channel-major: (a, b) as [c, N, N]
    float64 with a[ch, i, k] = a_{bidx, i, k, ch} (same for b). Both operands are needed in
    full for complete output lines: row i of x pairs one row of a with every row of b,
    column j every row of a with one row of b.

    Pairs are independent in these steps, so blocks of `chunk` residue rows are evaluated
    on `workers` threads (NumPy releases the interpreter lock inside its array loops); each
    block is the same arithmetic as `input_operands` on those rows."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    z = np.asarray(z)
    N = z.shape[1]
    w = {k: _f64(weights[k]) for k in WEIGHT_FIELDS}
    c = w["w_a_gate"].shape[0]
    m_b = np.ones((N, N)) if mask is None else _f64(np.asarray(mask)[bidx])
    a = np.empty((c, N, N))
    b = np.empty((c, N, N))

    def block(r0):
        r1 = min(N, r0 + chunk)
        _, a_rows, b_rows = input_operands(_f64(z[bidx, r0:r1]), m_b[r0:r1], w, eps)
        a[:, r0:r1, :] = np.moveaxis(a_rows, -1, 0)
        b[:, r0:r1, :] = np.moveaxis(b_rows, -1, 0)

    workers = workers or min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(block, range(0, N, chunk)))
    return a, b


def tri_mul_ref_lines(z, mask, weights, direction, bidx, rows, cols, eps=EPS, operands=None):
    """Complete output lines of batch item `bidx`: out[bidx, rows, :, :] as [R, N, c_z] and
    out[bidx, :, cols, :] as [N, C, c_z], float64.

    Steps 1-2 run over every pair of the batch item (`line_operands`; pass its result as
    `operands` to reuse it for the other direction), steps 3-6 only on the listed lines.
    For incoming, x_ij = sum_k a_ki b_kj is the outgoing pattern on the transposed
    operand planes.
    """
    z = np.asarray(z)
    N = z.shape[1]
    w = {k: _f64(weights[k]) for k in WEIGHT_FIELDS}
    rows = np.asarray(rows, dtype=np.int64).ravel()
    cols = np.asarray(cols, dtype=np.int64).ravel()
    a, b = operands if operands is not None else line_operands(z, mask, weights, bidx, eps)
    if direction == "incoming":
        a, b = np.swapaxes(a, 1, 2), np.swapaxes(b, 1, 2)
    elif direction != "outgoing":
        raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
    # x[ch, i, j] = sum_k a[ch, i, k] * b[ch, j, k], on the listed rows and columns
    x_rows = np.matmul(a[:, rows, :], np.swapaxes(b, 1, 2))          # [c, R, N]
    x_cols = np.matmul(a, np.swapaxes(b[:, cols, :], 1, 2))          # [c, N, C]
    m_b = np.ones((N, N)) if mask is None else _f64(np.asarray(mask)[bidx])
    zr, zc = _f64(z[bidx, rows]), _f64(z[bidx][:, cols])
    out_rows = output_stage(np.moveaxis(x_rows, 0, -1),
                            layer_norm(zr, w["ln_in_gamma"], w["ln_in_beta"], eps),
                            m_b[rows], w, eps)
    out_cols = output_stage(np.moveaxis(x_cols, 0, -1),
                            layer_norm(zc, w["ln_in_gamma"], w["ln_in_beta"], eps),
                            m_b[:, cols], w, eps)
    return out_rows, out_cols


def tri_mul_residual_ref(z, mask, weights, direction, eps=EPS):
    """z + out: the update followed by the masked residual add of the pair update
    [RFProteína architecture page, kernel table: a "masked residual" kernel follows each
    pair operation; out already carries the mask (reading R7), so padded pairs keep z]."""
    return _f64(z) + tri_mul_ref(z, mask, weights, direction, eps)


def pair_update_ref(z, mask, w_outgoing, w_incoming, eps=EPS):
    """The two triangle multiplicative updates of one pair-update step in model order:
    outgoing on z, then incoming on the result, each with its residual add
    [RFProteína architecture, "Inside the velocity network": the pair update runs the
    outgoing, then the incoming triangle multiplication]."""
    z1 = tri_mul_residual_ref(z, mask, w_outgoing, "outgoing", eps)
    return tri_mul_residual_ref(z1, mask, w_incoming, "incoming", eps)
