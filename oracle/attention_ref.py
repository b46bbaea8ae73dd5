"""fp64 CPU oracle for triangular attention around the starting and the ending node.

TEST INFRASTRUCTURE ONLY. The slow, plain definition the HIP triangular-attention
kernels are checked against. Only the test suite and the ``cpu_baseline`` leg of
``bench.py`` may import it; it shares no code, table or constant generator with the HIP
library and imports nothing from it.

Sources: the yage.ai summary of the biomolecular-software report names triangular
attention, with the triangular multiplicative update, as the pairwise operations whose
cost grows with the cube of the residue count, and reports a fused kernel for it; the
OpenFold-TRT summary lists triangular attention among the accelerated pair kernels. The
pages print no equations for it. The reading below is the plainest one those passages
support: attention over the third residue k, one softmax per pair (i, j) and head, with
a per-head bias from the pair that closes the triangle.

What is computed, per batch item b (H heads of width d; every step in float64 NumPy):

1. zhat = LayerNorm over the c_z channels (biased variance, eps = 1e-5, gamma / beta).
2. Per head h: q = zhat W_q[h]^T, k = zhat W_k[h]^T, v = zhat W_v[h]^T (d channels each,
   no bias); the pair bias beta_h = zhat . w_b[h] (one value per pair and head, no
   bias); the gate g = sigmoid(zhat W_g[h]^T + b_g[h]). Rows h*d .. h*d + d - 1 of the
   stacked [H*d][c_z] matrices belong to head h.
3. Starting node (the edges leaving i): query pair (i, j) attends over the pairs (i, k)
   of its row:  s_ijk = q_ij . k_ik / sqrt(d) + beta_jk.
   Ending node (the edges arriving at j): query pair (i, j) attends over the pairs
   (k, j) of its column:  s_ijk = q_ij . k_kj / sqrt(d) + beta_ki.
4. Mask: a key pair with mask 0 is left out of the softmax over k (its weight is exactly
   0); a query whose row (starting) or column (ending) holds no valid key pair has a
   zero attention output. [Reading: the pages ask only that padded residues contribute
   nothing; leaving keys out, rather than adding a large negative number to their
   logits, makes that exact and keeps all-padded rows well defined.]
5. o_ij = g_ij * sum_k softmax_k(s_ijk) v_key(k)  per head; out_ij = concat_h(o_ij) W_o^T
   + b_o. The output is not masked and carries no residual (the residual add is a
   separate step of the pair update).

Weights: fp32 host arrays, nn.Linear orientation ([out][in]); names in ATTENTION_FIELDS.

Parity pins (tests/test_attention_pins.py; none reuses this code): pure-Python loops on
tiny inputs (with an all-padded row), the ending node against the starting node on the
transposed pair tensor, torch's scaled-dot-product attention in float64, one valid key,
uniform attention, crop invariance under a block mask, pair permutation, an all-zero
mask, and linearity in (W_o, b_o).
"""

import numpy as np

EPS = 1e-5

ATTENTION_FIELDS = ("ln_gamma", "ln_beta", "w_q", "w_k", "w_v", "w_b", "w_g", "b_g",
                    "w_o", "b_o")
NODES = ("starting", "ending")


def attention_shapes(c_z, heads, d):
    hd = heads * d
    return {"ln_gamma": (c_z,), "ln_beta": (c_z,), "w_q": (hd, c_z), "w_k": (hd, c_z),
            "w_v": (hd, c_z), "w_b": (heads, c_z), "w_g": (hd, c_z), "b_g": (hd,),
            "w_o": (c_z, hd), "b_o": (c_z,)}


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _layer_norm(x, gamma, beta):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + EPS) * gamma + beta


def _sigmoid(t):
    return 1.0 / (1.0 + np.exp(-t))


def _heads(x, heads):
    """[..., H*d] -> [..., H, d] (head h = channels h*d .. h*d + d - 1)."""
    return x.reshape(x.shape[:-1] + (heads, x.shape[-1] // heads))


def _projections(z, w):
    """zhat, then per head q, k, v, g as [B, N, N, H, d] and the bias as [B, H, N, N]."""
    heads = _f64(w["w_b"]).shape[0]
    zhat = _layer_norm(_f64(z), _f64(w["ln_gamma"]), _f64(w["ln_beta"]))
    q = _heads(zhat @ _f64(w["w_q"]).T, heads)
    k = _heads(zhat @ _f64(w["w_k"]).T, heads)
    v = _heads(zhat @ _f64(w["w_v"]).T, heads)
    g = _heads(_sigmoid(zhat @ _f64(w["w_g"]).T + _f64(w["b_g"])), heads)
    bias = np.moveaxis(zhat @ _f64(w["w_b"]).T, -1, 1)  # [B, H, N(first), N(second)]
    return q, k, v, g, bias


def _masked_softmax(s, valid):
    """Softmax over the last axis with invalid entries left out; all-invalid -> zeros."""
    s = np.where(valid, s, -np.inf)
    top = s.max(axis=-1, keepdims=True)
    top = np.where(np.isfinite(top), top, 0.0)
    e = np.where(valid, np.exp(s - top), 0.0)
    tot = e.sum(axis=-1, keepdims=True)
    return np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)


def _attend(q, k, v, bias, mask, node, chunk):
    """Attention output per head, [B, N, N, H, d], before the gate. Around the starting
    node q, k, v and mask may hold a subset of the rows (the bias stays whole)."""
    B, N, _, H, d = q.shape
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, bh = q[b, :, :, h], k[b, :, :, h], v[b, :, :, h], bias[b, h]
            if node == "starting":
                # row i: queries (i, j), keys / values (i, k), bias beta_jk, key mask m_ik
                for i0 in range(0, N, chunk):
                    i1 = min(N, i0 + chunk)
                    s = np.matmul(qh[i0:i1], np.swapaxes(kh[i0:i1], 1, 2)) * scale
                    s = s + bh[None, :, :]
                    valid = (mask[b, i0:i1, None, :] != 0)
                    p = _masked_softmax(s, np.broadcast_to(valid, s.shape))
                    out[b, i0:i1, :, h] = np.matmul(p, vh[i0:i1])
            else:
                # column j: queries (i, j), keys / values (k, j), bias beta_ki, key mask m_kj
                qc = np.swapaxes(qh, 0, 1)  # [j][i][d]
                kc = np.swapaxes(kh, 0, 1)  # [j][k][d]
                vc = np.swapaxes(vh, 0, 1)
                for j0 in range(0, N, chunk):
                    j1 = min(N, j0 + chunk)
                    s = np.matmul(qc[j0:j1], np.swapaxes(kc[j0:j1], 1, 2)) * scale  # [j][i][k]
                    s = s + bh.T[None, :, :]  # beta_ki at [i][k]
                    valid = (mask[b, :, j0:j1].T[:, None, :] != 0)  # m_kj at [j][., k]
                    p = _masked_softmax(s, np.broadcast_to(valid, s.shape))
                    out[b, :, j0:j1, h] = np.swapaxes(np.matmul(p, vc[j0:j1]), 0, 1)
    return out


def tri_attention_ref(z, mask, w, node, chunk=64):
    """out [B, N, N, c_z] of triangular attention around the starting or ending node.
    z [B, N, N, c_z]; mask [B, N, N] (None = all ones); w: ATTENTION_FIELDS arrays."""
    if node not in NODES:
        raise ValueError(f"node must be one of {NODES}")
    z = _f64(z)
    B, N = z.shape[0], z.shape[1]
    mask = np.ones((B, N, N)) if mask is None else _f64(mask)
    q, k, v, g, bias = _projections(z, w)
    o = g * _attend(q, k, v, bias, mask, node, chunk)
    return o.reshape(B, N, N, -1) @ _f64(w["w_o"]).T + _f64(w["b_o"])


def tri_attention_ref_lines(z, mask, w, node, lines, chunk=64):
    """The output restricted to some query lines: rows i (starting node) or columns j
    (ending node) in `lines`; returns [B, len(lines), N, c_z] with [b, t, u] the pair
    (lines[t], u) around the starting node and (u, lines[t]) around the ending node.
    Each line only needs its own queries, keys and values plus the pair bias, so this is
    the same computation as tri_attention_ref on fewer lines."""
    if node not in NODES:
        raise ValueError(f"node must be one of {NODES}")
    z = _f64(z)
    B, N = z.shape[0], z.shape[1]
    mask = np.ones((B, N, N)) if mask is None else _f64(mask)
    lines = np.asarray(lines)
    q, k, v, g, bias = _projections(z, w)
    if node == "ending":  # the ending node is the starting node on the transposed grid
        q, k, v, g = (np.swapaxes(t, 1, 2) for t in (q, k, v, g))
        bias = np.swapaxes(bias, 2, 3)
        mask = np.swapaxes(mask, 1, 2)
    sel = _attend(q[:, lines], k[:, lines], v[:, lines], bias, mask[:, lines], "starting", chunk)
    o = g[:, lines] * sel
    return o.reshape(B, len(lines), N, -1) @ _f64(w["w_o"]).T + _f64(w["b_o"])
