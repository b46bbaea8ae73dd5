"""Pins for the triangular-attention oracle: each check compares it with something other
than itself (pure-Python loops, torch's scaled-dot-product attention in float64, closed
forms of special weights and masks, identities of the mathematics), and planted mistakes
in each of its steps must fail at least one pin. CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_ref as aref
from pair_rep_triangle_amd.inputs import make_attention_weights


def _case(B=1, N=3, c_z=4, heads=2, d=2, seed=0, mask="random"):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, N, N, c_z)) * 1.5 + 0.2
    w = {k: v.astype(np.float64) for k, v in
         make_attention_weights(rng, c_z, heads, d, random_affine=True).items()}
    if mask == "random":
        m = (rng.random((B, N, N)) < 0.7).astype(np.float64)
    elif mask == "rowpad":  # random, with residue 0 fully padded (row and column)
        m = (rng.random((B, N, N)) < 0.7).astype(np.float64)
        m[:, 0, :] = 0.0
        m[:, :, 0] = 0.0
    elif mask == "keyed":  # random, but every row and every column keeps a valid pair
        m = (rng.random((B, N, N)) < 0.6).astype(np.float64)
        idx = np.arange(N)
        m[:, idx, idx] = 1.0
    elif mask == "ones":
        m = np.ones((B, N, N))
    else:
        m = None
    return z, m, w


def _loops(z, m, w, node, eps=1e-5):
    """Triangular attention written out with Python loops and math only."""
    B, N, _, c_z = z.shape
    H = len(w["w_b"])
    d = len(w["w_q"]) // H
    m = np.ones((B, N, N)) if m is None else m

    def norm(x):
        x = [float(t) for t in x]
        mu = sum(x) / len(x)
        var = sum((t - mu) ** 2 for t in x) / len(x)
        return [(x[c] - mu) / math.sqrt(var + eps) * w["ln_gamma"][c] + w["ln_beta"][c]
                for c in range(len(x))]

    def lin(x, W, row):
        return sum(W[row][c] * x[c] for c in range(len(x)))

    out = np.zeros((B, N, N, c_z))
    for b in range(B):
        zh = [[norm(z[b, i, j]) for j in range(N)] for i in range(N)]
        for i in range(N):
            for j in range(N):
                o = []
                for h in range(H):
                    q = [lin(zh[i][j], w["w_q"], h * d + e) for e in range(d)]
                    logits, vals = [], []
                    for k in range(N):
                        kp = (i, k) if node == "starting" else (k, j)
                        if m[b][kp[0]][kp[1]] == 0:
                            continue
                        bp = (j, k) if node == "starting" else (k, i)
                        kk = [lin(zh[kp[0]][kp[1]], w["w_k"], h * d + e) for e in range(d)]
                        s = sum(q[e] * kk[e] for e in range(d)) / math.sqrt(d)
                        s += lin(zh[bp[0]][bp[1]], w["w_b"], h)
                        logits.append(s)
                        vals.append([lin(zh[kp[0]][kp[1]], w["w_v"], h * d + e) for e in range(d)])
                    att = [0.0] * d
                    if logits:
                        top = max(logits)
                        ex = [math.exp(s - top) for s in logits]
                        tot = sum(ex)
                        for a, vv in zip(ex, vals):
                            for e in range(d):
                                att[e] += a / tot * vv[e]
                    for e in range(d):
                        gl = lin(zh[i][j], w["w_g"], h * d + e) + w["b_g"][h * d + e]
                        o.append(att[e] / (1.0 + math.exp(-gl)))
                for c in range(c_z):
                    out[b, i, j, c] = w["b_o"][c] + sum(w["w_o"][c][t] * o[t] for t in range(H * d))
    return out


def _torch_starting(z, m, w):
    """The starting node composed from torch float64 library routines: layer_norm,
    linear, scaled_dot_product_attention with an additive float mask, sigmoid."""
    zt = torch.from_numpy(z)
    B, N, _, c_z = z.shape
    H = len(w["w_b"])
    d = len(w["w_q"]) // H
    T = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in w.items()}
    zh = torch.nn.functional.layer_norm(zt, (c_z,), T["ln_gamma"], T["ln_beta"], eps=1e-5)

    def heads(x):  # [B, N, N, H*d] -> [B, N(i), H, N(j), d]
        return x.reshape(B, N, N, H, d).permute(0, 1, 3, 2, 4)

    q = heads(torch.nn.functional.linear(zh, T["w_q"]))
    k = heads(torch.nn.functional.linear(zh, T["w_k"]))
    v = heads(torch.nn.functional.linear(zh, T["w_v"]))
    bias = torch.nn.functional.linear(zh, T["w_b"]).permute(0, 3, 1, 2)  # [B, H, j, k]
    keymask = torch.where(torch.from_numpy(m) != 0, 0.0, float("-inf")).to(torch.float64)
    attn_mask = bias[:, None, :, :, :] + keymask[:, :, None, None, :]  # [B, i, H, j, k]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=attn_mask)
    g = torch.sigmoid(torch.nn.functional.linear(zh, T["w_g"], T["b_g"]))
    o = o.permute(0, 1, 3, 2, 4).reshape(B, N, N, H * d) * g
    return torch.nn.functional.linear(o, T["w_o"], T["b_o"]).numpy()


# --- pins ---------------------------------------------------------------------------------

LOOP_CASES = [dict(B=1, N=3, c_z=4, heads=2, d=2, seed=0),
              dict(B=2, N=3, c_z=3, heads=1, d=3, seed=1, mask="rowpad"),
              dict(B=1, N=4, c_z=5, heads=2, d=2, seed=2, mask="none"),
              dict(B=1, N=2, c_z=4, heads=3, d=1, seed=3, mask="ones")]


def _pin_loops():
    for kw in LOOP_CASES:
        z, m, w = _case(**kw)
        for node in aref.NODES:
            if not np.allclose(aref.tri_attention_ref(z, m, w, node), _loops(z, m, w, node),
                               rtol=1e-11, atol=1e-11):
                return False
    return True


def _pin_transpose():
    """Ending node = starting node on the transposed pair tensor and mask, transposed back."""
    z, m, w = _case(B=2, N=5, c_z=6, heads=2, d=3, seed=4, mask="rowpad")
    end = aref.tri_attention_ref(z, m, w, "ending")
    start_t = aref.tri_attention_ref(z.transpose(0, 2, 1, 3), m.transpose(0, 2, 1), w, "starting")
    return np.allclose(end, start_t.transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)


def _pin_torch_sdpa():
    z, m, w = _case(B=2, N=6, c_z=8, heads=2, d=4, seed=5, mask="keyed")
    return np.allclose(aref.tri_attention_ref(z, m, w, "starting"), _torch_starting(z, m, w),
                       rtol=1e-10, atol=1e-10)


def _pin_single_key():
    """One valid key pair per row: its attention weight is 1, so o_ij = g_ij * v_ik*."""
    z, _, w = _case(B=1, N=5, c_z=6, heads=2, d=3, seed=6, mask="none")
    N = 5
    kstar = np.random.default_rng(60).integers(0, N, N)
    m = np.zeros((1, N, N))
    m[0, np.arange(N), kstar] = 1.0
    mu = z.mean(-1, keepdims=True)
    zh = (z - mu) / np.sqrt(z.var(-1, keepdims=True) + 1e-5) * w["ln_gamma"] + w["ln_beta"]
    v = zh @ w["w_v"].T
    g = 1.0 / (1.0 + np.exp(-(zh @ w["w_g"].T + w["b_g"])))
    want = (g * v[:, np.arange(N), kstar][:, :, None, :]) @ w["w_o"].T + w["b_o"]
    return np.allclose(aref.tri_attention_ref(z, m, w, "starting"), want, rtol=1e-11, atol=1e-11)


def _pin_uniform():
    """W_q = 0 and w_b = 0: every logit is 0, the output is g times the mean value of the
    valid keys of the row."""
    z, m, w = _case(B=1, N=5, c_z=6, heads=2, d=3, seed=7, mask="rowpad")
    w = dict(w, w_q=np.zeros_like(w["w_q"]), w_b=np.zeros_like(w["w_b"]))
    mu = z.mean(-1, keepdims=True)
    zh = (z - mu) / np.sqrt(z.var(-1, keepdims=True) + 1e-5) * w["ln_gamma"] + w["ln_beta"]
    v = zh @ w["w_v"].T  # [1, i, k, H*d]
    g = 1.0 / (1.0 + np.exp(-(zh @ w["w_g"].T + w["b_g"])))
    cnt = m.sum(-1)[..., None]
    mean = np.divide((m[..., None] * v).sum(2), cnt, out=np.zeros_like(v[:, :, 0]), where=cnt > 0)
    want = (g * mean[:, :, None, :]) @ w["w_o"].T + w["b_o"]
    return np.allclose(aref.tri_attention_ref(z, m, w, "starting"), want, rtol=1e-11, atol=1e-11)


def _pin_crop():
    """With a leading L x L block mask the valid block equals the op on the cropped
    input (padded residues contribute nothing), for both nodes."""
    N, L = 7, 4
    z, _, w = _case(B=1, N=N, c_z=6, heads=2, d=3, seed=8, mask="none")
    m = np.zeros((1, N, N))
    m[:, :L, :L] = 1.0
    for node in aref.NODES:
        full = aref.tri_attention_ref(z, m, w, node)[:, :L, :L]
        crop = aref.tri_attention_ref(z[:, :L, :L], None, w, node)
        if not np.allclose(full, crop, rtol=1e-12, atol=1e-12):
            return False
    return True


def _pin_permutation():
    """Relabelling the residues relabels the output: out(P z P^T) = P out(z) P^T."""
    z, m, w = _case(B=1, N=6, c_z=5, heads=1, d=4, seed=9, mask="random")
    perm = np.random.default_rng(90).permutation(6)
    for node in aref.NODES:
        out = aref.tri_attention_ref(z, m, w, node)
        outp = aref.tri_attention_ref(z[:, perm][:, :, perm], m[:, perm][:, :, perm], w, node)
        if not np.allclose(out[:, perm][:, :, perm], outp, rtol=1e-12, atol=1e-12):
            return False
    return True


def _pin_zero_mask():
    """No valid key anywhere: every attention output is 0 and out is b_o."""
    z, m, w = _case(B=1, N=4, c_z=5, heads=2, d=2, seed=10)
    for node in aref.NODES:
        out = aref.tri_attention_ref(z, np.zeros_like(m), w, node)
        if not np.array_equal(out, np.broadcast_to(w["b_o"], out.shape)):
            return False
    return True


def _pin_linear_output():
    """out is affine in (W_o, b_o): out(W1 + W2, b1 + b2) = out(W1, b1) + out(W2, b2)."""
    z, m, w = _case(B=1, N=4, c_z=5, heads=2, d=2, seed=11)
    rng = np.random.default_rng(110)
    w2 = dict(w, w_o=rng.standard_normal(w["w_o"].shape), b_o=rng.standard_normal(w["b_o"].shape))
    ws = dict(w, w_o=w["w_o"] + w2["w_o"], b_o=w["b_o"] + w2["b_o"])
    for node in aref.NODES:
        a = aref.tri_attention_ref(z, m, w, node) + aref.tri_attention_ref(z, m, w2, node)
        if not np.allclose(aref.tri_attention_ref(z, m, ws, node), a, rtol=1e-11, atol=1e-11):
            return False
    return True


def _pin_gate_half():
    """W_g = 0: b_g = 0 gives g = 1/2 exactly and b_g = 50 gives g = 1 in float64, so the
    first output minus b_o is half the second."""
    z, m, w = _case(B=1, N=4, c_z=5, heads=2, d=2, seed=12)
    w0 = dict(w, w_g=np.zeros_like(w["w_g"]), b_g=np.zeros_like(w["b_g"]))
    w1 = dict(w0, b_g=np.full_like(w["b_g"], 50.0))
    for node in aref.NODES:
        half = aref.tri_attention_ref(z, m, w0, node) - w["b_o"]
        one = aref.tri_attention_ref(z, m, w1, node) - w["b_o"]
        if not np.allclose(2 * half, one, rtol=1e-12, atol=1e-12):
            return False
    return True


PINS = [_pin_loops, _pin_transpose, _pin_torch_sdpa, _pin_single_key, _pin_uniform,
        _pin_crop, _pin_permutation, _pin_zero_mask, _pin_linear_output, _pin_gate_half]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__[5:])
def test_attention_pin(pin):
    assert pin()


# --- planted mistakes: each must fail at least one pin --------------------------------------

def _pins_pass():
    return all(p() for p in PINS)


def _mut_ln_unbiased(x, gamma, beta):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + aref.EPS) * gamma + beta


def _mut_ln_no_centering(x, gamma, beta):
    var = (x ** 2).mean(axis=-1, keepdims=True)
    return x / np.sqrt(var + aref.EPS) * gamma + beta


def _mut_sigmoid_sign(t):
    return 1.0 / (1.0 + np.exp(t))


def _mut_softmax_ignores_mask(s, valid):
    return aref_softmax(s, np.ones_like(valid))


def _mut_softmax_large_negative(s, valid):
    """Masked keys as a large negative logit instead of being left out."""
    s = np.where(valid, s, s - 1e9)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _mut_softmax_unnormalised(s, valid):
    s = np.where(valid, s, -np.inf)
    top = s.max(axis=-1, keepdims=True)
    top = np.where(np.isfinite(top), top, 0.0)
    return np.where(valid, np.exp(s - top), 0.0)


def _mut_heads_interleaved(x, heads):
    return np.swapaxes(x.reshape(x.shape[:-1] + (x.shape[-1] // heads, heads)), -1, -2)


def _attend_mutant(scale=True, bias_t=False, ending_rows=False, query_mask=False):
    """The oracle's attention step written with einsum over whole planes, with one
    optional mistake: no 1/sqrt(d) scale, the pair bias transposed, the ending node
    reading keys from the query's row, or the mask applied to queries instead of keys."""
    def attend(q, k, v, bias, mask, node, chunk):
        B, N, _, H, d = q.shape
        out = np.zeros_like(q)
        sc = 1.0 / np.sqrt(d) if scale else 1.0
        for b in range(B):
            for h in range(H):
                qh, kh, vh, bh = q[b, :, :, h], k[b, :, :, h], v[b, :, :, h], bias[b, h]
                if bias_t:
                    bh = bh.T
                if node == "starting":
                    bterm = bh[None, :, :]           # beta_jk at [i, j, k]
                else:
                    bterm = bh.T[:, None, :]         # beta_ki at [i, j, k]
                if query_mask:
                    valid = np.broadcast_to(mask[b][:, :, None], (N, N, N))   # m_ij
                elif node == "starting" or ending_rows:
                    valid = np.broadcast_to(mask[b][:, None, :], (N, N, N))   # m_ik
                else:
                    valid = np.broadcast_to(mask[b].T[None, :, :], (N, N, N))  # m_kj
                if node == "starting" or ending_rows:
                    s = np.einsum("ijd,ikd->ijk", qh, kh) * sc + bterm
                    p = aref_softmax(s, valid != 0)
                    out[b, :, :, h] = np.einsum("ijk,ikd->ijd", p, vh)
                else:
                    s = np.einsum("ijd,kjd->ijk", qh, kh) * sc + bterm
                    p = aref_softmax(s, valid != 0)
                    out[b, :, :, h] = np.einsum("ijk,kjd->ijd", p, vh)
        return out
    return attend


aref_softmax = aref._masked_softmax

MUTANTS = {
    "ln_unbiased_variance": ("_layer_norm", _mut_ln_unbiased),
    "ln_no_centering": ("_layer_norm", _mut_ln_no_centering),
    "gate_sigmoid_sign": ("_sigmoid", _mut_sigmoid_sign),
    "mask_ignored": ("_masked_softmax", _mut_softmax_ignores_mask),
    "mask_as_large_negative_logit": ("_masked_softmax", _mut_softmax_large_negative),
    "softmax_not_normalised": ("_masked_softmax", _mut_softmax_unnormalised),
    "heads_interleaved": ("_heads", _mut_heads_interleaved),
    "no_logit_scale": ("_attend", _attend_mutant(scale=False)),
    "bias_transposed": ("_attend", _attend_mutant(bias_t=True)),
    "ending_node_uses_rows": ("_attend", _attend_mutant(ending_rows=True)),
    "mask_on_queries": ("_attend", _attend_mutant(query_mask=True)),
}


def test_attention_mutant_of_nothing_matches_the_oracle():
    """The mutant attention with no mistake planted is the oracle's attention (so the
    planted variants differ from it only by their mistake)."""
    z, m, w = _case(B=2, N=5, c_z=6, heads=2, d=3, seed=13, mask="rowpad")
    q, k, v, g, bias = aref._projections(z, w)
    for node in aref.NODES:
        assert np.allclose(_attend_mutant()(q, k, v, bias, m, node, 64),
                           aref._attend(q, k, v, bias, m, node, 64), rtol=1e-12, atol=1e-12)


def test_attention_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_attention_planted_mistake_is_caught(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(aref, name, fn)
    assert not _pins_pass(), f"planted mistake {mutant!r} slipped through the pins"


@pytest.mark.parametrize("node", aref.NODES)
def test_line_restricted_oracle_equals_the_full_evaluation(node):
    """tri_attention_ref_lines (used for sampled parity at large N) returns exactly the
    chosen rows (starting) or columns (ending) of the full output."""
    z, m, w = _case(B=2, N=9, c_z=8, heads=2, d=4, seed=14, mask="rowpad")
    lines = [0, 2, 5, 8]
    full = aref.tri_attention_ref(z, m, w, node)
    sub = aref.tri_attention_ref_lines(z, m, w, node, lines)
    want = full[:, lines] if node == "starting" else np.swapaxes(full[:, :, lines], 1, 2)
    assert np.array_equal(sub, want)
