"""Pins for the pair-transition oracle: each test checks it against something other than
itself (pure-Python loops, closed forms of special weights, identities of the
mathematics), and planted mistakes in each of its steps must fail at least one pin.
CPU only."""

import math

import numpy as np
import pytest

from oracle import transition_ref as tref
from pair_rep_triangle_amd.inputs import make_transition_weights


def _case(B=1, N=3, c_z=4, hidden=8, seed=0, affine=True, mask="random"):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, N, N, c_z)) * 1.7 + 0.3
    w = {k: v.astype(np.float64) for k, v in
         make_transition_weights(rng, c_z, hidden, random_affine=affine).items()}
    if mask == "random":
        m = (rng.random((B, N, N)) < 0.7).astype(np.float64)
    elif mask == "ones":
        m = np.ones((B, N, N))
    else:
        m = None
    return z, m, w


def _loops(z, m, w, eps=1e-5):
    """The transition written out with Python loops and math only."""
    B, N, _, c_z = z.shape
    hidden = len(w["b1"])
    out = [[[[0.0] * c_z for _ in range(N)] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for i in range(N):
            for j in range(N):
                x = [float(v) for v in z[b, i, j]]
                mean = sum(x) / c_z
                var = sum((v - mean) ** 2 for v in x) / c_z
                xh = [(x[k] - mean) / math.sqrt(var + eps) * w["ln_gamma"][k] + w["ln_beta"][k]
                      for k in range(c_z)]
                h = []
                for o in range(hidden):
                    s = w["b1"][o]
                    for k in range(c_z):
                        s += w["w1"][o][k] * xh[k]
                    h.append(s if s > 0 else 0.0)
                mm = 1.0 if m is None else float(m[b, i, j])
                for o in range(c_z):
                    s = w["b2"][o]
                    for k in range(hidden):
                        s += w["w2"][o][k] * h[k]
                    out[b][i][j][o] = x[o] + mm * s
    return np.array(out)


# --- pins ---------------------------------------------------------------------------------

CASES = [dict(B=1, N=2, c_z=4, hidden=8, seed=0), dict(B=2, N=3, c_z=3, hidden=6, seed=1),
         dict(B=1, N=3, c_z=5, hidden=10, seed=2, mask="none"),
         dict(B=1, N=2, c_z=6, hidden=4, seed=3, mask="ones")]


def _pin_loops():
    for kw in CASES:
        z, m, w = _case(**kw)
        if not np.allclose(tref.pair_transition_ref(z, m, w), _loops(z, m, w), rtol=1e-11, atol=1e-11):
            return False
    return True


def _pin_zero_second_layer():
    """W_2 = 0 and b_2 = 0: the update vanishes and out is z, exactly."""
    z, m, w = _case(seed=4)
    w = dict(w, w2=np.zeros_like(w["w2"]), b2=np.zeros_like(w["b2"]))
    return np.array_equal(tref.pair_transition_ref(z, m, w), z)


def _pin_zero_mask():
    z, m, w = _case(seed=5)
    return np.array_equal(tref.pair_transition_ref(z, np.zeros_like(m), w), z)


def _pin_active_region():
    """b_1 large: every hidden unit is active, so the transition is affine in zhat with
    the composed matrix W_2 W_1 and offset W_2 b_1 + b_2."""
    z, m, w = _case(seed=6, c_z=5, hidden=7)
    w = dict(w, b1=np.full_like(w["b1"], 1e3))
    mu = z.mean(-1, keepdims=True)
    sd = np.sqrt(z.var(-1, keepdims=True) + 1e-5)
    zhat = (z - mu) / sd * w["ln_gamma"] + w["ln_beta"]
    comp = w["w2"] @ w["w1"]
    want = z + m[..., None] * (np.einsum("bijk,ok->bijo", zhat, comp) + w["w2"] @ w["b1"] + w["b2"])
    return np.allclose(tref.pair_transition_ref(z, m, w), want, rtol=1e-9, atol=1e-9)


def _pin_inactive_region():
    """b_1 very negative: no hidden unit is active and the update is m * b_2."""
    z, m, w = _case(seed=7)
    w = dict(w, b1=np.full_like(w["b1"], -1e3))
    want = z + m[..., None] * w["b2"]
    return np.allclose(tref.pair_transition_ref(z, m, w), want, rtol=0, atol=1e-12)


def _pin_layernorm_invariance():
    """A per-pair positive scale and shift of z leaves zhat, hence the update, unchanged
    (up to the epsilon under the square root: |d zhat| <= eps / (2 var) relative, below
    1e-5 here; the bar 1e-4 is far under what a missing centring or scale would move)."""
    z, m, w = _case(seed=8, c_z=6, hidden=12)
    rng = np.random.default_rng(80)
    a = rng.uniform(0.5, 3.0, z.shape[:-1] + (1,))
    c = rng.standard_normal(z.shape[:-1] + (1,))
    u1 = tref.pair_transition_ref(z, m, w) - z
    z2 = a * z + c
    u2 = tref.pair_transition_ref(z2, m, w) - z2
    return np.allclose(u1, u2, rtol=1e-4, atol=1e-4)


def _pin_pair_permutation():
    """A pointwise map over pairs: permuting the pairs permutes the outputs."""
    z, m, w = _case(B=1, N=4, seed=9)
    perm = np.random.default_rng(90).permutation(16)
    zf, mf = z.reshape(1, 1, 16, -1), m.reshape(1, 1, 16)
    out = tref.pair_transition_ref(zf, mf, w)
    outp = tref.pair_transition_ref(zf[:, :, perm], mf[:, :, perm], w)
    return np.allclose(out[:, :, perm], outp, rtol=0, atol=1e-12)


PINS = [_pin_loops, _pin_zero_second_layer, _pin_zero_mask, _pin_active_region,
        _pin_inactive_region, _pin_layernorm_invariance, _pin_pair_permutation]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__[5:])
def test_transition_pin(pin):
    assert pin()


def test_update_is_output_minus_z():
    z, m, w = _case(seed=10)
    assert np.allclose(tref.pair_transition_update(z, m, w), tref.pair_transition_ref(z, m, w) - z)


# --- planted mistakes: each must fail at least one pin --------------------------------------

def _pins_pass():
    return all(p() for p in PINS)


def _mut_ln_no_centering(x, gamma, beta):
    var = (x ** 2).mean(axis=-1, keepdims=True)
    return x / np.sqrt(var + tref.EPS) * gamma + beta


def _mut_ln_unbiased(x, gamma, beta):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + tref.EPS) * gamma + beta


def _mut_ln_no_affine(x, gamma, beta):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + tref.EPS)


def _mut_no_relu(zhat, w1, b1):
    return zhat @ w1.T + b1


def _mut_abs_not_relu(zhat, w1, b1):
    return np.abs(zhat @ w1.T + b1)


def _mut_first_no_bias(zhat, w1, b1):
    return np.maximum(zhat @ w1.T, 0.0)


def _mut_relu_before_bias(zhat, w1, b1):
    return np.maximum(zhat @ w1.T, 0.0) + b1


def _mut_second_no_bias(h, w2, b2):
    return h @ w2.T


def _mut_second_relu(h, w2, b2):
    return np.maximum(h @ w2.T + b2, 0.0)


def _mut_no_mask(z, u, mask):
    return z + u


def _mut_no_residual(z, u, mask):
    return u if mask is None else u * np.asarray(mask, np.float64)[..., None]


def _mut_mask_on_everything(z, u, mask):
    out = z + u
    return out if mask is None else out * np.asarray(mask, np.float64)[..., None]


MUTANTS = {
    "ln_no_centering": ("_layer_norm", _mut_ln_no_centering),
    "ln_unbiased_variance": ("_layer_norm", _mut_ln_unbiased),
    "ln_no_affine": ("_layer_norm", _mut_ln_no_affine),
    "no_relu": ("_first_layer", _mut_no_relu),
    "abs_not_relu": ("_first_layer", _mut_abs_not_relu),
    "first_layer_no_bias": ("_first_layer", _mut_first_no_bias),
    "relu_before_bias": ("_first_layer", _mut_relu_before_bias),
    "second_layer_no_bias": ("_second_layer", _mut_second_no_bias),
    "second_layer_relu": ("_second_layer", _mut_second_relu),
    "mask_not_applied": ("_masked_residual", _mut_no_mask),
    "no_residual": ("_masked_residual", _mut_no_residual),
    "mask_on_z_too": ("_masked_residual", _mut_mask_on_everything),
}


def test_transition_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_transition_planted_mistake_is_caught(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(tref, name, fn)
    assert not _pins_pass(), f"planted mistake {mutant!r} slipped through the pins"
