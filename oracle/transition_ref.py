"""fp64 CPU oracle for the pair transition applied as a masked residual.

TEST INFRASTRUCTURE ONLY. The slow, plain definition the HIP pair-transition kernel
is checked against. Only the test suite and the ``cpu_baseline`` leg of ``bench.py``
may import it; it shares no code, table or constant generator with the HIP library
and imports nothing from it.

What is computed (per batch item b and residue pair (i, j); float64 NumPy):

1. LayerNorm over the c_z channels of z_bij, biased variance, eps = 1e-5, affine
   gamma / beta.  [Reading: the RFProteína architecture page's kernel table lists the
   pair transition as "both linears, ReLU, mask, residual" and runs norms as their own
   kernels at every site; the transition is taken to act on the normalised pair
   tensor, the usual pre-norm form, and the HIP kernel fuses that norm.]
2. h = relu(zhat W_1^T + b_1), hidden width = expansion x c_z.  [RFProteína
   architecture, "Kernel support", the pair-transition paragraph of "Dispatch and
   fallback": both linears and the ReLU in one launch, the hidden activation kept
   on chip; the released pair width 384 uses an expansion of 2.]
3. u = h W_2^T + b_2 (back to c_z channels).
4. out_bij = z_bij + m_bij * u_bij.  [RFProteína architecture, "Inside the velocity
   network": the pair transition is applied as a masked residual, like the two
   triangle multiplications before it.]

Weights are fp32 host arrays in nn.Linear orientation ([out][in]); ``mask`` None means
all ones.

Parity pins (tests/test_transition_pins.py, none of them reuses this code): pure-Python
loops on tiny inputs, zero second layer (out = z exactly), zero mask, the all-active
ReLU region against the composed matrix W_2 W_1, the all-inactive region (update =
b_2), LayerNorm invariance to a per-pair affine change of z, and pair permutation.
"""

import numpy as np

EPS = 1e-5

TRANSITION_FIELDS = ("ln_gamma", "ln_beta", "w1", "b1", "w2", "b2")


def transition_shapes(c_z, hidden):
    return {"ln_gamma": (c_z,), "ln_beta": (c_z,), "w1": (hidden, c_z), "b1": (hidden,),
            "w2": (c_z, hidden), "b2": (c_z,)}


def _layer_norm(x, gamma, beta):
    """Step 1: per-pair LayerNorm over the last axis (biased variance)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + EPS) * gamma + beta


def _first_layer(zhat, w1, b1):
    """Step 2: h = relu(zhat W_1^T + b_1)."""
    return np.maximum(zhat @ w1.T + b1, 0.0)


def _second_layer(h, w2, b2):
    """Step 3: u = h W_2^T + b_2."""
    return h @ w2.T + b2


def _masked_residual(z, u, mask):
    """Step 4: z + m * u (m = 1 everywhere when mask is None)."""
    if mask is not None:
        u = u * np.asarray(mask, np.float64)[..., None]
    return z + u


def pair_transition_ref(z, mask, w):
    """z + m * (W_2 relu(W_1 LN(z) + b_1) + b_2), float64 [B][N][N][c_z]."""
    zf = np.asarray(z, dtype=np.float64)
    f64 = {k: np.asarray(v, np.float64) for k, v in w.items()}
    zhat = _layer_norm(zf, f64["ln_gamma"], f64["ln_beta"])
    h = _first_layer(zhat, f64["w1"], f64["b1"])
    u = _second_layer(h, f64["w2"], f64["b2"])
    return _masked_residual(zf, u, mask)


def pair_transition_update(z, mask, w):
    """The update alone: pair_transition_ref(z, mask, w) - z."""
    return pair_transition_ref(z, mask, w) - np.asarray(z, dtype=np.float64)
