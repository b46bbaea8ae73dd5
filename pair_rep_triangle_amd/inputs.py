"""Seeded synthetic inputs for the triangle multiplicative update.

This module draws random numbers and nothing else: it holds none of the
operator's arithmetic, so both the HIP path and the CPU oracle can consume
the same arrays.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this
order): the valid length L when the workload has a padded block mask, then
z ~ N(0, 1) as float32 [B, N, N, c_z], then the weights in the C struct's
field order. Weight matrices are N(0, 1/fan_in) (std 1/sqrt(fan_in)), biases 0,
LayerNorm gamma 1 and beta 0. ``random_affine=True`` also draws non-trivial
biases, gammas and betas (used by the tests so that every term is exercised).

The first five workloads mirror the pair shapes the pages discuss: AlphaFold2/
OpenFold pair width 128 (OpenFold-TRT summary, fixed pair dimension), the
generative design trunk's 384-wide pair track (RFProteína architecture,
"Inside the velocity network"), and residue counts from short targets up to
a large complex. A sixth, a batch of two items with valid lengths 300 and 512
padded to one side (the RFProteína page's parity runs include a padded
two-example batch, "Measured results"), exercises the mask-extent skipping.
"""

import numpy as np

# field order of the weights struct; matrices are [out][in] (nn.Linear)
WEIGHT_FIELDS = (
    "ln_in_gamma", "ln_in_beta",
    "w_a_gate", "b_a_gate", "w_a_proj", "b_a_proj",
    "w_b_gate", "b_b_gate", "w_b_proj", "b_b_proj",
    "ln_out_gamma", "ln_out_beta",
    "w_out", "b_out",
    "w_gate", "b_gate",
)

WORKLOADS = {
    # name: dtype, batch, residues, pair width c_z, hidden width c, mask kind
    "n32_cz16_c16_fp32": dict(dtype="fp32", batch=1, n=32, c_z=16, c=16, mask="ones"),
    "n256_cz128_c128_bf16": dict(dtype="bf16", batch=1, n=256, c_z=128, c=128, mask="ones"),
    "n512_cz128_c128_bf16_masked": dict(dtype="bf16", batch=1, n=512, c_z=128, c=128,
                                        mask="block", l_range=(384, 512)),
    "n768_cz384_c128_b2_bf16": dict(dtype="bf16", batch=2, n=768, c_z=384, c=128, mask="ones"),
    "n2048_cz128_c128_bf16_chains": dict(dtype="bf16", batch=1, n=2048, c_z=128, c=128,
                                         mask="chains", chains=(900, 700, 448)),
    # two items of different valid lengths padded to one side (a padded batch): the case
    # the mask-extent skipping is for
    "n512_cz128_c128_b2_bf16_ragged": dict(dtype="bf16", batch=2, n=512, c_z=128, c=128,
                                           mask="lengths", lengths=(300, 512)),
}
HEADLINE = "n512_cz128_c128_bf16_masked"


def weight_shapes(c_z, c):
    return {
        "ln_in_gamma": (c_z,), "ln_in_beta": (c_z,),
        "w_a_gate": (c, c_z), "b_a_gate": (c,), "w_a_proj": (c, c_z), "b_a_proj": (c,),
        "w_b_gate": (c, c_z), "b_b_gate": (c,), "w_b_proj": (c, c_z), "b_b_proj": (c,),
        "ln_out_gamma": (c,), "ln_out_beta": (c,),
        "w_out": (c_z, c), "b_out": (c_z,),
        "w_gate": (c_z, c_z), "b_gate": (c_z,),
    }


def make_weights(rng, c_z, c, random_affine=False):
    """float32 weights in field order. Matrices N(0, 1/fan_in)."""
    out = {}
    for name, shape in weight_shapes(c_z, c).items():
        if name.startswith("w_"):
            out[name] = (rng.standard_normal(shape) / np.sqrt(shape[1])).astype(np.float32)
        elif name.endswith("gamma"):
            out[name] = (1.0 + 0.2 * rng.standard_normal(shape) if random_affine
                         else np.ones(shape)).astype(np.float32)
        else:  # biases and betas
            out[name] = (0.2 * rng.standard_normal(shape) if random_affine
                         else np.zeros(shape)).astype(np.float32)
    return out


def transition_weight_shapes(c_z, hidden):
    return {"ln_gamma": (c_z,), "ln_beta": (c_z,), "w1": (hidden, c_z), "b1": (hidden,),
            "w2": (c_z, hidden), "b2": (c_z,)}


def make_transition_weights(rng, c_z, hidden, random_affine=False):
    """float32 pair-transition weights (nn.Linear orientation). Matrices N(0, 1/fan_in);
    LayerNorm gamma 1 / beta 0 and zero biases unless random_affine."""
    out = {}
    for name, shape in transition_weight_shapes(c_z, hidden).items():
        if name.startswith("w"):
            out[name] = (rng.standard_normal(shape) / np.sqrt(shape[1])).astype(np.float32)
        elif name == "ln_gamma":
            out[name] = (1.0 + 0.2 * rng.standard_normal(shape) if random_affine
                         else np.ones(shape)).astype(np.float32)
        else:
            out[name] = (0.2 * rng.standard_normal(shape) if random_affine
                         else np.zeros(shape)).astype(np.float32)
    return out


def attention_weight_shapes(c_z, heads, d):
    hd = heads * d
    return {"ln_gamma": (c_z,), "ln_beta": (c_z,), "w_q": (hd, c_z), "w_k": (hd, c_z),
            "w_v": (hd, c_z), "w_b": (heads, c_z), "w_g": (hd, c_z), "b_g": (hd,),
            "w_o": (c_z, hd), "b_o": (c_z,)}


def make_attention_weights(rng, c_z, heads, d, random_affine=False):
    """float32 triangular-attention weights (nn.Linear orientation, heads stacked along
    the output rows). Matrices N(0, 1/fan_in); LayerNorm gamma 1 / beta 0 and zero
    biases unless random_affine."""
    out = {}
    for name, shape in attention_weight_shapes(c_z, heads, d).items():
        if name.startswith("w_"):
            out[name] = (rng.standard_normal(shape) / np.sqrt(shape[1])).astype(np.float32)
        elif name == "ln_gamma":
            out[name] = (1.0 + 0.2 * rng.standard_normal(shape) if random_affine
                         else np.ones(shape)).astype(np.float32)
        else:
            out[name] = (0.2 * rng.standard_normal(shape) if random_affine
                         else np.zeros(shape)).astype(np.float32)
    return out


def block_mask(batch, n, lengths):
    """1 on the leading L x L block of each item, 0 on padding."""
    m = np.zeros((batch, n, n), dtype=np.float32)
    for b, L in enumerate(lengths):
        m[b, :L, :L] = 1.0
    return m


def make_workload(name, seed=0, random_affine=False):
    """Return dict(z=float32 [B,N,N,c_z], mask=float32 [B,N,N], weights, meta)."""
    spec = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    B, n, c_z, c = spec["batch"], spec["n"], spec["c_z"], spec["c"]
    meta = dict(spec, name=name, seed=seed)
    if spec["mask"] == "block":
        lo, hi = spec["l_range"]
        L = int(rng.integers(lo, hi + 1))  # inclusive U[lo, hi], drawn first
        meta["valid_length"] = L
        mask = block_mask(B, n, [L] * B)
    elif spec["mask"] == "lengths":
        meta["valid_lengths"] = list(spec["lengths"])
        mask = block_mask(B, n, list(spec["lengths"]))
    elif spec["mask"] == "chains":
        total = int(sum(spec["chains"]))
        meta["valid_length"] = total  # every chain residue is valid
        mask = block_mask(B, n, [total] * B)
    else:
        mask = np.ones((B, n, n), dtype=np.float32)
    z = rng.standard_normal((B, n, n, c_z), dtype=np.float32)
    weights = make_weights(rng, c_z, c, random_affine)
    return dict(z=z, mask=mask, weights=weights, meta=meta)


def make_random(batch, n, c_z, c, seed=0, mask="ones", valid=None, random_affine=True,
                z_shift=0.0, z_scale=1.0):
    """Free-form case for tests: mask in {"ones", "block", "random_residues", "random_pairs"}."""
    rng = np.random.default_rng(seed)
    if mask == "ones":
        m = np.ones((batch, n, n), dtype=np.float32)
    elif mask == "block":
        lengths = valid if valid is not None else [max(1, n - 1 - b) for b in range(batch)]
        m = block_mask(batch, n, lengths)
    elif mask == "random_residues":
        r = (rng.random((batch, n)) < 0.7).astype(np.float32)
        m = r[:, :, None] * r[:, None, :]
    elif mask == "random_pairs":
        m = (rng.random((batch, n, n)) < 0.7).astype(np.float32)
    else:
        raise ValueError(mask)
    z = (z_shift + z_scale * rng.standard_normal((batch, n, n, c_z))).astype(np.float32)
    weights = make_weights(rng, c_z, c, random_affine)
    return dict(z=z, mask=m, weights=weights)
