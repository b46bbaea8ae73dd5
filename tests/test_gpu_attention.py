"""GPU parity of triangular attention (tri_attn_forward) against the fp64 oracle, both
nodes. Tolerance: max |gpu - ref| / max |ref| <= 2e-2 (bf16 storage of z, out and the
projections; fp32 accumulation and softmax)."""

import numpy as np
import pytest
import torch

from oracle import tri_attention_ref, tri_attention_ref_lines
from pair_rep_triangle_amd.inputs import make_attention_weights, make_random, make_workload
from pair_rep_triangle_amd.trimul import TriAttention, TriMulError
from tests.gpu_util import TOL, note, rel_err, to_device

pytestmark = pytest.mark.gpu

NODES = ("starting", "ending")


def _run(B, n, c_z, heads, mask, seed, node, use_mask=True):
    d = make_random(B, n, c_z, 16, seed=seed, mask=mask)
    w = make_attention_weights(np.random.default_rng(seed + 100), c_z, heads, 32,
                               random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    if not use_mask:
        m, m_host = None, None
    mod = TriAttention(w, c_z, heads)
    out = mod.forward(z, m, node=node)
    torch.cuda.synchronize()
    return out, z, m, z_host, m_host, w, mod


@pytest.mark.parametrize("node", NODES)
@pytest.mark.parametrize("B,n,c_z,heads,mask", [
    (1, 40, 64, 2, "random_pairs"),
    (2, 33, 128, 4, "block"),            # ragged n, two items, the widest supported
    (1, 70, 32, 1, "random_residues"),   # fully padded residues: queries with no valid key
    (1, 64, 96, 3, "ones"),              # three heads (a wave of the workgroup idles)
    (1, 129, 64, 8, "random_pairs"),     # eight heads: each wave runs two
    (1, 45, 128, 8, "ones"),             # projection weights in two parts
    (1, 70, 160, 2, "random_residues"),  # five chunk groups: no z prefetch
    (2, 33, 256, 4, "block"),            # projection weights in two parts
    (1, 40, 384, 4, "random_pairs"),     # the wide pair track: three parts, twelve groups
    (1, 160, 384, 4, "block"),           # the same over several tiles and key steps
    (1, 50, 384, 8, "random_residues"),  # eight heads: six parts; W_o in three slices
])
def test_attention_full_output(node, B, n, c_z, heads, mask):
    note(f"attention {node} B={B} n={n} cz={c_z} heads={heads} {mask}")
    out, z, m, z_host, m_host, w, _ = _run(B, n, c_z, heads, mask, seed=n + c_z, node=node)
    got = out.to(torch.float64).cpu().numpy()
    want = tri_attention_ref(z_host, m_host, w, node)
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= TOL["bf16"]


@pytest.mark.parametrize("node", NODES)
def test_attention_null_mask_means_all_ones(node):
    note(f"attention null mask {node}")
    out, z, _, z_host, _, w, mod = _run(1, 45, 64, 2, "ones", seed=5, node=node, use_mask=False)
    ones = torch.ones(z.shape[:3], dtype=z.dtype, device=z.device)
    assert torch.equal(mod.forward(z, ones, node=node), out)
    want = tri_attention_ref(z_host, None, w, node)
    assert rel_err(out.to(torch.float64).cpu().numpy(), want) <= TOL["bf16"]


@pytest.mark.parametrize("node", NODES)
def test_attention_repeatable(node):
    """Two runs give the same bytes (no race between waves or workgroups)."""
    note(f"attention repeat {node}")
    out, z, m, _, _, _, mod = _run(1, 96, 128, 4, "random_pairs", seed=6, node=node)
    again = mod.forward(z, m, node=node)
    torch.cuda.synchronize()
    assert torch.equal(out, again)


@pytest.mark.parametrize("node", NODES)
@pytest.mark.parametrize("case", ["rising", "sinking", "leading_keys_masked"])
def test_attention_moving_softmax_reference(node, case):
    """Each query's softmax reference starts at 0 and moves up only when a score lies
    more than 16 (base 2) above it; at the query's first valid key step it drops to the
    step's largest score when that lies below -16. A pair channel that grows along the key
    index, with a large bias weight on it, shapes the scores: "rising" (about -18 to +22)
    moves the reference up later in the row for about 4% of the queries, with the sums
    scaled; "sinking" (about -29 to -2) drops it below 0 at the first key step for 25-60%
    of them. "leading_keys_masked": the first 70 keys of every row are masked, so the
    first two key steps have no valid key at all and the third is the first one summed. The
    result is the plain softmax every time. The scores are large, so the bf16 storage of
    z-hat, the weights, q, k, v, the gate, the bias and the probabilities costs more here
    than elsewhere: a CPU model of exactly those roundings, with the textbook softmax,
    lands at 1.0-1.5% on these inputs."""
    n, c_z, heads = 160, 64, 2
    note(f"attention softmax reference {case} {node} n={n}")
    d = make_random(1, n, c_z, 16, seed=11, mask="block")
    w = make_attention_weights(np.random.default_rng(111), c_z, heads, 32, random_affine=True)
    z, mask = d["z"].copy(), d["mask"].copy()
    # keys of the starting node are (i, k) with bias (j, k) and key mask (i, k); of the
    # ending node (k, j) with bias (k, i) and key mask (k, j): the key index is the second
    # residue axis, or the first
    if case in ("rising", "sinking"):
        amp, shift, wb = (3.0, 0.0, 2.0) if case == "rising" else (2.0, -8.0, 2.5)
        ramp = np.linspace(-amp, amp, n, dtype=np.float32) + np.float32(shift)
        if node == "starting":
            z[0, :, :, 0] += ramp[None, :]
        else:
            z[0, :, :, 0] += ramp[:, None]
        w["w_b"] = w["w_b"].copy()
        w["w_b"][:, 0] = wb
    elif node == "starting":
        mask[0, :, :70] = 0.0
    else:
        mask[0, :70, :] = 0.0
    zt, m, z_host, m_host = to_device(dict(z=z, mask=mask), "bf16")
    out = TriAttention(w, c_z, heads).forward(zt, m, node=node)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    want = tri_attention_ref(z_host, m_host, w, node)
    err = rel_err(got, want)
    note(f"  rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL["bf16"]


def test_attention_writes_nothing_past_the_output():
    note("attention guard band")
    d = make_random(1, 37, 64, 16, seed=7, mask="block")
    w = make_attention_weights(np.random.default_rng(7), 64, 2, 32, random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    mod = TriAttention(w, 64, 2)
    count = z.numel()
    big = torch.full((count + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:count].view_as(z)
    for node in NODES:
        mod.forward(z, m, out=out, node=node)
        torch.cuda.synchronize()
        assert torch.all(big[count:] == 7.0)
        assert rel_err(out.to(torch.float64).cpu().numpy(),
                       tri_attention_ref(z_host, m_host, w, node)) <= TOL["bf16"]


def test_attention_rejects_small_workspace_and_overlap():
    d = make_random(1, 24, 64, 16, seed=8)
    w = make_attention_weights(np.random.default_rng(8), 64, 2, 32)
    z, m, _, _ = to_device(d, "bf16")
    mod = TriAttention(w, 64, 2)
    small = torch.empty(mod.workspace_bytes(1, 24) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(TriMulError) as ei:
        mod.forward(z, m, workspace=small)
    assert ei.value.name == "WORKSPACE_TOO_SMALL"
    with pytest.raises(TriMulError) as ei:
        mod.forward(z, m, out=z)
    assert ei.value.name == "ALIAS"


@pytest.mark.parametrize("node", NODES)
def test_attention_headline_shape_sampled(node):
    """N = 512, c_z = 128, 4 heads of 32, bf16, the block mask of the headline workload
    (valid length 493): full device output, oracle on sampled query lines (the first and
    last lines, lines around the valid length, padded lines, random ones)."""
    note(f"attention headline {node}")
    d = make_workload("n512_cz128_c128_bf16_masked", seed=0)
    w = make_attention_weights(np.random.default_rng(2), 128, 4, 32, random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    mod = TriAttention(w, 128, 4)
    out = mod.forward(z, m, node=node)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    assert np.isfinite(got).all()
    L = d["meta"]["valid_length"]
    extra = np.random.default_rng(9).integers(0, 512, 4).tolist()
    lines = sorted({0, 1, L - 2, L - 1, L, 511} | set(extra))
    want = tri_attention_ref_lines(z_host, m_host, w, node, lines)
    sel = got[:, lines] if node == "starting" else np.swapaxes(got[:, :, lines], 1, 2)
    assert rel_err(sel, want) <= TOL["bf16"]


@pytest.mark.parametrize("node", NODES)
def test_attention_stages_compose_to_forward(node):
    """Stage 1 (projection) then stage 2 (attention) gives forward's bytes."""
    note(f"attention stages {node}")
    out, z, m, _, _, _, mod = _run(1, 50, 64, 2, "random_pairs", seed=10, node=node)
    ws = mod.new_workspace(1, 50)
    staged = torch.empty_like(out)
    mod.stage(1, z, m, out=staged, node=node, workspace=ws)
    mod.stage(2, z, m, out=staged, node=node, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(staged, out)
