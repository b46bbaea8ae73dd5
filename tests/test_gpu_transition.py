"""GPU parity of the pair transition (pair_transition_forward) against the fp64 oracle.

Tolerance (max |gpu - ref| / max |ref|): 1e-4 fp32, 2e-2 bf16, on the output; and on the
update u alone: every element within the tolerance times max|u_ref| of the
storage-rounded z + u_ref, plus one unit of the storage type for that final rounding."""

import numpy as np
import pytest
import torch

from oracle import pair_transition_ref
from pair_rep_triangle_amd.inputs import make_random, make_transition_weights
from pair_rep_triangle_amd.trimul import PairTransition, TriMulError
from tests.gpu_util import TOL, check_residual_update, note, rel_err, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _check(got, z_host, m_host, w, dtype):
    want = pair_transition_ref(z_host, m_host, w)
    upd = want - z_host
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= TOL[dtype]
    check_residual_update(got, z_host, upd, dtype)
    if m_host is not None:
        pad = m_host == 0
        assert np.array_equal(got[pad], z_host[pad])  # padded pairs keep z exactly


def _run(dtype, B, n, c_z, hidden, mask, seed, in_place=False, use_mask=True):
    d = make_random(B, n, c_z, 16, seed=seed, mask=mask)
    w = make_transition_weights(np.random.default_rng(seed + 100), c_z, hidden, random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    if not use_mask:
        m, m_host = None, None
    mod = PairTransition(w, c_z, hidden, dtype)
    if in_place:
        zi = z.clone()
        mod.forward(zi, m, out=zi)
        out = zi
    else:
        out = mod.forward(z, m)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    _check(got, z_host, m_host, w, dtype)
    return out, z, m, mod


@pytest.mark.parametrize("dtype,B,n,c_z,hidden,mask", [
    ("bf16", 1, 64, 128, 256, "random_pairs"),   # the released expansion of 2
    ("bf16", 2, 37, 64, 128, "block"),            # pairs not a multiple of the 32-pair tile
    ("bf16", 1, 45, 96, 200, "random_residues"),  # hidden padded to 224, three chunk groups
    ("bf16", 3, 9, 32, 64, "ones"),
    ("bf16", 1, 30, 128, 100, "random_pairs"),    # hidden smaller than c_z
    ("fp32", 1, 50, 64, 128, "random_pairs"),
    ("fp32", 2, 21, 16, 40, "block"),             # hidden padded to 48, one chunk group
    ("fp32", 1, 33, 48, 96, "random_residues"),
])
def test_transition_full_output(dtype, B, n, c_z, hidden, mask):
    note(f"transition {dtype} B={B} n={n} cz={c_z} hidden={hidden} {mask}")
    _run(dtype, B, n, c_z, hidden, mask, seed=n + c_z)


# Widths whose weights do not fit one workgroup's LDS: the bf16 form that streams them
# through LDS one hidden group of 32 units at a time (c_z padded to 128/256/384/512).
@pytest.mark.parametrize("B,n,c_z,hidden,mask", [
    (1, 64, 384, 768, "random_pairs"),    # the released pair width, expansion 2
    (2, 37, 256, 512, "block"),           # ragged last 128-pair tile
    (1, 45, 320, 640, "random_residues"), # c_z padded to 384 with zero channels
    (1, 33, 512, 1024, "ones"),
    (1, 50, 128, 1024, "random_pairs"),   # narrow width, hidden too wide for resident weights
    (1, 40, 384, 700, "block"),           # hidden padded to 704
])
def test_transition_streamed_weights_full_output(B, n, c_z, hidden, mask):
    note(f"transition streamed bf16 B={B} n={n} cz={c_z} hidden={hidden} {mask}")
    _run("bf16", B, n, c_z, hidden, mask, seed=n + c_z)


def test_transition_released_shape_n512():
    """c_z = 384, hidden 768, N = 512, block mask: every pair (about 0.3 TFLOP of fp64 work in
    the oracle), the shape and launch of its benchmark line."""
    note("transition streamed N=512 c_z=384 hidden 768")
    _run("bf16", 1, 512, 384, 768, "block", seed=1)


def test_transition_streamed_in_place_and_guard_band():
    """In place equals out of place; nothing past the output changes (last tile of 128 pairs
    holds 25 pairs)."""
    note("transition streamed in place and guard band")
    n, c_z, hidden = 39, 384, 768
    out, z, m, mod = _run("bf16", 1, n, c_z, hidden, "random_pairs", seed=5)
    zi = z.clone()
    mod.forward(zi, m, out=zi)
    torch.cuda.synchronize()
    assert torch.equal(zi, out)
    count = z.numel()
    big = torch.full((count + 256 * c_z,), 7.0, dtype=torch.bfloat16, device="cuda")
    mod.forward(z, m, out=big[:count].view_as(z))
    torch.cuda.synchronize()
    assert torch.all(big[count:] == 7.0)
    assert torch.equal(big[:count].view_as(z), out)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_transition_in_place_matches_out_of_place(dtype):
    note(f"transition in place {dtype}")
    out, z, m, mod = _run(dtype, 1, 40, 64, 128, "random_pairs", seed=3)
    zi = z.clone()
    mod.forward(zi, m, out=zi)
    torch.cuda.synchronize()
    assert torch.equal(zi, out)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_transition_null_mask_means_all_ones(dtype):
    note(f"transition null mask {dtype}")
    out, z, m, mod = _run(dtype, 1, 33, 64, 128, "ones", seed=4, use_mask=False)
    ones = torch.ones(z.shape[:3], dtype=z.dtype, device=z.device)
    assert torch.equal(mod.forward(z, ones), out)


def test_transition_headline_shape():
    """N = 512, c_z = 128, hidden 256, bf16, block mask: every pair (4.3 GFLOP in the
    oracle), the shape and launch of the benchmark."""
    note("transition headline shape")
    _run("bf16", 1, 512, 128, 256, "block", seed=0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n", [45, 43])  # last tile: 9 pairs (subtile 0 only), 25 pairs
def test_transition_writes_nothing_past_the_output(dtype, n):
    """The output sits at the start of a larger buffer filled with a sentinel: the ragged
    last tile's stores past the last pair must be dropped, in both 16-pair subtiles."""
    note(f"transition guard band {dtype} n={n}")
    c_z, hidden = (64, 128) if dtype == "fp32" else (128, 256)
    d = make_random(1, n, c_z, 16, seed=n, mask="random_pairs")
    w = make_transition_weights(np.random.default_rng(n), c_z, hidden, random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    mod = PairTransition(w, c_z, hidden, dtype)
    count = z.numel()
    big = torch.full((count + 64 * c_z,), 7.0, dtype=torch_dtype(dtype), device="cuda")
    out = big[:count].view_as(z)
    mod.forward(z, m, out=out)
    torch.cuda.synchronize()
    assert torch.all(big[count:] == 7.0)
    _check(out.to(torch.float64).cpu().numpy(), z_host, m_host, w, dtype)


def test_transition_several_tiles_per_wave_repeated():
    """More tiles than waves on a ragged pair count (N = 300, bf16, c_z 128): each wave
    runs its loop with a real next tile in flight while it stores; three runs, each
    checked in full."""
    note("transition several tiles per wave, repeated")
    d = make_random(1, 300, 128, 16, seed=5, mask="block")
    w = make_transition_weights(np.random.default_rng(5), 128, 256, random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    mod = PairTransition(w, 128, 256, "bf16")
    for _ in range(3):
        out = mod.forward(z, m)
        torch.cuda.synchronize()
        _check(out.to(torch.float64).cpu().numpy(), z_host, m_host, w, "bf16")


def test_transition_rejects_partial_overlap():
    d = make_random(1, 24, 64, 16, seed=2)
    w = make_transition_weights(np.random.default_rng(0), 64, 128)
    z, m, _, _ = to_device(d, "bf16")
    mod = PairTransition(w, 64, 128, "bf16")
    big = torch.zeros(2 * z.numel(), dtype=torch_dtype("bf16"), device="cuda")
    zb = big[: z.numel()].view_as(z)
    zb.copy_(z)
    shifted = big[64: 64 + z.numel()].view_as(z)
    with pytest.raises(TriMulError) as ei:
        mod.forward(zb, m, out=shifted)
    assert ei.value.name == "ALIAS"
