"""GPU parity of the fused residual add (tri_mul_forward_residual) and of the chained
pair update (outgoing, then incoming on its result) against the fp64 oracle."""

import numpy as np
import pytest
import torch

from oracle import pair_update_ref, tri_mul_ref, tri_mul_residual_ref
from pair_rep_triangle_amd.inputs import make_random, make_weights, make_workload
from pair_rep_triangle_amd.trimul import TriMul, TriMulError
from tests.gpu_util import TOL, note, rel_err, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _host(t):
    return t.to(torch.float64).cpu().numpy()


def _check_residual(got, z_host, m_host, w, direction, dtype):
    """z_out against z + out, and the increment z_out - z against out alone (the
    increment is the part the kernels compute; z dominates the plain comparison)."""
    want = tri_mul_residual_ref(z_host, m_host, w, direction)
    upd = tri_mul_ref(z_host, m_host, w, direction)
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= TOL[dtype]
    # the increment after rounding z_out to the storage type: bf16 rounding of a value of
    # size |z| costs about 2^-9 |z|, so the bar is scaled by max|z| / max|upd|
    slack = 1.0 if dtype == "fp32" else max(1.0, 4 * np.abs(z_host).max() / np.abs(upd).max())
    assert rel_err(got - z_host, upd) <= TOL[dtype] * slack
    # padded pairs keep z exactly (their update is 0)
    if m_host is not None:
        pad = m_host == 0
        assert np.array_equal(got[pad], z_host[pad])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,c_z,c,mask", [
    (1, 45, 32, 32, "block"), (2, 70, 64, 48, "random_pairs"), (1, 129, 128, 128, "block"),
])
def test_residual_out_of_place_and_in_place(dtype, direction, B, N, c_z, c, mask):
    d = make_random(B, N, c_z, c, seed=N + c, mask=mask, random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    note(f"residual {dtype} {direction} B={B} N={N} c_z={c_z} c={c} {mask}")
    mod = TriMul(d["weights"], c_z, c, dtype)
    ws = mod.new_workspace(B, N)
    out = mod.forward_residual(z, m, direction=direction, workspace=ws)
    torch.cuda.synchronize()
    got = _host(out)
    _check_residual(got, z_host, m_host, d["weights"], direction, dtype)
    # in place gives the same bytes
    zi = z.clone()
    mod.forward_residual(zi, m, out=zi, direction=direction, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(zi, out)


def test_residual_wide_shape_tile_shared_kernel():
    """c_z = 384, c = 256: the output kernel falls back to its tile-shared form."""
    d = make_random(1, 50, 384, 256, seed=5, mask="block", random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    note("residual wide bf16 384/256")
    mod = TriMul(d["weights"], 384, 256, "bf16")
    for direction in ("outgoing", "incoming"):
        zi = z.clone()
        mod.forward_residual(zi, m, out=zi, direction=direction)
        torch.cuda.synchronize()
        _check_residual(_host(zi), z_host, m_host, d["weights"], direction, "bf16")


@pytest.mark.parametrize("dtype,B,N,c_z,c", [
    ("fp32", 1, 40, 32, 16), ("bf16", 1, 96, 64, 64), ("bf16", 2, 61, 128, 128),
])
def test_chained_pair_update(dtype, B, N, c_z, c):
    d = make_random(B, N, c_z, c, seed=11 + N, mask="random_residues", random_affine=True)
    w_in = make_weights(np.random.default_rng(99), c_z, c, random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    note(f"chained pair update {dtype} B={B} N={N} c_z={c_z} c={c}")
    out_mod, in_mod = TriMul(d["weights"], c_z, c, dtype), TriMul(w_in, c_z, c, dtype)
    ws = out_mod.new_workspace(B, N)
    zi = z.clone()
    out_mod.forward_residual(zi, m, out=zi, direction="outgoing", workspace=ws)
    in_mod.forward_residual(zi, m, out=zi, direction="incoming", workspace=ws)
    torch.cuda.synchronize()
    got = _host(zi)
    want = pair_update_ref(z_host, m_host, d["weights"], w_in)
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= TOL[dtype]
    # the two increments together, against the oracle's
    slack = 1.0 if dtype == "fp32" else max(1.0, 4 * np.abs(z_host).max() /
                                            np.abs(want - z_host).max())
    assert rel_err(got - z_host, want - z_host) <= TOL[dtype] * slack


def test_chained_headline_workload_sampled():
    """The masked N = 512 workload, chained in place, checked on every pair of a few rows
    (the oracle evaluates the incoming step from the full outgoing result)."""
    d = make_workload("n512_cz128_c128_bf16_masked", seed=0)
    w_in = make_weights(np.random.default_rng(1), 128, 128)
    z, m, z_host, m_host = to_device(d, "bf16")
    note("chained headline workload")
    out_mod, in_mod = TriMul(d["weights"], 128, 128, "bf16"), TriMul(w_in, 128, 128, "bf16")
    zi = z.clone()
    out_mod.forward_residual(zi, m, out=zi, direction="outgoing")
    z1 = _host(zi)
    in_mod.forward_residual(zi, m, out=zi, direction="incoming")
    torch.cuda.synchronize()
    got = _host(zi)
    # step 1 exactly as the oracle, step 2 from the device's own bf16 z1 (what it read)
    z1_ref = tri_mul_residual_ref(z_host, m_host, d["weights"], "outgoing")
    assert rel_err(z1, z1_ref) <= TOL["bf16"]
    z2_ref = tri_mul_residual_ref(z1, m_host, w_in, "incoming")
    assert rel_err(got, z2_ref) <= TOL["bf16"]
    assert rel_err(got - z1, z2_ref - z1) <= TOL["bf16"] * 4


def test_residual_rejects_partial_overlap():
    d = make_random(1, 24, 32, 16, seed=2)
    z, m, _, _ = to_device(d, "bf16")
    mod = TriMul(d["weights"], 32, 16, "bf16")
    big = torch.zeros(2 * z.numel(), dtype=torch_dtype("bf16"), device="cuda")
    zb = big[: z.numel()].view_as(z)
    zb.copy_(z)
    shifted = big[32: 32 + z.numel()].view_as(z)  # overlaps zb, not equal to it
    with pytest.raises(TriMulError) as ei:
        mod.forward_residual(zb, m, out=shifted, direction="outgoing")
    assert ei.value.name == "ALIAS"
    with pytest.raises(TriMulError) as ei:
        mod.forward(zb, m, out=zb, direction="outgoing")  # in place only with the residual
    assert ei.value.name == "ALIAS"
