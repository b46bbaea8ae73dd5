"""GPU parity of the fused residual add (tri_mul_forward_residual) and of the chained
pair update (outgoing, then incoming on its result) against the fp64 oracle.

The output z + u is checked twice: as a whole against the oracle (2e-2 / 1e-4 of its
max-abs), and for the update u alone: every element within the tolerance times max|u_ref|
of the storage-rounded z + u_ref, plus one unit of the storage type for that rounding
(tests.gpu_util.check_residual_update). In place must give the same bytes as out of
place; shapes whose output kernel splits c_z over several workgroups reject in place."""

import numpy as np
import pytest
import torch

from oracle import pair_update_ref, tri_mul_ref, tri_mul_ref_lines, tri_mul_residual_ref
from pair_rep_triangle_amd.inputs import make_random, make_weights, make_workload
from pair_rep_triangle_amd.trimul import TriMul, TriMulError
from tests.gpu_util import TOL, check_residual_update, note, rel_err, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _host(t):
    return t.to(torch.float64).cpu().numpy()


def _check_residual(got, z_host, m_host, w, direction, dtype):
    upd = tri_mul_ref(z_host, m_host, w, direction)
    assert np.isfinite(got).all()
    assert rel_err(got, z_host + upd) <= TOL[dtype]
    check_residual_update(got, z_host, upd, dtype)
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
    _check_residual(_host(out), z_host, m_host, d["weights"], direction, dtype)
    if not mod.plan(B, N)["in_place_ok"]:
        return
    zi = z.clone()
    mod.forward_residual(zi, m, out=zi, direction=direction, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(zi, out)


@pytest.mark.parametrize("dtype,c_z,c", [("bf16", 128, 128), ("fp32", 64, 64), ("bf16", 96, 32)])
def test_in_place_many_tiles_per_wave_is_bitwise_out_of_place(dtype, c_z, c):
    """N = 512: every wave of the output kernel runs many tiles, so a read of z that raced
    a store of another wave would show. In place must equal out of place byte for byte."""
    d = make_random(1, 512, c_z, c, seed=c_z + 7, mask="random_pairs", random_affine=True)
    z, m, _, _ = to_device(d, dtype)
    mod = TriMul(d["weights"], c_z, c, dtype)
    plan = mod.plan(1, 512)
    assert plan["in_place_ok"] == 1 and plan["output_groups"] == 1
    ws = mod.new_workspace(1, 512)
    for direction in ("outgoing", "incoming"):
        note(f"in place N=512 {dtype} c_z={c_z} c={c} {direction}")
        ref = mod.forward_residual(z, m, direction=direction, workspace=ws)
        for _ in range(3):
            zi = z.clone()
            mod.forward_residual(zi, m, out=zi, direction=direction, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(zi, ref)


@pytest.mark.parametrize("dtype,N,c_z,c", [
    ("fp32", 512, 128, 128),   # wave-independent output kernel, 2 channel groups
    ("fp32", 64, 256, 128),    # tile-shared output kernel, 2 channel groups
    ("bf16", 64, 512, 512),    # tile-shared, 4 channel groups
])
def test_in_place_rejected_with_several_channel_groups(dtype, N, c_z, c):
    d = make_random(1, N, c_z, c, seed=3, mask="ones")
    z, m, _, _ = to_device(d, dtype)
    note(f"in place rejected {dtype} N={N} c_z={c_z} c={c}")
    mod = TriMul(d["weights"], c_z, c, dtype)
    plan = mod.plan(1, N)
    assert plan["output_groups"] > 1 and plan["in_place_ok"] == 0
    zi = z.clone()
    with pytest.raises(TriMulError) as ei:
        mod.forward_residual(zi, m, out=zi, direction="outgoing")
    assert ei.value.name == "ALIAS"
    torch.cuda.synchronize()
    assert torch.equal(zi, z)  # nothing was launched


@pytest.mark.parametrize("dtype,N,c_z,c,in_place", [
    ("bf16", 70, 128, 512, True),    # one channel group
    ("fp32", 45, 256, 128, False),   # two channel groups: out of place only
    ("bf16", 33, 512, 512, False),   # four channel groups
])
def test_residual_tile_shared_output_kernel(dtype, N, c_z, c, in_place):
    """Shapes whose output kernel takes the tile-shared form (asserted through the plan)."""
    d = make_random(1, N, c_z, c, seed=5 + c, mask="block", random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    mod = TriMul(d["weights"], c_z, c, dtype)
    plan = mod.plan(1, N)
    assert plan["output_form"] == 1 and plan["in_place_ok"] == int(in_place)
    for direction in ("outgoing", "incoming"):
        note(f"residual tile-shared {dtype} N={N} c_z={c_z} c={c} {direction}")
        out = mod.forward_residual(z, m, direction=direction)
        torch.cuda.synchronize()
        _check_residual(_host(out), z_host, m_host, d["weights"], direction, dtype)
        if in_place:
            zi = z.clone()
            mod.forward_residual(zi, m, out=zi, direction=direction)
            torch.cuda.synchronize()
            assert torch.equal(zi, out)


@pytest.mark.parametrize("B,N,c_z,c", [
    (2, 70, 384, 128),   # the wide pair track
    (1, 45, 256, 128),
    (1, 33, 512, 64),    # c padded to 128
    (1, 100, 320, 96),   # c_z padded to 384, c to 128
])
def test_streamed_output_gate(B, N, c_z, c):
    """bf16 c_z above 128: the output gate streams its weights and one workgroup writes every
    channel of its pairs, so in place is allowed and must equal out of place."""
    d = make_random(B, N, c_z, c, seed=N + c_z, mask="random_pairs", random_affine=True)
    z, m, z_host, m_host = to_device(d, "bf16")
    mod = TriMul(d["weights"], c_z, c, "bf16")
    plan = mod.plan(B, N)
    assert plan["output_form"] == 2 and plan["output_groups"] == 1 and plan["in_place_ok"] == 1
    for direction in ("outgoing", "incoming"):
        note(f"streamed output gate B={B} N={N} c_z={c_z} c={c} {direction}")
        want = tri_mul_ref(z_host, m_host, d["weights"], direction)
        out = mod.forward(z, m, direction=direction)
        torch.cuda.synchronize()
        assert rel_err(_host(out), want) <= TOL["bf16"]
        res = mod.forward_residual(z, m, direction=direction)
        torch.cuda.synchronize()
        check_residual_update(_host(res), z_host, want, "bf16")
        zi = z.clone()
        mod.forward_residual(zi, m, out=zi, direction=direction)
        torch.cuda.synchronize()
        assert torch.equal(zi, res)


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
    z1 = _host(zi)
    in_mod.forward_residual(zi, m, out=zi, direction="incoming", workspace=ws)
    torch.cuda.synchronize()
    got = _host(zi)
    want = pair_update_ref(z_host, m_host, d["weights"], w_in)
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= TOL[dtype]
    # each step's update on its own: the first from z, the second from the device's own
    # rounded intermediate (what the second step read)
    check_residual_update(z1, z_host, tri_mul_ref(z_host, m_host, d["weights"], "outgoing"), dtype)
    check_residual_update(got, z1, tri_mul_ref(z1, m_host, w_in, "incoming"), dtype)


def test_chained_headline_workload_lines():
    """The masked N = 512 workload, chained in place; complete output rows and columns
    through every contraction tile (256 rows by 128 or 256 columns), for both steps."""
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
    rows, cols = [0, 100, 300, 492, 493, 511], [5, 130, 260, 400, 492, 511]
    for zin, zout, w, direction in ((z_host, z1, d["weights"], "outgoing"),
                                    (z1, got, w_in, "incoming")):
        u_r, u_c = tri_mul_ref_lines(zin, m_host, w, direction, 0, rows, cols)
        check_residual_update(zout[0][rows], zin[0][rows], u_r, "bf16")
        check_residual_update(zout[0][:, cols], zin[0][:, cols], u_c, "bf16")
    # the whole chained result, as a sum of the two steps, against the oracle's
    z2_ref = tri_mul_residual_ref(z1, m_host, w_in, "incoming")
    assert rel_err(got, z2_ref) <= TOL["bf16"]


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
