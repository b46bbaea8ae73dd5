"""Mask extents (tri_mul_mask_extents) and the update with work skipping
(tri_mul_forward_extents) on the GPU.

The extents are integer results: bit-exact against NumPy. The update with skipping must
give exactly the plain update's values (outside each item's leading L x L square both
operands are zero, so the skipped products add nothing) and match the fp64 oracle at the
usual tolerance; that includes the padded two-item workload the skipping is for."""

import numpy as np
import pytest
import torch

from oracle import tri_mul_ref
from pair_rep_triangle_amd.inputs import block_mask, make_random, make_workload
from pair_rep_triangle_amd.trimul import TriMul, mask_extents
from tests.gpu_util import TOL, check_residual_update, note, rel_err, to_device, torch_dtype

pytestmark = pytest.mark.gpu
DIRS = ("outgoing", "incoming")


def extent_ref(mask):
    """1 + the largest max(i, j) over the nonzero entries of each item, 0 if none."""
    out = []
    for m in np.asarray(mask):
        ii, jj = np.nonzero(m)
        out.append(int(np.maximum(ii, jj).max()) + 1 if ii.size else 0)
    return out


def _masks(rng, batch, n):
    yield "ones", np.ones((batch, n, n), np.float32)
    yield "block", block_mask(batch, n, [int(v) for v in rng.integers(0, n + 1, batch)])
    r = (rng.random((batch, n)) < 0.6).astype(np.float32)
    yield "residues", r[:, :, None] * r[:, None, :]
    yield "pairs", (rng.random((batch, n, n)) < 0.01).astype(np.float32)
    m = np.zeros((batch, n, n), np.float32)
    m[0, n - 1, 0] = 1.0  # one nonzero pair in the last row: the extent is n
    if batch > 1:
        m[1, 0, n // 2] = 1.0
    yield "single", m
    yield "zeros", np.zeros((batch, n, n), np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("batch,n", [(1, 1), (3, 7), (2, 65), (1, 300), (2, 513), (1, 2048)])
def test_mask_extents_are_exact(dtype, batch, n):
    rng = np.random.default_rng(n + batch)
    for kind, m in _masks(rng, batch, n):
        note(f"extents {dtype} B={batch} n={n} {kind}")
        md = torch.from_numpy(m).to(torch_dtype(dtype)).cuda()
        parts = mask_extents(md)
        torch.cuda.synchronize()
        got = parts.max(dim=1).values.cpu().tolist()
        assert got == extent_ref(m), (kind, got, extent_ref(m))


@pytest.mark.parametrize("dtype,B,n,c_z,c,lengths", [
    ("bf16", 2, 300, 128, 128, (150, 300)),    # wave-independent projection kernels
    ("bf16", 3, 129, 64, 64, (0, 1, 97)),      # an empty item, a one-residue item
    ("bf16", 2, 520, 32, 32, (257, 33)),       # extents across 256-row contraction tiles
    ("fp32", 2, 200, 64, 48, (64, 199)),
    ("fp32", 1, 45, 16, 16, (45,)),
    ("bf16", 2, 70, 384, 128, (40, 70)),      # the wide pair track: streamed output gate
])
def test_forward_with_extents_equals_plain_forward(dtype, B, n, c_z, c, lengths):
    d = make_random(B, n, c_z, c, seed=n + c, mask="block", valid=list(lengths),
                    random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    mod = TriMul(d["weights"], c_z, c, dtype)
    ws = mod.new_workspace(B, n)
    ext = mask_extents(m)
    assert ext.max(dim=1).values.cpu().tolist() == list(lengths)
    for direction in DIRS:
        note(f"extents forward {dtype} B={B} n={n} c_z={c_z} c={c} {lengths} {direction}")
        plain = mod.forward(z, m, direction=direction, workspace=ws).clone()
        skip = mod.forward(z, m, direction=direction, workspace=ws, extents=ext)
        torch.cuda.synchronize()
        assert torch.equal(plain, skip)
        want = tri_mul_ref(z_host, m_host, d["weights"], direction)
        assert rel_err(skip.double().cpu().numpy(), want) <= TOL[dtype]
        # with the residual add, out of place and (where allowed) in place
        res = mod.forward_residual(z, m, direction=direction, workspace=ws, extents=ext)
        torch.cuda.synchronize()
        check_residual_update(res.double().cpu().numpy(), z_host, want, dtype)
        if mod.plan(B, n)["in_place_ok"]:
            zi = z.clone()
            mod.forward_residual(zi, m, out=zi, direction=direction, workspace=ws, extents=ext)
            torch.cuda.synchronize()
            assert torch.equal(zi, res)


@pytest.mark.parametrize("direction", DIRS)
def test_padded_batch_workload_with_extents(direction):
    """B = 2, N = 512, valid lengths 300 and 512: the full output against the oracle."""
    name = "n512_cz128_c128_b2_bf16_ragged"
    d = make_workload(name, seed=0)
    z, m, z_host, m_host = to_device(d, "bf16")
    mod = TriMul(d["weights"], 128, 128, "bf16")
    ext = mask_extents(m)
    note(f"{name} {direction} with extents")
    out = mod.forward(z, m, direction=direction, extents=ext)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    want = tri_mul_ref(z_host, m_host, d["weights"], direction)
    err = rel_err(got, want)
    print(f"{name} {direction}: rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.all(got[0, 300:] == 0) and np.all(got[0, :, 300:] == 0)


def test_forward_extents_rejects_bad_calls():
    d = make_random(2, 40, 32, 32, seed=1, mask="block", valid=[20, 40])
    z, m, _, _ = to_device(d, "bf16")
    note("extents validation")
    mod = TriMul(d["weights"], 32, 32, "bf16")
    lib, h = mod.lib, mod._h
    ws = mod.new_workspace(2, 40)
    out = torch.empty_like(z)
    ext = mask_extents(m)
    st = torch.cuda.current_stream().cuda_stream
    args = (z.data_ptr(), m.data_ptr())
    call = lambda e, o, res, w: lib.tri_mul_forward_extents(  # noqa: E731
        h, *args, e, o, 2, 40, 0, res, w, ws.numel(), st)
    assert call(ext.data_ptr(), out.data_ptr(), 0, ws.data_ptr()) == 0
    assert call(None, out.data_ptr(), 0, ws.data_ptr()) == -1           # no extents
    assert call(ext.data_ptr(), out.data_ptr(), 2, ws.data_ptr()) == -1  # residual flag
    assert call(ext.data_ptr() + 2, out.data_ptr(), 0, ws.data_ptr()) == -4
    # extents inside the workspace or the output would be overwritten before they are read
    assert call(ws.data_ptr() + 1024, out.data_ptr(), 0, ws.data_ptr()) == -5
    assert call(out.data_ptr(), out.data_ptr(), 0, ws.data_ptr()) == -5
    # the extents kernel itself: dtype, NULL, alignment, overlap with the mask
    assert lib.tri_mul_mask_extents(7, m.data_ptr(), 2, 40, ext.data_ptr(), st) == -2
    assert lib.tri_mul_mask_extents(1, None, 2, 40, ext.data_ptr(), st) == -1
    assert lib.tri_mul_mask_extents(1, m.data_ptr(), 2, 40, ext.data_ptr() + 2, st) == -4
    assert lib.tri_mul_mask_extents(1, m.data_ptr(), 2, 40, m.data_ptr(), st) == -5
    with pytest.raises(ValueError):
        mod.forward(z, m, extents=ext[:1])
    with pytest.raises(ValueError):
        mod.forward(z, m, extents=ext.cpu())
    torch.cuda.synchronize()
