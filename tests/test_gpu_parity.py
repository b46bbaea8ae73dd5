"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (max |gpu - ref| / max |ref|): 1e-4 for fp32 storage, 2e-2 for bf16
storage with fp32 accumulation. Full-output comparisons at sizes the oracle
finishes in seconds; sampled pairs at the large workloads, run in the same
launch configuration the benchmark times."""

import numpy as np
import pytest
import torch

from pair_rep_triangle_amd.inputs import WORKLOADS, make_random, make_workload
from oracle import line_operands, tri_mul_ref_lines
from tests.gpu_util import (TOL, TriMul, check_full, check_residual_update, note, rel_err,
                            run_full, to_device, tri_mul_intermediates, tri_mul_ref, torch_dtype)

pytestmark = pytest.mark.gpu
DIRS = ("outgoing", "incoming")


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


# --- the five workloads ---------------------------------------------------------------------

@pytest.mark.parametrize("direction", DIRS)
@pytest.mark.parametrize("name", ["n32_cz16_c16_fp32", "n256_cz128_c128_bf16",
                                  "n512_cz128_c128_bf16_masked"])
def test_workload_full_output(name, direction):
    note(f"workload {name} {direction} full")
    d = make_workload(name, seed=0)
    err, _, _ = check_full(d, WORKLOADS[name]["dtype"], direction)
    print(f"{name} {direction}: rel err {err:.3e}")


@pytest.mark.parametrize("direction", DIRS)
def test_wide_pair_track_workload_full_output(direction):
    """B = 2, N = 768, c_z = 384: every output element against the oracle (about 1.2 TFLOP
    of fp64 work per direction on the host)."""
    name = "n768_cz384_c128_b2_bf16"
    note(f"workload {name} {direction} full")
    d = make_workload(name, seed=0)
    err, _, _ = check_full(d, "bf16", direction)
    print(f"{name} {direction}: rel err {err:.3e}")


def _line_set(rng, n, valid=None):
    """Complete rows and columns that pass through every tile of the contraction, 256 rows
    by 128 or 256 columns (one random row per 256 rows, one random column per 128
    columns), plus the first and last residue and, when padded, both sides of the valid
    boundary."""
    rows = [int(rng.integers(r, min(n, r + 256))) for r in range(0, n, 256)]
    cols = [int(rng.integers(c0, min(n, c0 + 128))) for c0 in range(0, n, 128)]
    edge = [0, n - 1] + ([valid - 1, valid] if valid is not None and valid < n else [])
    return sorted(set(rows + edge)), sorted(set(cols + edge))


def _check_lines(name_or_d, spec, plan_check=None, label=""):
    d = make_workload(name_or_d, seed=0) if isinstance(name_or_d, str) else name_or_d
    B, n, c_z, c, dtype = spec["batch"], spec["n"], spec["c_z"], spec["c"], spec["dtype"]
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    z = torch.from_numpy(d["z"]).to(dt)
    m = torch.from_numpy(d["mask"]).to(dt)
    mod = TriMul(d["weights"], c_z, c, dtype)
    if plan_check:
        plan_check(mod.plan(B, n))
    rng = np.random.default_rng(7)
    lines = [_line_set(rng, n, d.get("meta", {}).get("valid_length")) for _ in range(B)]
    got = {}
    zc, mc = z.cuda(), m.cuda()
    ws = mod.new_workspace(B, n)
    for direction in DIRS:
        note(f"{label} {direction} lines")
        out = mod.forward(zc, mc, direction=direction, workspace=ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all().item())
        for b, (rows, cols) in enumerate(lines):
            got[direction, b] = (out[b, rows].double().cpu().numpy(),
                                 out[b][:, cols].double().cpu().numpy())
        del out
    del zc, mc, ws
    torch.cuda.synchronize()
    zh, mh = z.double().numpy(), m.double().numpy()
    for b, (rows, cols) in enumerate(lines):
        ops = line_operands(zh, mh, d["weights"], b)  # both directions share a and b
        for direction in DIRS:
            want_r, want_c = tri_mul_ref_lines(zh, mh, d["weights"], direction, b, rows, cols,
                                               operands=ops)
            got_r, got_c = got[direction, b]
            scale = max(np.abs(want_r).max(), np.abs(want_c).max())
            err = max(np.abs(got_r - want_r).max(), np.abs(got_c - want_c).max()) / scale
            print(f"{label} {direction} b={b}: {len(rows)} rows, {len(cols)} cols, "
                  f"rel err {err:.3e}")
            assert err <= TOL[dtype]
        del ops


def test_large_complex_workload_lines():
    """N = 2048 (chains 900/700/448, all valid): complete output rows and columns through
    every contraction tile, both directions, in the benchmark's launch configuration."""
    name = "n2048_cz128_c128_bf16_chains"
    _check_lines(name, WORKLOADS[name], label=name)


def test_operands_over_2gib_take_the_64bit_forms():
    """N = 2900, c_z = c = 128, bf16: one batch item's z (2.15 GB) and x plane set (2.4 GB)
    exceed the 32-bit lane offsets of the wave-independent forms, so both projection kernels
    run their tile-shared forms with 64-bit indexing. Complete lines, both directions."""
    spec = {"batch": 1, "n": 2900, "c_z": 128, "c": 128, "dtype": "bf16"}
    d = make_random(1, 2900, 128, 128, seed=29, mask="ones")

    def plan_check(p):
        assert p["input_form"] == 1 and p["output_form"] == 1, p

    _check_lines(d, spec, plan_check, label="n2900 over 2 GiB")


def test_headline_padding_is_zero():
    name = "n512_cz128_c128_bf16_masked"
    d = make_workload(name, seed=0)
    L = d["meta"]["valid_length"]
    for direction in DIRS:
        note(f"headline padding {direction}")
        got, _, _, _ = run_full(d, "bf16", direction)
        assert np.all(got[:, L:, :, :] == 0) and np.all(got[:, :, L:, :] == 0)


# --- ragged sizes, widths, masks, batches -----------------------------------------------------

RAGGED = [
    # batch, n, c_z, c, mask
    (1, 1, 16, 16, "ones"), (2, 7, 16, 32, "random_pairs"), (1, 33, 32, 16, "block"),
    (2, 100, 48, 32, "random_residues"), (1, 130, 64, 48, "random_pairs"),
    (1, 129, 128, 128, "block"), (3, 64, 32, 64, "ones"),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("direction", DIRS)
@pytest.mark.parametrize("batch,n,c_z,c,mask", RAGGED)
def test_ragged_full_output(batch, n, c_z, c, mask, direction, dtype):
    note(f"ragged B={batch} n={n} cz={c_z} c={c} {mask} {direction} {dtype}")
    d = make_random(batch, n, c_z, c, seed=n + c_z, mask=mask, random_affine=True)
    check_full(d, dtype, direction)


# Four chunk groups along c_z (97..128 channels in bf16, 49..64 in fp32) with at least two
# 64-pair tiles per wave of a full grid select the wave-independent input-gate kernel:
# ragged row ends (n < n_pad), batch items past the first, both storage types.
@pytest.mark.parametrize("direction", DIRS)
@pytest.mark.parametrize("dtype,batch,n,c_z,c,mask", [
    ("bf16", 1, 450, 128, 128, "random_pairs"), ("fp32", 1, 450, 64, 32, "block"),
    ("bf16", 2, 300, 112, 64, "random_residues"),
])
def test_wave_input_gate_ragged_full_output(dtype, batch, n, c_z, c, mask, direction):
    note(f"wave input gate {dtype} B={batch} n={n} cz={c_z} c={c} {mask} {direction}")
    d = make_random(batch, n, c_z, c, seed=n + c_z, mask=mask, random_affine=True)
    check_full(d, dtype, direction)


@pytest.mark.parametrize("direction", DIRS)
@pytest.mark.parametrize("batch,n,c_z,c,mask", [
    (1, 70, 64, 512, "random_pairs"), (1, 50, 384, 256, "block"), (2, 33, 512, 384, "ones"),
])
def test_wide_bf16_full_output(batch, n, c_z, c, mask, direction):
    note(f"wide bf16 B={batch} n={n} cz={c_z} c={c} {mask} {direction}")
    d = make_random(batch, n, c_z, c, seed=n + c, mask=mask, random_affine=True)
    check_full(d, "bf16", direction)


@pytest.mark.parametrize("direction", DIRS)
def test_widest_fp32_full_output(direction):
    note(f"widest fp32 {direction}")
    d = make_random(1, 45, 256, 128, seed=77, mask="random_pairs", random_affine=True)
    check_full(d, "fp32", direction)


@pytest.mark.parametrize("dtype,B,n,c_z,c,forms", [
    ("bf16", 1, 450, 128, 128, (0, 0)),   # both projection kernels wave-independent
    ("bf16", 1, 129, 128, 128, (1, 0)),   # tile-shared input gate, wave-independent output
    ("bf16", 2, 70, 128, 512, (1, 1)),    # both tile-shared
    ("bf16", 1, 75, 384, 128, (1, 2)),    # streamed output-gate weights
    ("fp32", 1, 450, 64, 32, (0, 0)),
    ("fp32", 1, 45, 256, 128, (1, 1)),
])
def test_writes_nothing_outside_out_and_workspace(dtype, B, n, c_z, c, forms):
    """out and the workspace sit inside larger buffers filled with a byte pattern, at a
    ragged n (partial last tiles in every kernel): nothing before or after them may
    change, z and the mask must be left as they were, and out must still match the
    oracle. Both directions, with and without the residual add."""
    d = make_random(B, n, c_z, c, seed=n + c, mask="random_pairs", random_affine=True)
    z, m, z_host, m_host = to_device(d, dtype)
    mod = TriMul(d["weights"], c_z, c, dtype)
    plan = mod.plan(B, n)
    assert (plan["input_form"], plan["output_form"]) == forms, plan
    esz = 2 if dtype == "bf16" else 4
    guard = 16384  # bytes on each side (keeps every buffer 16-byte aligned)
    obytes = z.numel() * esz
    obig = torch.full((obytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    out = obig[guard:guard + obytes].view(torch_dtype(dtype)).view_as(z)
    wsb = mod.workspace_bytes(B, n)
    wbig = torch.full((wsb + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = wbig[guard:guard + wsb]
    z0, m0 = z.clone(), m.clone()
    for direction in DIRS:
        want = tri_mul_ref(z_host, m_host, d["weights"], direction)
        for residual in (False, True):
            note(f"guard bands {dtype} B={B} n={n} c_z={c_z} c={c} {direction} "
                 f"residual={residual}")
            if residual:
                mod.forward_residual(z, m, out=out, direction=direction, workspace=ws)
            else:
                mod.forward(z, m, out=out, direction=direction, workspace=ws)
            torch.cuda.synchronize()
            assert torch.all(obig[:guard] == 0x5A) and torch.all(obig[guard + obytes:] == 0x5A)
            assert torch.all(wbig[:guard] == 0xA5) and torch.all(wbig[guard + wsb:] == 0xA5)
            assert torch.equal(z, z0) and torch.equal(m, m0)
            got = out.to(torch.float64).cpu().numpy()
            if residual:
                check_residual_update(got, z_host, want, dtype)
            else:
                assert rel_err(got, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_null_mask_means_all_ones(dtype):
    d = make_random(1, 40, 32, 32, seed=5, mask="ones")
    note(f"null mask {dtype}")
    got_null, z_host, _, mod = run_full(d, dtype, "incoming", use_mask=False)
    got_ones, _, _, _ = run_full(d, dtype, "incoming", use_mask=True, module=mod)
    assert np.array_equal(got_null, got_ones)


@pytest.mark.parametrize("shift", [3.0, -5.0])
def test_nonzero_mean_input_folded_layernorm(shift):
    """The kernels apply LayerNorm after the projection (folded weights); inputs
    with a large common offset must stay within tolerance."""
    d = make_random(1, 48, 64, 32, seed=9, mask="random_pairs", z_shift=shift)
    note(f"nonzero mean {shift}")
    for dtype in ("fp32", "bf16"):
        check_full(d, dtype, "outgoing")


# --- intermediates through the documented workspace layout ----------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("direction", DIRS)
def test_intermediates_in_workspace(direction, dtype):
    batch, n, c_z, c = 2, 37, 32, 48
    d = make_random(batch, n, c_z, c, seed=3, mask="random_pairs")
    z, m, z_host, m_host = to_device(d, dtype)
    note(f"intermediates {direction} {dtype}")
    mod = TriMul(d["weights"], c_z, c, dtype)
    ws = mod.new_workspace(batch, n)
    out = mod.forward(z, m, direction=direction, workspace=ws)
    torch.cuda.synchronize()
    A, Bm, X = (v.to(torch.float64).cpu().numpy() for v in mod.workspace_views(ws, batch, n))
    it = tri_mul_intermediates(z_host, m_host, d["weights"], direction)
    a_ref = np.moveaxis(it["a"], -1, 1)  # [B, c, N, N]
    b_ref = np.moveaxis(it["b"], -1, 1)
    if direction == "incoming":
        a_ref, b_ref = np.swapaxes(a_ref, -1, -2), np.swapaxes(b_ref, -1, -2)
    tol = TOL[dtype]
    assert rel_err(A[:, :, :n, :n], a_ref) <= tol
    assert rel_err(Bm[:, :, :n, :n], b_ref) <= tol
    assert np.all(A[:, :, n:, :] == 0) and np.all(A[:, :, :, n:] == 0)
    assert np.all(Bm[:, :, n:, :] == 0) and np.all(Bm[:, :, :, n:] == 0)
    assert rel_err(X[:, :, :n, :n], np.moveaxis(it["x"], -1, 1)) <= tol
    assert rel_err(out.to(torch.float64).cpu().numpy(), it["out"]) <= tol


def test_stages_in_order_equal_forward():
    d = make_random(1, 70, 32, 32, seed=4, mask="block")
    z, m, _, _ = to_device(d, "bf16")
    note("stages vs forward")
    mod = TriMul(d["weights"], 32, 32, "bf16")
    ws = mod.new_workspace(1, 70)
    full = mod.forward(z, m, direction="incoming", workspace=ws).clone()
    out = torch.empty_like(z)
    for s in (1, 2, 3):
        mod.stage(s, z, m, out=out, direction="incoming", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(full, out)


# --- identities on the GPU ----------------------------------------------------------------------

def _swap_ab(w):
    s = dict(w)
    for part in ("gate", "proj"):
        s[f"w_a_{part}"], s[f"w_b_{part}"] = w[f"w_b_{part}"], w[f"w_a_{part}"]
        s[f"b_a_{part}"], s[f"b_b_{part}"] = w[f"b_b_{part}"], w[f"b_a_{part}"]
    return s


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_transpose_identity_two_handles(dtype):
    """incoming(z, m; W_a, W_b) == outgoing(z^T, m^T; W_b, W_a)^T."""
    d = make_random(1, 90, 32, 32, seed=6, mask="random_pairs")
    z, m, _, _ = to_device(d, dtype)
    note(f"transpose identity {dtype}")
    inc = TriMul(d["weights"], 32, 32, dtype).forward(z, m, direction="incoming")
    zt = z.transpose(1, 2).contiguous()
    mt = m.transpose(1, 2).contiguous()
    out_t = TriMul(_swap_ab(d["weights"]), 32, 32, dtype).forward(zt, mt, direction="outgoing")
    torch.cuda.synchronize()
    err = rel_err(inc.double().cpu().numpy(), out_t.transpose(1, 2).double().cpu().numpy())
    assert err <= TOL[dtype] / 4


def test_crop_invariance_on_gpu():
    n, L = 150, 97
    d = make_random(1, n, 32, 32, seed=8, mask="block", valid=[L])
    z, m, _, _ = to_device(d, "bf16")
    note("crop invariance")
    mod = TriMul(d["weights"], 32, 32, "bf16")
    for direction in DIRS:
        full = mod.forward(z, m, direction=direction)
        crop = mod.forward(z[:, :L, :L].contiguous(), None, direction=direction)
        torch.cuda.synchronize()
        err = rel_err(full[:, :L, :L].double().cpu().numpy(), crop.double().cpu().numpy())
        assert err <= 1e-2
        assert torch.all(full[:, L:] == 0) and torch.all(full[:, :, L:] == 0)


def test_deterministic_and_stream_safe():
    d = make_workload("n256_cz128_c128_bf16", seed=0)
    z, m, _, _ = to_device(d, "bf16")
    note("determinism / side stream")
    mod = TriMul(d["weights"], 128, 128, "bf16")
    first = mod.forward(z, m, direction="outgoing")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        second = mod.forward(z, m, direction="outgoing")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


# --- argument validation on a real handle ------------------------------------------------------

def test_forward_rejects_bad_calls():
    from pair_rep_triangle_amd.trimul import TriMulError
    d = make_random(1, 24, 16, 16, seed=1)
    z, m, _, _ = to_device(d, "bf16")
    note("validation")
    mod = TriMul(d["weights"], 16, 16, "bf16")
    lib, h = mod.lib, mod._h
    ws = mod.new_workspace(1, 24)
    wsb = ws.numel()
    out = torch.empty_like(z)
    st = torch.cuda.current_stream().cuda_stream
    zp, mp, op, wp = z.data_ptr(), m.data_ptr(), out.data_ptr(), ws.data_ptr()
    assert lib.tri_mul_forward(h, zp, mp, op, 1, 24, 0, wp, wsb, st) == 0
    assert lib.tri_mul_forward(h, zp, mp, op, 1, 24, 2, wp, wsb, st) == -1   # direction
    assert lib.tri_mul_forward(h, zp, mp, op, 0, 24, 0, wp, wsb, st) == -1   # batch
    assert lib.tri_mul_forward(h, zp, mp, op, 1, 0, 0, wp, wsb, st) == -1    # n
    assert lib.tri_mul_forward(h, None, mp, op, 1, 24, 0, wp, wsb, st) == -1
    assert lib.tri_mul_forward(h, zp + 2, mp, op, 1, 24, 0, wp, wsb, st) == -4
    assert lib.tri_mul_forward(h, zp, mp, op, 1, 24, 0, wp, wsb - 16, st) == -6
    assert lib.tri_mul_forward(h, zp, mp, zp, 1, 24, 0, wp, wsb, st) == -5   # out == z
    assert lib.tri_mul_forward(h, zp, mp, op, 1, 24, 0, op, wsb, st) == -5   # ws over out
    assert lib.tri_mul_forward_stage(h, 4, zp, mp, op, 1, 24, 0, wp, wsb, st) == -1
    with pytest.raises(TriMulError):
        mod.forward(z, m, direction="incoming", workspace=ws[:16])
    # host tensors are refused by the binding before anything is launched
    with pytest.raises(ValueError):
        mod.forward(z, m.cpu())
    with pytest.raises(ValueError):
        mod.forward(z, m, out=torch.empty(z.shape, dtype=z.dtype))
    with pytest.raises(ValueError):
        mod.forward(z, m, workspace=torch.empty(wsb, dtype=torch.uint8))
    torch.cuda.synchronize()


def test_temporary_workspace_is_kept_for_a_side_stream():
    """A forward call on another stream without a workspace: the binding's temporary
    workspace (allocated on the current stream) must not be handed out again to the
    current stream while the side stream may still use it."""
    d = make_random(1, 200, 64, 64, seed=12, mask="random_pairs")
    z, m, _, _ = to_device(d, "bf16")
    note("temporary workspace on a side stream")
    mod = TriMul(d["weights"], 64, 64, "bf16")
    ref = mod.forward(z, m, direction="outgoing")
    torch.cuda.synchronize()
    taken = []
    plain = mod.new_workspace

    def recording(*args, **kw):
        t = plain(*args, **kw)
        taken.append(t.data_ptr())
        return t

    mod.new_workspace = recording
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)  # keeps the side stream busy past the next allocation
    out = torch.empty_like(z)
    torch.cuda.current_stream().synchronize()
    mod.forward(z, m, out=out, direction="outgoing", stream=side.cuda_stream)
    again = torch.empty(mod.workspace_bytes(1, 200), dtype=torch.uint8, device="cuda")
    assert len(taken) == 1 and again.data_ptr() != taken[0]
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
