"""The allocation-free entry point (tri_mul_forward_static) through the C ABI: its output
must equal tri_mul_forward's with a caller workspace, byte for byte (same kernels, same
inputs), and match the fp64 oracle; two calls in a row, the second on a smaller input,
so the second runs on the array the first left behind. Sizes beyond the array are
rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import tri_mul_ref
from pair_rep_triangle_amd.inputs import make_random, make_workload
from pair_rep_triangle_amd.trimul import TriMul
from tests.gpu_util import TOL, note, rel_err, to_device

pytestmark = pytest.mark.gpu

STATIC_BYTES = 256 * 1024 * 1024  # TRI_MUL_STATIC_WORKSPACE_BYTES


def _static(mod, z, m, out, direction):
    st = torch.cuda.current_stream().cuda_stream
    B, n = z.shape[0], z.shape[1]
    return mod.lib.tri_mul_forward_static(mod._h, z.data_ptr(), None if m is None else m.data_ptr(),
                                          out.data_ptr(), B, n, {"outgoing": 0, "incoming": 1}[direction],
                                          st)


def _with_workspace(mod, z, m, out, direction):
    B, n = z.shape[0], z.shape[1]
    ws = mod.new_workspace(B, n)
    st = torch.cuda.current_stream().cuda_stream
    rc = mod.lib.tri_mul_forward(mod._h, z.data_ptr(), None if m is None else m.data_ptr(),
                                 out.data_ptr(), B, n, {"outgoing": 0, "incoming": 1}[direction],
                                 ws.data_ptr(), ws.numel(), st)
    torch.cuda.synchronize()
    return rc


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_static_workspace_matches_caller_workspace(direction):
    big = make_workload("n512_cz128_c128_bf16_masked", seed=0)      # 192 MiB of workspace
    small = make_random(1, 77, 128, 128, seed=3, mask="random_pairs")  # a smaller second call
    mod = TriMul(big["weights"], 128, 128, "bf16")
    for label, d in (("n512 masked", big), ("n77 after n512", small)):
        note(f"static workspace {direction} {label}")
        if label.startswith("n77"):
            mod = TriMul(d["weights"], 128, 128, "bf16")
        z, m, z_host, m_host = to_device(d, "bf16")
        got = torch.empty_like(z)
        assert _static(mod, z, m, got, direction) == 0
        torch.cuda.synchronize()
        want = torch.empty_like(z)
        assert _with_workspace(mod, z, m, want, direction) == 0
        assert torch.equal(got, want)
        ref = tri_mul_ref(z_host, m_host, d["weights"], direction)
        err = rel_err(got.to(torch.float64).cpu().numpy(), ref)
        print(f"static {direction} {label}: rel err {err:.3e}")
        assert err <= TOL["bf16"]


def test_static_workspace_fp32_and_null_mask():
    d = make_random(2, 45, 32, 32, seed=4, mask="ones")
    z, _, z_host, _ = to_device(d, "fp32")
    mod = TriMul(d["weights"], 32, 32, "fp32")
    note("static workspace fp32, null mask")
    got = torch.empty_like(z)
    assert _static(mod, z, None, got, "incoming") == 0
    torch.cuda.synchronize()
    want = torch.empty_like(z)
    assert _with_workspace(mod, z, None, want, "incoming") == 0
    assert torch.equal(got, want)
    assert rel_err(got.double().cpu().numpy(), tri_mul_ref(z_host, None, d["weights"], "incoming")) <= TOL["fp32"]


def test_static_workspace_rejects_sizes_beyond_the_array():
    d = make_random(1, 8, 128, 128, seed=1)
    mod = TriMul(d["weights"], 128, 128, "bf16")
    note("static workspace size limit")
    # n = 600 pads to 640: 3 * 128 * 640^2 * 2 bytes = 300 MiB > 256 MiB (576 fits)
    assert mod.workspace_bytes(1, 600) > STATIC_BYTES >= mod.workspace_bytes(1, 576)
    z = torch.zeros((1, 600, 600, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(z, 3.0)
    assert _static(mod, z, None, out, "outgoing") == -6  # TRI_MUL_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)  # nothing ran
    assert _static(mod, z, None, z, "outgoing") in (-5, -6)
