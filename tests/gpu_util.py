"""Helpers shared by the GPU tests: move a seeded case to the device, run the
HIP path through the C ABI, and compare with the fp64 oracle."""

import sys

import numpy as np
import torch

from oracle import tri_mul_ref, tri_mul_ref_pairs, tri_mul_intermediates
from pair_rep_triangle_amd.trimul import TriMul

TOL = {"fp32": 1e-4, "bf16": 2e-2}  # max |gpu - ref| / max |ref|


def note(msg):
    """Print (and flush) what the next GPU step is, so a failing run names its case."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(d, dtype):
    """z, mask as device tensors in the storage dtype, plus the exact values the
    device holds (as float64 NumPy) for the oracle."""
    dt = torch_dtype(dtype)
    z = torch.from_numpy(d["z"]).to(dt)
    m = torch.from_numpy(d["mask"]).to(dt)
    z_host = z.to(torch.float64).numpy()
    m_host = m.to(torch.float64).numpy()
    return z.cuda(), m.cuda(), z_host, m_host


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = np.abs(want).max()
    return float(np.abs(got - want).max() / (scale if scale > 0 else 1.0))


def storage_round(x, dtype):
    """x (float64) rounded to the storage type, as float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch_dtype(dtype)).to(torch.float64).numpy()


def storage_ulp(x, dtype):
    """The spacing of the storage type at |x| (8 significand bits for bf16, 24 for fp32)."""
    bits = 8 if dtype == "bf16" else 24
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - (bits - 1))


def check_residual_update(got, z_host, upd_ref, dtype, tol=None):
    """A residual output got = round(z + u) against the oracle's update u_ref: every element
    within tol * max|u_ref| of round(z + u_ref), plus one unit of the storage type at
    z + u_ref for the final rounding. This holds the computed update itself to the
    tolerance, whatever the size of z."""
    want = np.asarray(z_host, np.float64) + upd_ref
    rounded = storage_round(want, dtype)
    unit = np.maximum(storage_ulp(want, dtype), storage_ulp(rounded, dtype))
    bound = (tol or TOL[dtype]) * np.abs(upd_ref).max() + unit
    excess = np.abs(np.asarray(got, np.float64) - rounded) - bound
    worst = float(excess.max())
    assert worst <= 0, (f"update off by {worst:.3e} beyond tol * max|u_ref| + 1 ulp "
                        f"(max|u_ref| {np.abs(upd_ref).max():.3e})")
    return float((np.abs(got - rounded) / np.abs(upd_ref).max()).max())


def run_full(d, dtype, direction, use_mask=True, module=None):
    z, m, z_host, m_host = to_device(d, dtype)
    c_z, c = d["z"].shape[-1], d["weights"]["w_a_gate"].shape[0]
    mod = module or TriMul(d["weights"], c_z, c, dtype)
    out = mod.forward(z, m if use_mask else None, direction=direction)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    return got, z_host, (m_host if use_mask else None), mod


def check_full(d, dtype, direction, use_mask=True, tol=None):
    got, z_host, m_host, _ = run_full(d, dtype, direction, use_mask)
    want = tri_mul_ref(z_host, m_host, d["weights"], direction)
    err = rel_err(got, want)
    assert np.isfinite(got).all(), "non-finite output"
    assert err <= (tol or TOL[dtype]), f"rel err {err:.3e} > {tol or TOL[dtype]:.1e}"
    return err, got, want


def sample_pairs(rng, batch, n, count, valid=None):
    v = n if valid is None else valid
    bi = rng.integers(0, batch, count)
    ii = rng.integers(0, n, count)
    jj = rng.integers(0, n, count)
    # always include the corners and, when padded, the first padded row / column
    extra = [(0, 0, 0), (batch - 1, n - 1, n - 1), (0, 0, n - 1), (0, n - 1, 0),
             (0, v - 1, v - 1)]
    if v < n:
        extra += [(0, v, 0), (0, 0, v), (0, v - 1, v)]
    bi = np.concatenate([bi, [e[0] for e in extra]])
    ii = np.concatenate([ii, [e[1] for e in extra]])
    jj = np.concatenate([jj, [e[2] for e in extra]])
    return bi, ii, jj


__all__ = ["TOL", "note", "to_device", "rel_err", "run_full", "check_full", "sample_pairs",
           "storage_round", "storage_ulp", "check_residual_update",
           "tri_mul_ref", "tri_mul_ref_pairs", "tri_mul_intermediates", "TriMul", "torch_dtype"]
