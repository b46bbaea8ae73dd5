"""Builds libtrimul.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m pair_rep_triangle_amd.build

The library lands next to this file; the Python binding loads it from there.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtrimul.so")
SOURCES = ("k0_mask_extents.hip", "k1_input_gate.hip", "k2_contract.hip", "k3_output_gate.hip", "k3_stream.hip", "kt_transition.hip", "kt_transition_wide.hip",
           "ka_attention.hip", "tri_mul.cpp", "tri_mul_static.hip", "pair_transition.cpp",
           "tri_attention.cpp")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off: the compiler must not emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source additions. The attention kernels feed every MFMA result to vector ALU work
# (softmax, rescaling); the MFMA forms that write vector registers avoid a copy out of the
# accumulation registers for each use.
EXTRA = {"ka_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose=True):
    """Compile every source and link libtrimul.so (always recompiles)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor
    objs = [os.path.join(objdir, src + ".o") for src in SOURCES]
    jobs = [[HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
