"""Builds libtrimul.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m pair_rep_triangle_amd.build              # the library
    python -m pair_rep_triangle_amd.build --sanitize   # host code with ASan + UBSan

The library lands next to this file; the Python binding loads it from there. The
sanitized build holds the host code only (argument checks, weight folding and LDS image
building, plans, launch set-up), instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer; it lands in _build_san/ and serves the CPU tests, run with
the sanitizer runtime preloaded (tests/test_host_sanitizers.py does that).
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
# accumulation registers for each use. Their scores hold no NaN (masked keys are -inf), so
# the maxima of the softmax need no quieting of signalling NaNs first.
EXTRA = {"ka_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"]}


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


# Host-only objects (no device code) with both sanitizers; a UBSan report is fatal.
SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libtrimul_san.so")
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "--cuda-host-only",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Wall", "-Wno-unused-function",
             f"-I{INCLUDE}", f"-I{CSRC}"]


def sanitizer_runtime():
    """The compiler's shared AddressSanitizer runtime (to preload into Python)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_sanitized(verbose=True):
    """Link _build_san/libtrimul_san.so: the host-only sources (the C-ABI entry points,
    weight folding, image building, plans and argument checks) compiled with ASan +
    UBSan, and the kernel sources as in the plain build (their objects from _build/,
    compiled first if missing)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor
    jobs, objs = [], []
    for src in SOURCES:
        if src.endswith(".cpp"):
            obj = os.path.join(SAN_DIR, src + ".o")
            jobs.append([HIPCC, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            obj = os.path.join(objdir, src + ".o")
            if not os.path.exists(obj):
                jobs.append([HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                             "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8) or 1) as ex:
        list(ex.map(_run, jobs))
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, *objs])
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
