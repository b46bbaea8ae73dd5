"""Device assembly checks of every kernel source (CPU: hipcc cross-compiles for gfx950).

A buffer descriptor that the compiler keeps in vector registers makes it wrap every load or
store through the descriptor in a loop over the wave's distinct descriptors: a 64-bit
compare of scalar against vector registers, then the access under a narrowed exec mask.
The loop runs once when the descriptor is uniform, but each access then sits in a basic
block of its own, out of reach of the scheduling that interleaves loads with MFMAs (the
contraction kernel lost its load/MFMA overlap this way). No kernel may contain it.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from pair_rep_triangle_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")

HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
WATERFALL = re.compile(r"v_cmp_eq_u64_e(32|64)\s+\S+,\s*s\[\d+:\d+\],\s*v\[\d+:\d+\]")


def _device_asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, *build.COMMON, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_no_descriptor_waterfall_loops(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        asms = list(ex.map(lambda s: _device_asm(s, tmp_path), HIP_SOURCES))
    bad = {src: len(WATERFALL.findall(a)) for src, a in zip(HIP_SOURCES, asms)}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"descriptor loops (count per source): {bad}"
    # the check would see one: the contraction's loads really are buffer loads into LDS
    k2 = asms[HIP_SOURCES.index("k2_contract.hip")]
    assert "buffer_load_dwordx4" in k2 and " lds" in k2
