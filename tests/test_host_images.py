"""The host side of every create call at every supported form, without a GPU.

Each create folds the LayerNorm affine into the weights and builds the kernels' LDS
images on the host before it looks for the device, so on a machine without a GPU a valid
create walks all of that code and then returns TRI_MUL_ERR_HIP (on a GPU it succeeds and
the handle is destroyed again). Run under the sanitized host build
(tests/test_host_sanitizers.py), this is where AddressSanitizer and UBSan watch the
folding and image code of every form: tile-shared and wave-independent input gates,
plain and streamed output gates, both transition forms, the attention images."""

import ctypes

import numpy as np
import pytest

from pair_rep_triangle_amd import trimul as tm
from pair_rep_triangle_amd.inputs import (make_attention_weights, make_transition_weights,
                                          make_weights)


@pytest.fixture(scope="module")
def lib():
    return tm.load_library()


def _struct(cls, w):
    keep = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in w.items()}
    s = cls()
    for k, v in keep.items():
        setattr(s, k, v.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return s, keep


@pytest.mark.parametrize("c_z,c,dtype", [
    (16, 16, tm.TRI_MUL_BF16), (128, 128, tm.TRI_MUL_BF16), (96, 32, tm.TRI_MUL_BF16),
    (128, 512, tm.TRI_MUL_BF16), (384, 128, tm.TRI_MUL_BF16), (320, 96, tm.TRI_MUL_BF16),
    (512, 64, tm.TRI_MUL_BF16), (256, 128, tm.TRI_MUL_BF16), (512, 512, tm.TRI_MUL_BF16),
    (16, 16, tm.TRI_MUL_FP32), (64, 48, tm.TRI_MUL_FP32), (256, 128, tm.TRI_MUL_FP32),
])
def test_tri_mul_create_builds_images(lib, c_z, c, dtype):
    s, keep = _struct(tm.Weights, make_weights(np.random.default_rng(c_z + c), c_z, c,
                                               random_affine=True))
    h = ctypes.c_void_p()
    rc = lib.tri_mul_create(ctypes.byref(s), c_z, c, dtype, ctypes.byref(h))
    assert rc in (0, -7), rc
    if rc == 0:
        lib.tri_mul_destroy(h)
    else:
        assert h.value is None


@pytest.mark.parametrize("c_z,hidden,dtype", [
    (64, 128, tm.TRI_MUL_BF16), (128, 256, tm.TRI_MUL_BF16), (96, 200, tm.TRI_MUL_BF16),
    (384, 768, tm.TRI_MUL_BF16), (256, 512, tm.TRI_MUL_BF16), (160, 100, tm.TRI_MUL_BF16),
    (64, 128, tm.TRI_MUL_FP32), (32, 48, tm.TRI_MUL_FP32),
])
def test_transition_create_builds_images(lib, c_z, hidden, dtype):
    s, keep = _struct(tm.TransitionWeights,
                      make_transition_weights(np.random.default_rng(c_z), c_z, hidden,
                                              random_affine=True))
    h = ctypes.c_void_p()
    rc = lib.pair_transition_create(ctypes.byref(s), c_z, hidden, dtype, ctypes.byref(h))
    assert rc in (0, -7), rc
    if rc == 0:
        lib.pair_transition_destroy(h)


@pytest.mark.parametrize("c_z,heads,d", [(64, 2, 32), (128, 4, 32), (96, 1, 32), (128, 8, 32),
                                          (160, 2, 32), (256, 4, 32), (384, 4, 32),
                                          (384, 8, 32)])
def test_attention_create_builds_images(lib, c_z, heads, d):
    s, keep = _struct(tm.AttentionWeights,
                      make_attention_weights(np.random.default_rng(c_z), c_z, heads, d,
                                             random_affine=True))
    h = ctypes.c_void_p()
    rc = lib.tri_attn_create(ctypes.byref(s), c_z, heads, d, tm.TRI_MUL_BF16, ctypes.byref(h))
    assert rc in (0, -7), rc
    if rc == 0:
        lib.tri_attn_destroy(h)
