"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol include/tri_mul.h, include/pair_transition.h and include/tri_attention.h
declare, and rejects bad create arguments before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

from pair_rep_triangle_amd import trimul as tm
from pair_rep_triangle_amd.inputs import (make_attention_weights, make_transition_weights,
                                          make_weights)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="tri_mul.h", prefix="tri_mul_"):
    with open(os.path.join(ROOT, "include", header)) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(" + prefix + r"[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return tm.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(tm.EXPORTS)


def test_transition_header_declares_the_entry_points():
    assert _declared_functions("pair_transition.h", "pair_transition_") == sorted(tm.TRANSITION_EXPORTS)


def test_attention_header_declares_the_entry_points():
    assert _declared_functions("tri_attention.h", "tri_attn_") == sorted(tm.ATTENTION_EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in (_declared_functions() + _declared_functions("pair_transition.h", "pair_transition_")
                 + _declared_functions("tri_attention.h", "tri_attn_")):
        assert hasattr(lib, name), name


def test_mask_extents_rejects_bad_arguments_before_touching_the_device(lib):
    buf = ctypes.c_void_p(64)
    assert lib.tri_mul_mask_extents(7, buf, 1, 16, buf, None) == -2   # dtype
    assert lib.tri_mul_mask_extents(1, None, 1, 16, buf, None) == -1  # no mask
    assert lib.tri_mul_mask_extents(1, buf, 0, 16, buf, None) == -1   # batch
    assert lib.tri_mul_mask_extents(1, buf, 1, 0, buf, None) == -1    # n


def test_forward_extents_rejects_a_null_handle(lib):
    buf = ctypes.c_void_p(64)
    assert lib.tri_mul_forward_extents(None, buf, None, buf, buf, 1, 16, 0, 0, buf, 1 << 20,
                                       None) == -1


def test_query_plan_rejects_bad_arguments(lib):
    plan = tm.Plan()
    assert lib.tri_mul_query_plan(None, 1, 16, ctypes.byref(plan)) == -1


def test_strerror_covers_every_code(lib):
    for code in tm.ERRORS:
        msg = lib.tri_mul_strerror(code).decode()
        assert msg and msg != "unknown error code"
    assert lib.tri_mul_strerror(12345).decode() == "unknown error code"


def _weights_struct(w):
    keep = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in w.items()}
    s = tm.Weights()
    for k, v in keep.items():
        setattr(s, k, v.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return s, keep


@pytest.mark.parametrize("c_z,c,dtype,code", [
    (24, 16, tm.TRI_MUL_BF16, -2), (16, 40, tm.TRI_MUL_BF16, -2), (528, 16, tm.TRI_MUL_BF16, -2),
    (16, 528, tm.TRI_MUL_BF16, -2), (272, 16, tm.TRI_MUL_FP32, -2), (16, 144, tm.TRI_MUL_FP32, -2),
    (16, 16, 7, -2), (0, 16, tm.TRI_MUL_FP32, -1), (16, -16, tm.TRI_MUL_FP32, -1),
])
def test_create_rejects_bad_shapes_before_touching_the_device(lib, c_z, c, dtype, code):
    w = make_weights(np.random.default_rng(0), max(c_z, 1), max(c, 1))
    s, keep = _weights_struct(w)
    h = ctypes.c_void_p(1)
    assert lib.tri_mul_create(ctypes.byref(s), c_z, c, dtype, ctypes.byref(h)) == code
    assert h.value is None


def test_create_requires_weight_matrices(lib):
    w = make_weights(np.random.default_rng(0), 16, 16)
    del w["w_gate"]
    s, keep = _weights_struct(w)
    h = ctypes.c_void_p()
    assert lib.tri_mul_create(ctypes.byref(s), 16, 16, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    assert lib.tri_mul_create(None, 16, 16, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    assert lib.tri_mul_create(ctypes.byref(s), 16, 16, tm.TRI_MUL_BF16, None) == -1


def test_null_handle_is_rejected(lib):
    n = ctypes.c_size_t()
    assert lib.tri_mul_workspace_bytes(None, 1, 8, ctypes.byref(n)) == -1
    assert lib.tri_mul_workspace_layout(None, 1, 8, None) == -1
    assert lib.tri_mul_forward(None, 16, 16, 32, 1, 8, 0, 48, 1 << 20, None) == -1
    assert lib.tri_mul_forward_stage(None, 1, 16, 16, 32, 1, 8, 0, 48, 1 << 20, None) == -1
    lib.tri_mul_destroy(None)  # no-op


def test_binding_raises_with_a_named_error():
    with pytest.raises(tm.TriMulError) as ei:
        tm.TriMul(make_weights(np.random.default_rng(0), 16, 16), 20, 16, "bf16")
    assert ei.value.name == "UNSUPPORTED"


def _transition_struct(w):
    keep = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in w.items()}
    s = tm.TransitionWeights()
    for k, v in keep.items():
        setattr(s, k, v.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return s, keep


@pytest.mark.parametrize("c_z,hidden,dtype,code", [
    (48, 96, tm.TRI_MUL_BF16, -2), (544, 1088, tm.TRI_MUL_BF16, -2), (512, 8192, tm.TRI_MUL_BF16, -2),
    (24, 48, tm.TRI_MUL_FP32, -2), (128, 256, tm.TRI_MUL_FP32, -2), (64, 64, 9, -2),
    (0, 64, tm.TRI_MUL_BF16, -1), (64, 0, tm.TRI_MUL_BF16, -1),
])
def test_transition_create_rejects_bad_shapes(lib, c_z, hidden, dtype, code):
    w = make_transition_weights(np.random.default_rng(0), max(c_z, 1), max(hidden, 1))
    s, keep = _transition_struct(w)
    h = ctypes.c_void_p(1)
    assert lib.pair_transition_create(ctypes.byref(s), c_z, hidden, dtype, ctypes.byref(h)) == code
    assert h.value is None


def test_transition_null_arguments(lib):
    w = make_transition_weights(np.random.default_rng(0), 64, 128)
    s, keep = _transition_struct(w)
    h = ctypes.c_void_p()
    assert lib.pair_transition_create(None, 64, 128, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    assert lib.pair_transition_create(ctypes.byref(s), 64, 128, tm.TRI_MUL_BF16, None) == -1
    s.w2 = None
    assert lib.pair_transition_create(ctypes.byref(s), 64, 128, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    assert lib.pair_transition_forward(None, 16, None, 32, 1, 8, None) == -1
    lib.pair_transition_destroy(None)  # no-op


def _attention_struct(w):
    keep = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in w.items()}
    s = tm.AttentionWeights()
    for k, v in keep.items():
        setattr(s, k, v.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return s, keep


@pytest.mark.parametrize("c_z,heads,d,dtype,code", [
    (48, 4, 32, tm.TRI_MUL_BF16, -2), (176, 4, 32, tm.TRI_MUL_BF16, -2),
    (416, 4, 32, tm.TRI_MUL_BF16, -2), (64, 9, 32, tm.TRI_MUL_BF16, -2),
    (128, 4, 16, tm.TRI_MUL_BF16, -2), (128, 4, 32, tm.TRI_MUL_FP32, -2),
    (0, 4, 32, tm.TRI_MUL_BF16, -1), (64, 0, 32, tm.TRI_MUL_BF16, -1),
])
def test_attention_create_rejects_bad_shapes(lib, c_z, heads, d, dtype, code):
    w = make_attention_weights(np.random.default_rng(0), max(c_z, 1), max(heads, 1), max(d, 1))
    s, keep = _attention_struct(w)
    h = ctypes.c_void_p(1)
    assert lib.tri_attn_create(ctypes.byref(s), c_z, heads, d, dtype, ctypes.byref(h)) == code
    assert h.value is None


def test_attention_null_arguments(lib):
    w = make_attention_weights(np.random.default_rng(0), 64, 2, 32)
    s, keep = _attention_struct(w)
    h = ctypes.c_void_p()
    assert lib.tri_attn_create(None, 64, 2, 32, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    assert lib.tri_attn_create(ctypes.byref(s), 64, 2, 32, tm.TRI_MUL_BF16, None) == -1
    s.w_o = None
    assert lib.tri_attn_create(ctypes.byref(s), 64, 2, 32, tm.TRI_MUL_BF16, ctypes.byref(h)) == -1
    n = ctypes.c_size_t()
    assert lib.tri_attn_workspace_bytes(None, 1, 8, ctypes.byref(n)) == -1
    assert lib.tri_attn_forward(None, 16, None, 32, 1, 8, 0, 48, 1 << 20, None) == -1
    lib.tri_attn_destroy(None)  # no-op
