"""Python binding of libtrimul.so (ctypes): argument marshalling only.

Every step of the operators runs in the HIP kernels behind the C ABI
(include/tri_mul.h, include/pair_transition.h); PyTorch supplies device memory and
the stream. There is
no other execution path: if the library is missing or the call fails, this
module raises.
"""

import ctypes
import os

import numpy as np

from .inputs import WEIGHT_FIELDS

TRANSITION_FIELDS = ("ln_gamma", "ln_beta", "w1", "b1", "w2", "b2")
ATTENTION_FIELDS = ("ln_gamma", "ln_beta", "w_q", "w_k", "w_v", "w_b", "w_g", "b_g", "w_o",
                    "b_o")
NODES = {"starting": 0, "ending": 1}

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; PAIR_REP_TRIANGLE_LIB names another build of the same library
LIB_PATH = os.environ.get("PAIR_REP_TRIANGLE_LIB") or os.path.join(_HERE, "libtrimul.so")

TRI_MUL_FP32, TRI_MUL_BF16 = 0, 1
DIRECTIONS = {"outgoing": 0, "incoming": 1}
DTYPES = {"fp32": TRI_MUL_FP32, "bf16": TRI_MUL_BF16}
ERRORS = {
    0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "UNSUPPORTED_DEVICE", -4: "ALIGNMENT",
    -5: "ALIAS", -6: "WORKSPACE_TOO_SMALL", -7: "HIP", -8: "OUT_OF_MEMORY",
}
EXPORTS = ("tri_mul_create", "tri_mul_workspace_bytes", "tri_mul_workspace_layout",
           "tri_mul_query_plan", "tri_mul_forward_static", "tri_mul_forward",
           "tri_mul_forward_residual", "tri_mul_forward_stage", "tri_mul_mask_extents",
           "tri_mul_forward_extents", "tri_mul_destroy", "tri_mul_strerror",
           "tri_mul_last_hip_error")
TRANSITION_EXPORTS = ("pair_transition_create", "pair_transition_forward",
                      "pair_transition_destroy")
ATTENTION_EXPORTS = ("tri_attn_create", "tri_attn_workspace_bytes", "tri_attn_forward",
                     "tri_attn_forward_stage", "tri_attn_destroy")


class TriMulError(RuntimeError):
    def __init__(self, code, what, detail=""):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        super().__init__(f"{what}: TRI_MUL_ERR_{self.name} ({code}) {detail}".rstrip())


class Weights(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_float)) for name in WEIGHT_FIELDS]


class TransitionWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_float)) for name in TRANSITION_FIELDS]


class AttentionWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_float)) for name in ATTENTION_FIELDS]


class Plan(ctypes.Structure):
    _fields_ = [("input_form", ctypes.c_int), ("output_form", ctypes.c_int),
                ("output_groups", ctypes.c_int), ("in_place_ok", ctypes.c_int),
                ("n_pad", ctypes.c_int)]


class Layout(ctypes.Structure):
    _fields_ = [("a_offset", ctypes.c_size_t), ("b_offset", ctypes.c_size_t),
                ("x_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t),
                ("n_pad", ctypes.c_int), ("elem_bytes", ctypes.c_int)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libtrimul.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -m pair_rep_triangle_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.tri_mul_create.argtypes = [ctypes.POINTER(Weights), i, i, i, ctypes.POINTER(vp)]
    lib.tri_mul_workspace_bytes.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.tri_mul_workspace_layout.argtypes = [vp, i, i, ctypes.POINTER(Layout)]
    lib.tri_mul_query_plan.argtypes = [vp, i, i, ctypes.POINTER(Plan)]
    lib.tri_mul_forward.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.tri_mul_forward_residual.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.tri_mul_forward_static.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.tri_mul_mask_extents.argtypes = [i, vp, i, i, vp, vp]
    lib.tri_mul_forward_extents.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.tri_mul_forward_stage.argtypes = [vp, i, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.tri_mul_destroy.argtypes = [vp]
    lib.tri_mul_destroy.restype = None
    lib.tri_mul_strerror.argtypes = [i]
    lib.tri_mul_strerror.restype = ctypes.c_char_p
    lib.tri_mul_last_hip_error.argtypes = []
    lib.tri_mul_last_hip_error.restype = ctypes.c_char_p
    lib.pair_transition_create.argtypes = [ctypes.POINTER(TransitionWeights), i, i, i,
                                           ctypes.POINTER(vp)]
    lib.pair_transition_forward.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.pair_transition_destroy.argtypes = [vp]
    lib.tri_attn_create.argtypes = [ctypes.POINTER(AttentionWeights), i, i, i, i,
                                    ctypes.POINTER(vp)]
    lib.tri_attn_workspace_bytes.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.tri_attn_forward.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.tri_attn_forward_stage.argtypes = [vp, i, vp, vp, vp, i, i, i, vp, sz, vp]
    lib.tri_attn_destroy.argtypes = [vp]
    lib.tri_attn_destroy.restype = None
    lib.pair_transition_destroy.restype = None
    for name in ("tri_mul_create", "tri_mul_workspace_bytes", "tri_mul_workspace_layout",
                 "tri_mul_query_plan", "tri_mul_forward_static", "tri_mul_forward",
                 "tri_mul_forward_residual", "tri_mul_forward_stage", "tri_mul_mask_extents",
                 "tri_mul_forward_extents", "pair_transition_create", "pair_transition_forward"):
        getattr(lib, name).restype = i
    _lib = lib
    return lib


def _check(rc, what):
    if rc != 0:
        detail = ""
        if rc == -7:
            detail = "- " + load_library().tri_mul_last_hip_error().decode()
        raise TriMulError(rc, what, detail)


def _check_device(name, t, z):
    """Every buffer of a call must be device memory on z's device: a host pointer handed to
    the kernels is a GPU page fault the C ABI cannot detect."""
    if t is not None and (not t.is_cuda or t.device != z.device):
        raise ValueError(f"{name} must be a CUDA tensor on {z.device}, got {t.device}")


def _keep_for_stream(t, stream, z):
    """A buffer allocated here on the current stream but used on `stream`: mark it used there,
    so the caching allocator does not hand it out again before that stream's work is done."""
    import torch
    if stream != torch.cuda.current_stream(z.device).cuda_stream:
        t.record_stream(torch.cuda.ExternalStream(stream, device=z.device))


def _host_f32(v):
    if hasattr(v, "detach"):
        v = v.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(v, dtype=np.float32))


EXTENT_PARTS = 64  # TRI_MUL_EXTENT_PARTS


def mask_extents(mask, out=None, stream=None):
    """tri_mul_mask_extents: the per-item mask extents of a [B, N, N] bf16 or fp32 CUDA mask,
    as a [B, 64] int32 tensor of partial maxima (the extent of item b is out[b].max()).
    Computed once per model forward and passed to every update that shares the mask."""
    import torch
    lib = load_library()
    if mask.dim() != 3 or mask.shape[1] != mask.shape[2] or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous [B, N, N] tensor")
    if not mask.is_cuda:
        raise ValueError("mask must be a CUDA tensor")
    dt = {torch.bfloat16: TRI_MUL_BF16, torch.float32: TRI_MUL_FP32}.get(mask.dtype)
    if dt is None:
        raise ValueError("mask must be bfloat16 or float32")
    batch, n = int(mask.shape[0]), int(mask.shape[1])
    if out is None:
        out = torch.empty((batch, EXTENT_PARTS), dtype=torch.int32, device=mask.device)
    elif (tuple(out.shape) != (batch, EXTENT_PARTS) or out.dtype != torch.int32
          or not out.is_contiguous() or out.device != mask.device):
        raise ValueError("out must be a contiguous int32 [B, 64] tensor on the mask's device")
    if stream is None:
        stream = torch.cuda.current_stream(mask.device).cuda_stream
    _check(lib.tri_mul_mask_extents(dt, mask.data_ptr(), batch, n, out.data_ptr(), stream),
           "tri_mul_mask_extents")
    return out


class TriMul:
    """One triangle multiplicative update module (one weight set, one dtype).

    weights: mapping with the tri_mul_weights field names, fp32 host arrays in
    nn.Linear orientation (missing gamma -> ones, missing beta / bias -> zeros).
    """

    def __init__(self, weights, c_z, c, dtype="bf16"):
        self.lib = load_library()
        self.c_z, self.c, self.dtype = int(c_z), int(c), dtype
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
        self._keep = {}
        ws = Weights()
        for name in WEIGHT_FIELDS:
            v = weights.get(name) if hasattr(weights, "get") else None
            if v is None:
                continue
            arr = _host_f32(v)
            self._keep[name] = arr
            setattr(ws, name, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        h = ctypes.c_void_p()
        _check(self.lib.tri_mul_create(ctypes.byref(ws), self.c_z, self.c, DTYPES[dtype],
                                       ctypes.byref(h)), "tri_mul_create")
        self._h = h
        self._keep.clear()

    # -- sizes -------------------------------------------------------------------------
    def workspace_bytes(self, batch, n):
        out = ctypes.c_size_t()
        _check(self.lib.tri_mul_workspace_bytes(self._h, batch, n, ctypes.byref(out)),
               "tri_mul_workspace_bytes")
        return out.value

    def layout(self, batch, n):
        lay = Layout()
        _check(self.lib.tri_mul_workspace_layout(self._h, batch, n, ctypes.byref(lay)),
               "tri_mul_workspace_layout")
        return lay

    def plan(self, batch, n):
        """The kernel forms a call of (batch, n) takes (tri_mul_query_plan)."""
        p = Plan()
        _check(self.lib.tri_mul_query_plan(self._h, int(batch), int(n), ctypes.byref(p)),
               "tri_mul_query_plan")
        return {name: getattr(p, name) for name, _ in Plan._fields_}

    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def new_workspace(self, batch, n, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(batch, n), dtype=torch.uint8, device=device)

    def workspace_views(self, ws, batch, n):
        """(a, b, x) views [batch, c, n_pad, n_pad] into a workspace tensor."""
        lay = self.layout(batch, n)
        dt = self.torch_dtype()
        numel = batch * self.c * lay.n_pad * lay.n_pad
        views = []
        for off in (lay.a_offset, lay.b_offset, lay.x_offset):
            views.append(ws[off:off + numel * lay.elem_bytes].view(dt)
                         .view(batch, self.c, lay.n_pad, lay.n_pad))
        return tuple(views)

    # -- calls -------------------------------------------------------------------------
    def _args(self, z, mask, out, workspace, direction, stream, workspace_needed=True):
        import torch
        if z.dim() != 4 or z.shape[1] != z.shape[2] or z.shape[3] != self.c_z:
            raise ValueError(f"z must be [B, N, N, {self.c_z}], got {tuple(z.shape)}")
        if z.dtype != self.torch_dtype() or not z.is_cuda or not z.is_contiguous():
            raise ValueError("z must be a contiguous CUDA tensor of the handle's dtype")
        batch, n = int(z.shape[0]), int(z.shape[1])
        if mask is not None:
            if tuple(mask.shape) != (batch, n, n) or mask.dtype != z.dtype or not mask.is_contiguous():
                raise ValueError("mask must be a contiguous [B, N, N] tensor of z's dtype")
        for name, t in (("mask", mask), ("out", out), ("workspace", workspace)):
            _check_device(name, t, z)
        if direction not in DIRECTIONS:
            raise ValueError("direction must be 'outgoing' or 'incoming'")
        if out is None:
            out = torch.empty_like(z)
        elif out.shape != z.shape or out.dtype != z.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped like z")
        if stream is None:
            stream = torch.cuda.current_stream(z.device).cuda_stream
        if workspace is None and workspace_needed:
            workspace = self.new_workspace(batch, n, device=z.device)
            _keep_for_stream(workspace, stream, z)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        return (z.data_ptr(), None if mask is None else mask.data_ptr(), out.data_ptr(),
                batch, n, DIRECTIONS[direction], ws_ptr, ws_bytes, stream), out, workspace

    def _extents_ptr(self, extents, z):
        import torch
        batch = int(z.shape[0])
        if (tuple(extents.shape) != (batch, EXTENT_PARTS) or extents.dtype != torch.int32
                or not extents.is_contiguous()):
            raise ValueError("extents must be the contiguous int32 [B, 64] tensor of mask_extents")
        _check_device("extents", extents, z)
        return extents.data_ptr()

    def forward(self, z, mask=None, out=None, direction="outgoing", workspace=None, stream=None,
                extents=None):
        """The update; with `extents` (mask_extents of this mask) the contraction skips the
        padding past each item's extent (tri_mul_forward_extents)."""
        args, out, _ = self._args(z, mask, out, workspace, direction, stream)
        if extents is not None:
            e = self._extents_ptr(extents, z)
            _check(self.lib.tri_mul_forward_extents(self._h, args[0], args[1], e, *args[2:6], 0,
                                                    *args[6:]), "tri_mul_forward_extents")
            return out
        _check(self.lib.tri_mul_forward(self._h, *args), "tri_mul_forward")
        return out

    __call__ = forward

    def forward_static(self, z, mask=None, out=None, direction="outgoing", stream=None):
        """forward with the library's own static workspace (tri_mul_forward_static): no
        workspace is allocated or passed. Calls that overlap on one GPU race on it."""
        args, out, _ = self._args(z, mask, out, None, direction, stream, workspace_needed=False)
        _check(self.lib.tri_mul_forward_static(self._h, *args[:6], args[8]),
               "tri_mul_forward_static")
        return out

    def forward_residual(self, z, mask=None, out=None, direction="outgoing", workspace=None,
                         stream=None, extents=None):
        """out = z + update (out may be z itself for an in-place pair update)."""
        args, out, _ = self._args(z, mask, out, workspace, direction, stream)
        if extents is not None:
            e = self._extents_ptr(extents, z)
            _check(self.lib.tri_mul_forward_extents(self._h, args[0], args[1], e, *args[2:6], 1,
                                                    *args[6:]), "tri_mul_forward_extents")
            return out
        _check(self.lib.tri_mul_forward_residual(self._h, *args), "tri_mul_forward_residual")
        return out

    def stage(self, stage, z, mask=None, out=None, direction="outgoing", workspace=None,
              stream=None):
        args, out, workspace = self._args(z, mask, out, workspace, direction, stream)
        _check(self.lib.tri_mul_forward_stage(self._h, int(stage), *args), "tri_mul_forward_stage")
        return out, workspace

    def close(self):
        if getattr(self, "_h", None):
            self.lib.tri_mul_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PairTransition:
    """The pair transition as a masked residual (one weight set, one dtype):
    out = z + m * (W2 relu(W1 LN(z) + b1) + b2), hidden width `hidden`.

    weights: mapping with the pair_transition_weights field names, fp32 host arrays in
    nn.Linear orientation (missing gamma -> ones, missing beta / biases -> zeros).
    """

    def __init__(self, weights, c_z, hidden, dtype="bf16"):
        self.lib = load_library()
        self.c_z, self.hidden, self.dtype = int(c_z), int(hidden), dtype
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
        keep = {}
        ws = TransitionWeights()
        for name in TRANSITION_FIELDS:
            v = weights.get(name) if hasattr(weights, "get") else None
            if v is None:
                continue
            keep[name] = _host_f32(v)
            setattr(ws, name, keep[name].ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        h = ctypes.c_void_p()
        _check(self.lib.pair_transition_create(ctypes.byref(ws), self.c_z, self.hidden,
                                               DTYPES[dtype], ctypes.byref(h)),
               "pair_transition_create")
        self._h = h

    def forward(self, z, mask=None, out=None, stream=None):
        """out = z + m * transition(z); out may be z itself (in place)."""
        import torch
        dt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if z.dim() != 4 or z.shape[1] != z.shape[2] or z.shape[3] != self.c_z:
            raise ValueError(f"z must be [B, N, N, {self.c_z}], got {tuple(z.shape)}")
        if z.dtype != dt or not z.is_cuda or not z.is_contiguous():
            raise ValueError("z must be a contiguous CUDA tensor of the handle's dtype")
        batch, n = int(z.shape[0]), int(z.shape[1])
        if mask is not None and (tuple(mask.shape) != (batch, n, n) or mask.dtype != z.dtype
                                 or not mask.is_contiguous()):
            raise ValueError("mask must be a contiguous [B, N, N] tensor of z's dtype")
        for name, t in (("mask", mask), ("out", out)):
            _check_device(name, t, z)
        if out is None:
            out = torch.empty_like(z)
        elif out.shape != z.shape or out.dtype != z.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped like z")
        if stream is None:
            stream = torch.cuda.current_stream(z.device).cuda_stream
        _check(self.lib.pair_transition_forward(self._h, z.data_ptr(),
                                                None if mask is None else mask.data_ptr(),
                                                out.data_ptr(), batch, n, stream),
               "pair_transition_forward")
        return out

    __call__ = forward

    def close(self):
        if getattr(self, "_h", None):
            self.lib.pair_transition_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class TriAttention:
    """Triangular attention around the starting or ending node (one weight set; bf16).

    weights: mapping with the tri_attn_weights field names, fp32 host arrays in nn.Linear
    orientation, heads stacked along the output rows (missing gamma -> ones, missing
    beta / b_g / b_o -> zeros).
    """

    def __init__(self, weights, c_z, heads, head_dim=32, dtype="bf16"):
        self.lib = load_library()
        self.c_z, self.heads, self.head_dim, self.dtype = int(c_z), int(heads), int(head_dim), dtype
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
        keep = {}
        ws = AttentionWeights()
        for name in ATTENTION_FIELDS:
            v = weights.get(name) if hasattr(weights, "get") else None
            if v is None:
                continue
            keep[name] = _host_f32(v)
            setattr(ws, name, keep[name].ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        h = ctypes.c_void_p()
        _check(self.lib.tri_attn_create(ctypes.byref(ws), self.c_z, self.heads, self.head_dim,
                                        DTYPES[dtype], ctypes.byref(h)), "tri_attn_create")
        self._h = h

    def workspace_bytes(self, batch, n):
        out = ctypes.c_size_t()
        _check(self.lib.tri_attn_workspace_bytes(self._h, int(batch), int(n), ctypes.byref(out)),
               "tri_attn_workspace_bytes")
        return out.value

    def new_workspace(self, batch, n, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(batch, n), dtype=torch.uint8, device=device)

    def forward(self, z, mask=None, out=None, node="starting", workspace=None, stream=None):
        """out = triangular attention of z around `node` ("starting" or "ending")."""
        return self._call(0, z, mask, out, node, workspace, stream)

    def stage(self, stage, z, mask=None, out=None, node="starting", workspace=None, stream=None):
        """One kernel of forward alone: 1 = projection into the workspace, 2 = attention
        and output projection from it."""
        return self._call(int(stage), z, mask, out, node, workspace, stream)

    def _call(self, stage, z, mask, out, node, workspace, stream):
        import torch
        if node not in NODES:
            raise ValueError(f"node must be one of {sorted(NODES)}")
        if z.dim() != 4 or z.shape[1] != z.shape[2] or z.shape[3] != self.c_z:
            raise ValueError(f"z must be [B, N, N, {self.c_z}], got {tuple(z.shape)}")
        if z.dtype != torch.bfloat16 or not z.is_cuda or not z.is_contiguous():
            raise ValueError("z must be a contiguous bfloat16 CUDA tensor")
        batch, n = int(z.shape[0]), int(z.shape[1])
        if mask is not None and (tuple(mask.shape) != (batch, n, n) or mask.dtype != z.dtype
                                 or not mask.is_contiguous()):
            raise ValueError("mask must be a contiguous [B, N, N] tensor of z's dtype")
        for name, t in (("mask", mask), ("out", out), ("workspace", workspace)):
            _check_device(name, t, z)
        if out is None:
            out = torch.empty_like(z)
        elif out.shape != z.shape or out.dtype != z.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped like z")
        if stream is None:
            stream = torch.cuda.current_stream(z.device).cuda_stream
        if workspace is None:
            workspace = self.new_workspace(batch, n, z.device)
            _keep_for_stream(workspace, stream, z)
        args = (z.data_ptr(), None if mask is None else mask.data_ptr(), out.data_ptr(), batch, n,
                NODES[node], workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
        if stage == 0:
            _check(self.lib.tri_attn_forward(self._h, *args), "tri_attn_forward")
        else:
            _check(self.lib.tri_attn_forward_stage(self._h, stage, *args), "tri_attn_forward_stage")
        return out

    __call__ = forward

    def close(self):
        if getattr(self, "_h", None):
            self.lib.tri_attn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
