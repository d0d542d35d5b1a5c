"""Python binding of libmoe.so (C ABI in include/moe.h): argument marshalling only.

Every function has the name of the C entry point it calls and does nothing but turn
torch tensors into device pointers, sizes into the ``moe_dims``/``moe_opts`` structs and
the current torch stream into a ``hipStream_t``. All arithmetic runs in the library's HIP
kernels; if the library is missing these functions raise instead of computing anything.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = 0, 1
MOE_W_UP, MOE_W_DOWN = 0, 1
MOE_STAGE_ROUTE, MOE_STAGE_PERMUTE, MOE_STAGE_EXPERT_UP, MOE_STAGE_EXPERT_DOWN, MOE_STAGE_COMBINE = range(5)
MOE_NUM_STAGES = 5
MOE_STAGE_ATTENTION, MOE_BLOCK_NUM_STAGES = 5, 6  # moe_block_forward's extra stage and array size
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

# every symbol include/moe.h declares
SYMBOLS = ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_pack_weights", "moe_workspace_bytes",
           "moe_forward", "moe_forward_noalloc", "moe_backward_workspace_bytes", "moe_backward", "moe_rmsnorm", "moe_attention",
           "moe_block_workspace_bytes", "moe_block_forward", "moe_status_string", "moe_last_error",
           "moe_abi_version")


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("F", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


class moe_opts(ctypes.Structure):
    _fields_ = [("gate_bias", ctypes.c_void_p), ("y_dtype", ctypes.c_int32), ("accumulate", ctypes.c_int32),
                ("stage_events", ctypes.c_void_p), ("activations", ctypes.c_void_p)]


class moe_attn_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("eps", ctypes.c_float)]


@dataclass(frozen=True)
class AttnDims:
    T: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int = 128
    rope_base: float = 1e6
    eps: float = 1e-5

    def c(self) -> moe_attn_dims:
        return moe_attn_dims(self.T, self.d, self.n_heads, self.n_kv_heads, self.head_dim, self.rope_base, self.eps)


@dataclass(frozen=True)
class Dims:
    T: int
    d: int
    F: int
    E: int
    K: int
    dtype: int  # MOE_F32 or MOE_BF16
    layout: int = MOE_LAYOUT_ROWMAJOR  # of w1, w3, w2

    def c(self) -> moe_dims:
        return moe_dims(self.T, self.d, self.F, self.E, self.K, self.dtype, self.layout)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by sparse_mixture_experts_33_amd/build.py). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        P = ctypes.POINTER
        L.moe_route.argtypes = [P(moe_dims), P(moe_opts), vp, vp, vp, vp, vp, vp]
        L.moe_permute.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_combine.argtypes = [P(moe_dims), P(moe_opts), vp, vp, vp, vp, vp]
        L.moe_pack_weights.argtypes = [P(moe_dims), i32, vp, vp, vp]
        L.moe_workspace_bytes.argtypes = [P(moe_dims)]
        L.moe_workspace_bytes.restype = sz
        L.moe_forward.argtypes = [P(moe_dims), P(moe_opts), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward_noalloc.argtypes = [P(moe_dims), P(moe_opts), vp, vp, vp, vp, vp, vp, vp]
        L.moe_backward_workspace_bytes.argtypes = [P(moe_dims)]
        L.moe_backward_workspace_bytes.restype = sz
        L.moe_backward.argtypes = [P(moe_dims), P(moe_opts), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                   vp]
        L.moe_rmsnorm.argtypes = [i64, i32, f32, vp, vp, vp]
        L.moe_attention.argtypes = [P(moe_attn_dims), vp, vp, vp, vp, vp]
        L.moe_block_workspace_bytes.argtypes = [P(moe_dims), P(moe_attn_dims)]
        L.moe_block_workspace_bytes.restype = sz
        L.moe_block_forward.argtypes = [P(moe_dims), P(moe_attn_dims), P(moe_opts), vp, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_abi_version.restype = i32
        for name in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_pack_weights", "moe_forward",
                     "moe_forward_noalloc", "moe_backward", "moe_rmsnorm", "moe_attention", "moe_block_forward"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _opts(gate_bias=None, y_dtype=None, accumulate=False, dtype=MOE_BF16, stage_events=None, activations=None):
    return moe_opts(_ptr(gate_bias), dtype if y_dtype is None else y_dtype, 1 if accumulate else 0,
                    stage_events, _ptr(activations))


def stage_event_array(events: dict, stages: int = MOE_NUM_STAGES):
    """ctypes array of 2*stages hipEvent_t handles for moe_opts.stage_events (stages:
    MOE_NUM_STAGES for moe_forward, MOE_BLOCK_NUM_STAGES for moe_block_forward).

    events maps an array position (2*stage for the start, 2*stage+1 for the end of that stage's
    kernel) to a raw hipEvent_t handle (e.g. torch.cuda.Event(...).cuda_event); other positions
    stay NULL."""
    arr = (ctypes.c_void_p * (2 * stages))()
    for i, h in events.items():
        arr[i] = h
    return arr


def moe_route(dims: Dims, x, w_gate, topk_idx, topk_w, logits=None, gate_bias=None, stream=None):
    o = _opts(gate_bias, dtype=dims.dtype)
    _check(lib().moe_route(ctypes.byref(dims.c()), ctypes.byref(o), _ptr(x), _ptr(w_gate), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(logits), _stream(stream)))


def moe_permute(dims: Dims, topk_idx, x, counts, offsets, row_token, token_row, x_perm=None, stream=None):
    _check(lib().moe_permute(ctypes.byref(dims.c()), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                             _ptr(row_token), _ptr(token_row), _ptr(x_perm), _stream(stream)))


def moe_expert_ffn(dims: Dims, x_perm, offsets, w1, w3, w2, h_ws, y_perm, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(dims.c()), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2),
                                _ptr(h_ws), _ptr(y_perm), _stream(stream)))


def moe_combine(dims: Dims, y_perm, token_row, topk_w, y, y_dtype=None, accumulate=False, stream=None):
    o = _opts(None, y_dtype, accumulate, dims.dtype)
    _check(lib().moe_combine(ctypes.byref(dims.c()), ctypes.byref(o), _ptr(y_perm), _ptr(token_row), _ptr(topk_w),
                             _ptr(y), _stream(stream)))


def moe_pack_weights(dims: Dims, which: int, w, w_packed, stream=None):
    _check(lib().moe_pack_weights(ctypes.byref(dims.c()), which, _ptr(w), _ptr(w_packed), _stream(stream)))


def moe_workspace_bytes(dims: Dims) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(dims.c())))


def moe_forward(dims: Dims, x, w_gate, w1, w3, w2, y, workspace, gate_bias=None, y_dtype=None, accumulate=False,
                stream=None, workspace_bytes=None, stage_events=None, activations=None):
    """stage_events: None or the result of stage_event_array() (kept alive by the caller).
    activations: None or an fp32 device tensor of 2*T*K*F elements that receives the expert
    pre-activations for moe_backward (moe_opts.activations)."""
    o = _opts(gate_bias, y_dtype, accumulate, dims.dtype,
              None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p).value, activations)
    nbytes = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None and not isinstance(workspace, int) else 0)
    _check(lib().moe_forward(ctypes.byref(dims.c()), ctypes.byref(o), _ptr(x), _ptr(w_gate), _ptr(w1), _ptr(w3),
                             _ptr(w2), _ptr(y), _ptr(workspace), nbytes, _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static per-device scratch of moe_forward_noalloc


def moe_forward_noalloc(dims: Dims, x, w_gate, w1, w3, w2, y, gate_bias=None, y_dtype=None, accumulate=False,
                        stream=None, stage_events=None, activations=None):
    """moe_forward with the library's static per-device scratch as its workspace (include/moe.h):
    allocates nothing; calls overlapping in time on one device race on the scratch."""
    o = _opts(gate_bias, y_dtype, accumulate, dims.dtype,
              None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p).value, activations)
    _check(lib().moe_forward_noalloc(ctypes.byref(dims.c()), ctypes.byref(o), _ptr(x), _ptr(w_gate), _ptr(w1),
                                     _ptr(w3), _ptr(w2), _ptr(y), _stream(stream)))


def moe_backward_workspace_bytes(dims: Dims) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(dims.c())))


def moe_backward(dims: Dims, x, w_gate, w1, w3, w2, dy, dx, dw_gate, dw1, dw3, dw2, workspace, dlogits=None,
                 gate_bias=None, stream=None, workspace_bytes=None, activations=None):
    """Gradients of the layer (include/moe.h, moe_backward). dy and every output are fp32 device tensors.
    activations: None (recompute the expert pre-activations) or the tensor a moe_forward call on
    the same inputs filled."""
    o = _opts(gate_bias, dtype=dims.dtype, activations=activations)
    nbytes = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None and not isinstance(workspace, int) else 0)
    _check(lib().moe_backward(ctypes.byref(dims.c()), ctypes.byref(o), _ptr(x), _ptr(w_gate), _ptr(w1), _ptr(w3),
                              _ptr(w2), _ptr(dy), _ptr(dx), _ptr(dw_gate), _ptr(dw1), _ptr(dw3), _ptr(dw2),
                              _ptr(dlogits), _ptr(workspace), nbytes, _stream(stream)))


def moe_rmsnorm(T: int, d: int, eps: float, h, x_bf16, stream=None):
    _check(lib().moe_rmsnorm(T, d, eps, _ptr(h), _ptr(x_bf16), _stream(stream)))


def moe_attention(attn: AttnDims, q, k, v, o, stream=None):
    """q [n_heads][T][128], k, v [n_kv_heads][T][128] bf16 -> o [T][n_heads*128] bf16."""
    _check(lib().moe_attention(ctypes.byref(attn.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _stream(stream)))


def moe_block_workspace_bytes(dims: Dims, attn: AttnDims) -> int:
    return int(lib().moe_block_workspace_bytes(ctypes.byref(dims.c()), ctypes.byref(attn.c())))


def moe_block_forward(dims: Dims, attn: AttnDims, h, w_qkv, w_o, w_gate, w1, w3, w2, workspace, gate_bias=None,
                      stream=None, workspace_bytes=None, stage_events=None):
    """One decoder block in place on the fp32 residual stream h [T][d] (include/moe.h)."""
    o = _opts(gate_bias, None, True, dims.dtype,
              None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p).value)
    nbytes = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None and not isinstance(workspace, int) else 0)
    _check(lib().moe_block_forward(ctypes.byref(dims.c()), ctypes.byref(attn.c()), ctypes.byref(o), _ptr(h),
                                   _ptr(w_qkv), _ptr(w_o), _ptr(w_gate), _ptr(w1), _ptr(w3), _ptr(w2),
                                   _ptr(workspace), nbytes, _stream(stream)))


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())
