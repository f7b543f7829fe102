"""Python binding of the MI355X MoE-layer hot path (argument marshalling only).

Every function here has the name of the C entry point it calls (include/moe.h) and only converts
torch tensors into device pointers, checks shapes and dtypes, and raises on a non-zero status. All
computation runs in the gfx950 HIP library `libmoe_gfx950.so`, built in-tree by
`python -m combine_router_gemm_amd.build`. There is no fallback: if the library is missing, every call
raises.

Tensors must be contiguous, on the current HIP device; work is enqueued on torch's current stream
unless `stream` is given.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["MOE_F32", "MOE_BF16", "MOE_FP8_BLOCK", "MoeError", "Layout", "library_path", "load_library",
           "moe_route", "moe_dispatch", "moe_expert_mlp", "moe_combine", "moe_dispatch_fp8", "moe_expert_mlp_fp8",
           "moe_combine_send", "moe_combine_recv", "moe_expert_mlp_combine", "moe_dispatch_noalloc",
           "MOE_DISPATCH_NOALLOC_MAX_WORKSPACE",
           "moe_expert_mlp_combine_workspace_bytes", "moe_rows_max", "moe_route_workspace_bytes", "moe_dispatch_workspace_bytes",
           "moe_expert_mlp_workspace_bytes", "moe_status_string", "EXPORTED_SYMBOLS"]

MOE_F32 = 0
MOE_BF16 = 1
MOE_FP8_BLOCK = 128  # hidden elements per fp8 block scale
MOE_DISPATCH_NOALLOC_MAX_WORKSPACE = 4 << 20  # bytes of moe_dispatch_noalloc's static scratch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_gfx950.so"

EXPORTED_SYMBOLS = ("moe_status_string", "moe_rows_max", "moe_route_workspace_bytes", "moe_route",
                    "moe_dispatch_workspace_bytes", "moe_dispatch", "moe_expert_mlp_workspace_bytes",
                    "moe_expert_mlp", "moe_combine", "moe_dispatch_fp8", "moe_expert_mlp_fp8", "moe_combine_send",
                    "moe_combine_recv", "moe_expert_mlp_combine", "moe_expert_mlp_combine_workspace_bytes",
                    "moe_dispatch_noalloc")


class MoeError(RuntimeError):
    """A non-zero status from the HIP library."""


class _CLayout(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("k", ctypes.c_int32), ("E", ctypes.c_int32), ("R", ctypes.c_int32),
                ("C", ctypes.c_int32), ("H", ctypes.c_int32),
                ("expert_count", ctypes.c_void_p), ("expert_kept", ctypes.c_void_p),
                ("expert_overflow", ctypes.c_void_p), ("expert_offset", ctypes.c_void_p),
                ("row_token", ctypes.c_void_p), ("row_slot", ctypes.c_void_p), ("pair_row", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load (once) and return the ctypes handle of the HIP library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise MoeError(f"{path} is missing: build it with `python -m combine_router_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_rows_max.argtypes = [i32, i32, i32, i32]
    lib.moe_rows_max.restype = i64
    lib.moe_route_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.moe_route_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_route.restype = i32
    lib.moe_dispatch_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_dispatch_workspace_bytes.restype = sz
    lib.moe_dispatch.argtypes = [vp, i32, vp, ctypes.POINTER(_CLayout), vp, vp, sz, vp]
    lib.moe_dispatch.restype = i32
    lib.moe_dispatch_noalloc.argtypes = [vp, i32, vp, ctypes.POINTER(_CLayout), vp, vp]
    lib.moe_dispatch_noalloc.restype = i32
    lib.moe_expert_mlp_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.moe_expert_mlp_workspace_bytes.restype = sz
    lib.moe_expert_mlp.argtypes = [vp, i32, ctypes.POINTER(_CLayout), vp, vp, i32, vp, vp, sz, vp]
    lib.moe_expert_mlp.restype = i32
    lib.moe_combine.argtypes = [vp, i32, ctypes.POINTER(_CLayout), vp, vp, vp]
    lib.moe_combine.restype = i32
    lib.moe_dispatch_fp8.argtypes = [vp, i32, vp, ctypes.POINTER(_CLayout), vp, vp, vp, sz, vp]
    lib.moe_dispatch_fp8.restype = i32
    lib.moe_expert_mlp_fp8.argtypes = [vp, vp, ctypes.POINTER(_CLayout), vp, vp, i32, vp, vp, sz, vp]
    lib.moe_expert_mlp_fp8.restype = i32
    lib.moe_expert_mlp_combine.argtypes = [vp, i32, ctypes.POINTER(_CLayout), vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_expert_mlp_combine.restype = i32
    lib.moe_expert_mlp_combine_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.moe_expert_mlp_combine_workspace_bytes.restype = sz
    lib.moe_combine_send.argtypes = [vp, i32, ctypes.POINTER(_CLayout), vp, vp, vp]
    lib.moe_combine_send.restype = i32
    lib.moe_combine_recv.argtypes = [vp, i32, ctypes.POINTER(_CLayout), vp, vp]
    lib.moe_combine_recv.restype = i32
    _lib = lib
    return lib


# ------------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise MoeError(f"unsupported activation dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise MoeError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream_obj(stream) -> torch.cuda.Stream:
    """The torch stream object the call's kernels are enqueued on."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream) -> Optional[int]:
    return _stream_obj(stream).cuda_stream


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().moe_status_string(status).decode()
        raise MoeError(f"{what} failed: {msg} ({status})")


# ------------------------------------------------------------------------------------------------
# sizes
# ------------------------------------------------------------------------------------------------

def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_rows_max(T: int, k: int, E: int, C: int) -> int:
    return int(load_library().moe_rows_max(T, k, E, C))


def moe_route_workspace_bytes(T: int, H: int, E: int, xdt: int) -> int:
    return int(load_library().moe_route_workspace_bytes(T, H, E, xdt))


def moe_dispatch_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(load_library().moe_dispatch_workspace_bytes(T, k, E))


def moe_expert_mlp_workspace_bytes(T: int, k: int, E: int, R: int, C: int, F: int, xdt: int) -> int:
    return int(load_library().moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, xdt))


def moe_expert_mlp_combine_workspace_bytes(T: int, k: int, E: int, R: int, C: int, H: int, F: int, xdt: int) -> int:
    return int(load_library().moe_expert_mlp_combine_workspace_bytes(T, k, E, R, C, H, F, xdt))


# ------------------------------------------------------------------------------------------------
# layout descriptor
# ------------------------------------------------------------------------------------------------

class Layout:
    """The per-rank send-buffer layout: scalars plus caller-owned int32 device arrays.

    Allocates the arrays with torch on `device` (allocation is the caller's side of the ABI);
    `moe_dispatch` fills them.
    """

    def __init__(self, T: int, k: int, E: int, R: int, C: int, H: int, device="cuda"):
        self.T, self.k, self.E, self.R, self.C, self.H = T, k, E, R, C, H
        self.rows_max = max(0, min(T * k, E * C)) if (T > 0 and C > 0) else 0
        i32 = dict(dtype=torch.int32, device=device)
        self.expert_count = torch.empty(E, **i32)
        self.expert_kept = torch.empty(E, **i32)
        self.expert_overflow = torch.empty(E, **i32)
        self.expert_offset = torch.empty(E + 1, **i32)
        self.row_token = torch.empty(self.rows_max, **i32)
        self.row_slot = torch.empty(self.rows_max, **i32)
        self.pair_row = torch.empty(T, k, **i32)

    @property
    def El(self) -> int:
        return self.E // self.R

    def c_struct(self) -> _CLayout:
        def p(t):
            return t.data_ptr() if t.numel() > 0 else None
        return _CLayout(self.T, self.k, self.E, self.R, self.C, self.H,
                        p(self.expert_count), p(self.expert_kept), p(self.expert_overflow),
                        p(self.expert_offset), p(self.row_token), p(self.row_slot), p(self.pair_row))


def _workspace(nbytes: int, workspace: Optional[torch.Tensor], device, stream) -> Optional[torch.Tensor]:
    """The caller's workspace, or a temporary one. A temporary workspace is allocated on torch's current
    stream and freed when the call returns, while the kernels that use it may still be queued on
    `stream`: record_stream makes the caching allocator wait for that stream before reusing it."""
    if nbytes == 0:
        return workspace
    if workspace is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        ws.record_stream(_stream_obj(stream))
        return ws
    if _nbytes(workspace) < nbytes:
        raise MoeError(f"workspace too small: need {nbytes} bytes")
    return workspace


def _nbytes(t: Optional[torch.Tensor]) -> int:
    """Size in bytes of a workspace tensor of any element type."""
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------------------------------------
# the four calls
# ------------------------------------------------------------------------------------------------

def moe_route(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor], k: int,
              logits: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Router logits, top-k ids (ties to the lower id) and softmax weights over the k selected."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    stride = 0
    if logit_bias is not None:
        if logit_bias.dim() == 1:
            _ptr(logit_bias, "logit_bias", torch.float32, (E,), dev)
        else:
            _ptr(logit_bias, "logit_bias", torch.float32, (T, E), dev)
            stride = E
    ws = _workspace(moe_route_workspace_bytes(T, H, E, _dtype_code(x)), workspace, dev, stream)
    st = load_library().moe_route(
        _ptr(x, "x", device=dev), _dtype_code(x), _ptr(w_router, "w_router", torch.float32, (E, H), dev),
        _ptr(logit_bias, "logit_bias"), stride, T, H, E, k,
        _ptr(logits, "logits", torch.float32, (T, E), dev), _ptr(topk_ids, "topk_ids", torch.int32, (T, k), dev),
        _ptr(topk_w, "topk_w", torch.float32, (T, k), dev), _ptr(ws, "workspace"),
        _nbytes(ws), _stream(stream))
    _check(st, "moe_route")


def moe_dispatch(x: torch.Tensor, topk_ids: torch.Tensor, layout: Layout, send_buf: torch.Tensor,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Histogram, capacity-clamped prefix scan and stable scatter of token rows into `send_buf`."""
    dev = x.device
    L = layout
    _ptr(x, "x", shape=(L.T, L.H), device=dev)
    _ptr(send_buf, "send_buf", x.dtype, (L.rows_max, L.H), dev)
    ws = _workspace(moe_dispatch_workspace_bytes(L.T, L.k, L.E), workspace, dev, stream)
    cl = L.c_struct()
    st = load_library().moe_dispatch(
        _ptr(x, "x"), _dtype_code(x), _ptr(topk_ids, "topk_ids", torch.int32, (L.T, L.k), dev), ctypes.byref(cl),
        _ptr(send_buf, "send_buf"), _ptr(ws, "workspace"), _nbytes(ws), _stream(stream))
    _check(st, "moe_dispatch")


def moe_dispatch_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, layout: Layout, send_buf: torch.Tensor,
                         stream=None) -> None:
    """moe_dispatch with the library's static per-GPU scratch instead of a workspace (allocates nothing).
    Calls that may overlap on one GPU race; calls on one stream are ordered."""
    dev = x.device
    L = layout
    _ptr(x, "x", shape=(L.T, L.H), device=dev)
    _ptr(send_buf, "send_buf", x.dtype, (L.rows_max, L.H), dev)
    cl = L.c_struct()
    st = load_library().moe_dispatch_noalloc(
        _ptr(x, "x"), _dtype_code(x), _ptr(topk_ids, "topk_ids", torch.int32, (L.T, L.k), dev), ctypes.byref(cl),
        _ptr(send_buf, "send_buf"), _stream(stream))
    _check(st, "moe_dispatch_noalloc")


def moe_expert_mlp(send_buf: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                   out_buf: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Per-expert SwiGLU MLP (grouped MFMA GEMM) on the dispatched rows; output row-aligned with send_buf."""
    dev = send_buf.device
    L = layout
    El = L.E // L.R
    F = w_gate_up.shape[1] // 2
    dt = _dtype_code(send_buf)
    _ptr(send_buf, "send_buf", shape=(L.rows_max, L.H), device=dev)
    _ptr(w_gate_up, "w_gate_up", send_buf.dtype, (El, 2 * F, L.H), dev)
    _ptr(w_down, "w_down", send_buf.dtype, (El, L.H, F), dev)
    _ptr(out_buf, "out_buf", send_buf.dtype, (L.rows_max, L.H), dev)
    ws = _workspace(moe_expert_mlp_workspace_bytes(L.T, L.k, L.E, L.R, L.C, F, dt), workspace, dev, stream)
    cl = L.c_struct()
    st = load_library().moe_expert_mlp(
        _ptr(send_buf, "send_buf"), dt, ctypes.byref(cl), _ptr(w_gate_up, "w_gate_up"), _ptr(w_down, "w_down"), F,
        _ptr(out_buf, "out_buf"), _ptr(ws, "workspace"), _nbytes(ws), _stream(stream))
    _check(st, "moe_expert_mlp")


def moe_expert_mlp_combine(send_buf: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                           topk_w: torch.Tensor, out_buf: torch.Tensor, y: torch.Tensor,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_expert_mlp with moe_combine fused into its down GEMM: writes out_buf and y in one call."""
    dev = send_buf.device
    L = layout
    El = L.E // L.R
    F = w_gate_up.shape[1] // 2
    dt = _dtype_code(send_buf)
    _ptr(send_buf, "send_buf", shape=(L.rows_max, L.H), device=dev)
    _ptr(w_gate_up, "w_gate_up", send_buf.dtype, (El, 2 * F, L.H), dev)
    _ptr(w_down, "w_down", send_buf.dtype, (El, L.H, F), dev)
    _ptr(out_buf, "out_buf", send_buf.dtype, (L.rows_max, L.H), dev)
    _ptr(y, "y", send_buf.dtype, (L.T, L.H), dev)
    ws = _workspace(moe_expert_mlp_combine_workspace_bytes(L.T, L.k, L.E, L.R, L.C, L.H, F, dt), workspace, dev, stream)
    cl = L.c_struct()
    st = load_library().moe_expert_mlp_combine(
        _ptr(send_buf, "send_buf"), dt, ctypes.byref(cl), _ptr(w_gate_up, "w_gate_up"), _ptr(w_down, "w_down"), F,
        _ptr(topk_w, "topk_w", torch.float32, (L.T, L.k), dev), _ptr(out_buf, "out_buf"), _ptr(y, "y"),
        _ptr(ws, "workspace"), _nbytes(ws), _stream(stream))
    _check(st, "moe_expert_mlp_combine")


def moe_combine(out_buf: torch.Tensor, layout: Layout, topk_w: torch.Tensor, y: torch.Tensor,
                stream=None) -> None:
    """y[t] = sum of the kept slots' routing weight times their expert output row (fp32 accumulate)."""
    dev = y.device
    L = layout
    _ptr(out_buf, "out_buf", y.dtype, (L.rows_max, L.H), dev)
    _ptr(y, "y", shape=(L.T, L.H), device=dev)
    cl = L.c_struct()
    st = load_library().moe_combine(
        _ptr(out_buf, "out_buf"), _dtype_code(y), ctypes.byref(cl),
        _ptr(topk_w, "topk_w", torch.float32, (L.T, L.k), dev), _ptr(y, "y"), _stream(stream))
    _check(st, "moe_combine")


def moe_combine_send(out_buf: torch.Tensor, layout: Layout, topk_w: torch.Tensor, partial: torch.Tensor,
                     stream=None) -> None:
    """Sender-side partial rows: partial[r, t] = sum of t's kept slots on rank r of weight times expert
    output (fp32 accumulate, rounded once). partial is [R, T, H] in the activation type; slots of ranks
    holding no kept slot of t are left as they are."""
    dev = partial.device
    L = layout
    _ptr(out_buf, "out_buf", partial.dtype, (L.rows_max, L.H), dev)
    _ptr(partial, "partial", shape=(L.R, L.T, L.H), device=dev)
    cl = L.c_struct()
    st = load_library().moe_combine_send(
        _ptr(out_buf, "out_buf"), _dtype_code(partial), ctypes.byref(cl),
        _ptr(topk_w, "topk_w", torch.float32, (L.T, L.k), dev), _ptr(partial, "partial"), _stream(stream))
    _check(st, "moe_combine_send")


def moe_combine_recv(partial: torch.Tensor, layout: Layout, y: torch.Tensor, stream=None) -> None:
    """y[t] = sum over the ranks holding kept slots of t (ascending) of partial[r, t] (fp32, rounded once)."""
    dev = y.device
    L = layout
    _ptr(partial, "partial", y.dtype, (L.R, L.T, L.H), dev)
    _ptr(y, "y", shape=(L.T, L.H), device=dev)
    cl = L.c_struct()
    st = load_library().moe_combine_recv(_ptr(partial, "partial"), _dtype_code(y), ctypes.byref(cl), _ptr(y, "y"),
                                         _stream(stream))
    _check(st, "moe_combine_recv")


def moe_dispatch_fp8(x: torch.Tensor, topk_ids: torch.Tensor, layout: Layout, send_q: torch.Tensor,
                     send_scale: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_dispatch with fp8 block-scaled send rows: E4M3 codes (uint8) and one power-of-two fp32 scale
    per 128 hidden elements. x must be bf16."""
    dev = x.device
    L = layout
    _ptr(x, "x", torch.bfloat16, (L.T, L.H), dev)
    _ptr(send_q, "send_q", torch.uint8, (L.rows_max, L.H), dev)
    _ptr(send_scale, "send_scale", torch.float32, (L.rows_max, L.H // MOE_FP8_BLOCK), dev)
    ws = _workspace(moe_dispatch_workspace_bytes(L.T, L.k, L.E), workspace, dev, stream)
    cl = L.c_struct()
    st = load_library().moe_dispatch_fp8(
        _ptr(x, "x"), MOE_BF16, _ptr(topk_ids, "topk_ids", torch.int32, (L.T, L.k), dev), ctypes.byref(cl),
        _ptr(send_q, "send_q"), _ptr(send_scale, "send_scale"), _ptr(ws, "workspace"),
        _nbytes(ws), _stream(stream))
    _check(st, "moe_dispatch_fp8")


def moe_expert_mlp_fp8(send_q: torch.Tensor, send_scale: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor,
                       w_down: torch.Tensor, out_buf: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """Expert SwiGLU MLP on fp8 block-scaled rows (decoded to bf16 in the GEMM); bf16 weights and output."""
    dev = send_q.device
    L = layout
    El = L.E // L.R
    F = w_gate_up.shape[1] // 2
    _ptr(send_q, "send_q", torch.uint8, (L.rows_max, L.H), dev)
    _ptr(send_scale, "send_scale", torch.float32, (L.rows_max, L.H // MOE_FP8_BLOCK), dev)
    _ptr(w_gate_up, "w_gate_up", torch.bfloat16, (El, 2 * F, L.H), dev)
    _ptr(w_down, "w_down", torch.bfloat16, (El, L.H, F), dev)
    _ptr(out_buf, "out_buf", torch.bfloat16, (L.rows_max, L.H), dev)
    ws = _workspace(moe_expert_mlp_workspace_bytes(L.T, L.k, L.E, L.R, L.C, F, MOE_BF16), workspace, dev, stream)
    cl = L.c_struct()
    st = load_library().moe_expert_mlp_fp8(
        _ptr(send_q, "send_q"), _ptr(send_scale, "send_scale"), ctypes.byref(cl), _ptr(w_gate_up, "w_gate_up"),
        _ptr(w_down, "w_down"), F, _ptr(out_buf, "out_buf"), _ptr(ws, "workspace"), _nbytes(ws),
        _stream(stream))
    _check(st, "moe_expert_mlp_fp8")
