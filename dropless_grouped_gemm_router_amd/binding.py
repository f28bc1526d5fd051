"""ctypes binding of libmoe (``include/moe.h``): the same entry points with
the same names, marshalling arguments only. Every stage runs in the HIP
kernels of libmoe.so; there is no other implementation behind these calls,
and loading fails loudly when the library has not been built.

Tensors are passed by device pointer (``tensor.data_ptr()``); PyTorch is
used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_TOO_LARGE = -5
MOE_FP32, MOE_BF16 = 0, 1
DTYPES = {"fp32": MOE_FP32, "bf16": MOE_BF16}
MOE_DISPATCH_GATHER, MOE_DISPATCH_SORTED, MOE_DISPATCH_FUSED_GSUM = 0, 1, 2
DISPATCH = {"gather": MOE_DISPATCH_GATHER, "sorted": MOE_DISPATCH_SORTED,
            "fused_gsum": MOE_DISPATCH_FUSED_GSUM}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class moe_problem(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_hidden", ctypes.c_int32),
                ("d_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "expert_offsets", "perm", "inv_perm", "tiles", "num_tiles")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


EXPORTED = ["moe_version", "moe_status_string", "moe_check_problem", "moe_max_tiles",
            "moe_param_count", "moe_workspace_bytes", "moe_saved_bytes", "moe_route",
            "moe_permute", "moe_permute_static", "moe_ffn_fwd", "moe_combine", "moe_forward_workspace_bytes",
            "moe_forward", "moe_bwd", "moe_trace_enable", "moe_trace_summary"]

_lib = None


def load(path: str = LIB_PATH):
    """Loads libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m dropless_grouped_gemm_router_amd.build`")
    lib = ctypes.CDLL(path)
    P, PP = ctypes.c_void_p, ctypes.POINTER(moe_problem)
    sig = {
        "moe_version": (ctypes.c_char_p, []),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_check_problem": (ctypes.c_int, [PP]),
        "moe_max_tiles": (ctypes.c_int64, [PP]),
        "moe_param_count": (ctypes.c_int64, [PP]),
        "moe_workspace_bytes": (ctypes.c_size_t, [PP, ctypes.c_int]),
        "moe_saved_bytes": (ctypes.c_size_t, [PP]),
        "moe_route": (ctypes.c_int, [PP, P, P, ctypes.POINTER(moe_routing), P]),
        "moe_permute": (ctypes.c_int, [PP, ctypes.POINTER(moe_routing), P, ctypes.c_size_t, P]),
        "moe_permute_static": (ctypes.c_int, [PP, ctypes.POINTER(moe_routing), P]),
        "moe_ffn_fwd": (ctypes.c_int, [PP, P, ctypes.POINTER(moe_weights),
                                       ctypes.POINTER(moe_routing), P, P, P, P, ctypes.c_size_t, P]),
        "moe_combine": (ctypes.c_int, [PP, P, ctypes.POINTER(moe_routing), P, P, P]),
        "moe_forward_workspace_bytes": (ctypes.c_size_t, [PP, ctypes.c_int, ctypes.c_int]),
        "moe_forward": (ctypes.c_int, [PP, ctypes.c_int, P, ctypes.POINTER(moe_weights),
                                       ctypes.POINTER(moe_routing), P, P, P, P, ctypes.c_size_t,
                                       P, P]),
        "moe_bwd": (ctypes.c_int, [PP, P, ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing),
                                   P, P, P, P, ctypes.POINTER(moe_grads), P, ctypes.c_size_t, P,
                                   P]),
        "moe_trace_enable": (ctypes.c_int, [ctypes.c_int]),
        "moe_trace_summary": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_size_t]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ----------------------------------------------------------- marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _side(side_stream) -> Optional[int]:
    """The optional second stream: None stays NULL (no second stream)."""
    if side_stream is None:
        return None
    if isinstance(side_stream, int):
        return side_stream
    return side_stream.cuda_stream


def problem_struct(p) -> moe_problem:
    """From any object with the problem fields (e.g. ``inputs.Problem``)."""
    return moe_problem(int(p.tokens), int(p.experts), int(p.top_k), int(p.d_model),
                       int(p.d_hidden), int(p.d_shared),
                       DTYPES[p.dtype] if isinstance(p.dtype, str) else int(p.dtype),
                       int(p.block_m), int(getattr(p, "capacity", 0)))


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def moe_version() -> str:
    return load().moe_version().decode()


def moe_check_problem(p) -> int:
    return load().moe_check_problem(ctypes.byref(problem_struct(p)))


def moe_max_tiles(p) -> int:
    return int(load().moe_max_tiles(ctypes.byref(problem_struct(p))))


def moe_param_count(p) -> int:
    return int(load().moe_param_count(ctypes.byref(problem_struct(p))))


def moe_workspace_bytes(p, training: bool = False) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(problem_struct(p)), int(training)))


def moe_saved_bytes(p) -> int:
    return int(load().moe_saved_bytes(ctypes.byref(problem_struct(p))))


def weights_struct(w: Dict) -> moe_weights:
    return moe_weights(*[_ptr(w.get(n)) for n in
                         ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")])


def routing_struct(r: Dict) -> moe_routing:
    return moe_routing(*[_ptr(r.get(n)) for n in
                         ("topk_idx", "topk_w", "expert_offsets", "perm", "inv_perm", "tiles",
                          "num_tiles")])


def grads_struct(g: Dict) -> moe_grads:
    return moe_grads(*[_ptr(g.get(n)) for n in
                       ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")])


def moe_route(p, x, w_router, routing: Dict, stream=None):
    r = routing_struct(routing)
    _check(load().moe_route(ctypes.byref(problem_struct(p)), _ptr(x), _ptr(w_router),
                            ctypes.byref(r), _stream(stream)), "moe_route")


def moe_permute(p, routing: Dict, workspace, workspace_bytes: Optional[int] = None, stream=None):
    r = routing_struct(routing)
    nb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_permute(ctypes.byref(problem_struct(p)), ctypes.byref(r), _ptr(workspace),
                              nb, _stream(stream)), "moe_permute")


def moe_permute_static(p, routing: Dict, stream=None):
    r = routing_struct(routing)
    _check(load().moe_permute_static(ctypes.byref(problem_struct(p)), ctypes.byref(r),
                                     _stream(stream)), "moe_permute_static")


def moe_ffn_fwd(p, x, weights: Dict, routing: Dict, y_sorted, shared_out, saved, workspace,
                workspace_bytes: Optional[int] = None, stream=None):
    w, r = weights_struct(weights), routing_struct(routing)
    nb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_ffn_fwd(ctypes.byref(problem_struct(p)), _ptr(x), ctypes.byref(w),
                              ctypes.byref(r), _ptr(y_sorted), _ptr(shared_out), _ptr(saved),
                              _ptr(workspace), nb, _stream(stream)), "moe_ffn_fwd")


def moe_combine(p, y_sorted, routing: Dict, shared_out, out, stream=None):
    r = routing_struct(routing)
    _check(load().moe_combine(ctypes.byref(problem_struct(p)), _ptr(y_sorted), ctypes.byref(r),
                              _ptr(shared_out), _ptr(out), _stream(stream)), "moe_combine")


def _dispatch(dispatch) -> int:
    return DISPATCH[dispatch] if isinstance(dispatch, str) else int(dispatch)


def moe_forward_workspace_bytes(p, dispatch, training: bool = False) -> int:
    return int(load().moe_forward_workspace_bytes(ctypes.byref(problem_struct(p)),
                                                  _dispatch(dispatch), int(training)))


def moe_forward(p, dispatch, x, weights: Dict, routing: Dict, y_sorted, saved, out, workspace,
                workspace_bytes: Optional[int] = None, stream=None, side_stream=None):
    w, r = weights_struct(weights), routing_struct(routing)
    nb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_forward(ctypes.byref(problem_struct(p)), _dispatch(dispatch), _ptr(x),
                              ctypes.byref(w), ctypes.byref(r), _ptr(y_sorted), _ptr(saved),
                              _ptr(out), _ptr(workspace), nb, _stream(stream), _side(side_stream)),
           "moe_forward")


def moe_bwd(p, x, weights: Dict, routing: Dict, y_sorted, saved, grad_out, grad_x, grads: Dict,
            workspace, workspace_bytes: Optional[int] = None, stream=None, side_stream=None):
    w, r, g = weights_struct(weights), routing_struct(routing), grads_struct(grads)
    nb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_bwd(ctypes.byref(problem_struct(p)), _ptr(x), ctypes.byref(w),
                          ctypes.byref(r), _ptr(y_sorted), _ptr(saved), _ptr(grad_out),
                          _ptr(grad_x), ctypes.byref(g), _ptr(workspace), nb, _stream(stream),
                          _side(side_stream)),
           "moe_bwd")


def moe_trace_enable(on: bool = True):
    _check(load().moe_trace_enable(int(on)), "moe_trace_enable")


def moe_trace_summary() -> Dict:
    """Per-kernel {"ms": total, "count": launches} since moe_trace_enable(True)."""
    import json
    buf = ctypes.create_string_buffer(1 << 16)
    _check(load().moe_trace_summary(buf, len(buf)), "moe_trace_summary")
    return json.loads(buf.value.decode())


# ------------------------------------------------- device buffers (torch)

@dataclass
class Buffers:
    """Device buffers of one layer call, allocated once with torch."""

    routing: Dict
    y_sorted: object
    shared_out: Optional[object]
    out: object
    workspace: object
    saved: Optional[object] = None
    grad_x: Optional[object] = None
    grads: Optional[Dict] = None


def torch_dtype(p):
    import torch
    return torch.bfloat16 if (p.dtype == "bf16" or p.dtype == MOE_BF16) else torch.float32


def allocate(p, device="cuda", training: bool = False, dispatch=None) -> Buffers:
    """Buffers for the staged calls; with ``dispatch`` the workspace also
    covers moe_forward with that variant."""
    import torch
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    S = T * k
    dt = torch_dtype(p)
    i32 = dict(dtype=torch.int32, device=device)
    routing = dict(
        topk_idx=torch.empty((T, k), **i32),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
        expert_offsets=torch.empty(E + 1, **i32),
        perm=torch.empty(S, **i32),
        inv_perm=torch.empty(S, **i32),
        tiles=torch.empty((max(1, moe_max_tiles(p)), 3), **i32),
        num_tiles=torch.empty(1, **i32),
    )
    nws = moe_workspace_bytes(p, training)
    if dispatch is not None:
        nws = max(nws, moe_forward_workspace_bytes(p, dispatch, training))
    ws = torch.empty(nws, dtype=torch.uint8, device=device)
    b = Buffers(routing=routing,
                y_sorted=torch.empty((S, d), dtype=dt, device=device),
                shared_out=torch.empty((T, d), dtype=dt, device=device) if hs else None,
                out=torch.empty((T, d), dtype=dt, device=device),
                workspace=ws)
    if training:
        b.saved = torch.empty(moe_saved_bytes(p), dtype=torch.uint8, device=device)
        b.grad_x = torch.empty((T, d), dtype=dt, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        b.grads = dict(w_router=torch.empty((d, E), **f32), w_gate=torch.empty((E, d, h), **f32),
                       w_up=torch.empty((E, d, h), **f32), w_down=torch.empty((E, h, d), **f32))
        if hs:
            b.grads.update(ws_gate=torch.empty((d, hs), **f32), ws_up=torch.empty((d, hs), **f32),
                           ws_down=torch.empty((hs, d), **f32))
    return b


def forward(p, x, weights: Dict, buf: Buffers, training: bool = False, stream=None):
    """route -> permute -> grouped FFN (+ shared) -> combine; returns buf.out."""
    moe_route(p, x, weights["w_router"], buf.routing, stream)
    moe_permute(p, buf.routing, buf.workspace, stream=stream)
    moe_ffn_fwd(p, x, weights, buf.routing, buf.y_sorted, buf.shared_out,
                buf.saved if training else None, buf.workspace, stream=stream)
    moe_combine(p, buf.y_sorted, buf.routing, buf.shared_out, buf.out, stream)
    return buf.out


def forward_dispatch(p, dispatch, x, weights: Dict, buf: Buffers, training: bool = False,
                     stream=None, side_stream=None):
    """The whole forward in one moe_forward call with a dispatch variant
    (buf from ``allocate(..., dispatch=...)``); returns buf.out."""
    moe_forward(p, dispatch, x, weights, buf.routing, buf.y_sorted,
                buf.saved if training else None, buf.out, buf.workspace, stream=stream,
                side_stream=side_stream)
    return buf.out


def backward(p, x, weights: Dict, grad_out, buf: Buffers, stream=None, side_stream=None):
    """Gradients of sum(out * grad_out) after forward(..., training=True)."""
    moe_bwd(p, x, weights, buf.routing, buf.y_sorted, buf.saved, grad_out, buf.grad_x, buf.grads,
            buf.workspace, stream=stream, side_stream=side_stream)
    return buf.grad_x, buf.grads


def device_inputs(inputs: Dict, device="cuda") -> Dict:
    """Moves generated inputs (``inputs.Tensor.stored``) to the device with
    their storage dtype (bf16 bit patterns become torch.bfloat16)."""
    import numpy as np
    import torch
    out = {}
    for name, t in inputs.items():
        a = t.stored
        if a.dtype == np.uint16:
            out[name] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out
