"""Deterministic MoE layer (forward and backward) for one AMD MI355X: Python binding.

This module is a ctypes binding of ``libmoe_mi355x.so`` whose functions carry the C ABI's names
(``moe_query``, ``moe_route``, ``moe_permute``, ``moe_forward``, ``moe_backward``). It only
marshals arguments: tensors become device pointers, and the current torch stream becomes the
``hipStream_t``. Every step of the layer runs in the library's HIP kernels. There is no Python or
CPU fallback: if the library is missing, loading it raises.

The C header ``include/moe.h`` documents each call: the operation, the layouts, ownership and
the errors.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK = 0
MOE_PREC_BF16 = 0
MOE_PREC_MXFP8 = 1
MOE_PREC_MXFP4 = 2
MOE_FLAG_PERSISTENT = 1
MOE_FLAG_MXFP8_WGRAD = 2
MOE_FLAG_BF16_DW = 4
MOE_DEVICE_BAD_EXPERT_INDEX = 1
MOE_DEVICE_BARRIER_TIMEOUT = 2


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class MoeCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class MoeSizes(ctypes.Structure):
    _fields_ = [("ring_slot", ctypes.c_size_t), ("saved", ctypes.c_size_t),
                ("saved_H", ctypes.c_size_t), ("saved_A", ctypes.c_size_t),
                ("workspace", ctypes.c_size_t), ("ws_O", ctypes.c_size_t),
                ("ws_dH", ctypes.c_size_t), ("ws_dXp", ctypes.c_size_t),
                ("wq", ctypes.c_size_t)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGS = {
    "moe_query": [ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeSizes)],
    "moe_route": [ctypes.POINTER(MoeCfg), _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_permute": [ctypes.POINTER(MoeCfg), _P, _P, _P, _SZ, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_forward": [ctypes.POINTER(MoeCfg), _P, _SZ, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P, _P,
                    _SZ, _P, _SZ, _P],
    "moe_backward": [ctypes.POINTER(MoeCfg), _P, _SZ, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                     _SZ, _P, _SZ, _P, _P, _P, _P, _P, _P, _I32, _P, _SZ, _P],
    "moe_quantize_weights": [ctypes.POINTER(MoeCfg), _P, _P, _P, _SZ, _P],
    "moe_forward_fused": [ctypes.POINTER(MoeCfg), _P, _P, _P, _P, _P, _P, _SZ, _I32, _P, _P, _P,
                          _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P],
    "moe_permute_static": [ctypes.POINTER(MoeCfg), _P, _P, _P, _SZ, _I32, _P, _P, _P, _P, _P,
                           _P],
}

MOE_STATIC_SCRATCH_BYTES = 4 << 20


def lib() -> ctypes.CDLL:
    """The loaded library (built in-tree by ``python -m mixture_experts_layer_deterministic_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_deterministic_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_trace_begin.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_char_p)]
        L.moe_trace_begin.restype = ctypes.c_int
        L.moe_trace_end.argtypes = []
        L.moe_trace_end.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def moe_trace_begin(event_handles, names_buf=None):
    """Starts launch tracing into caller-created events (raw hipEvent_t handles)."""
    arr = (ctypes.c_void_p * len(event_handles))(*event_handles)
    _check(lib().moe_trace_begin(arr, len(event_handles), names_buf), "moe_trace_begin")
    return arr


def moe_trace_end() -> int:
    return lib().moe_trace_end()


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def make_cfg(T, d, E, k, I, precision=MOE_PREC_BF16, flags=0) -> MoeCfg:
    return MoeCfg(T, d, E, k, I, precision, flags)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(status, what)


def moe_query(cfg: MoeCfg) -> MoeSizes:
    out = MoeSizes()
    _check(lib().moe_query(ctypes.byref(cfg), ctypes.byref(out)), "moe_query")
    return out


def moe_route(cfg, x, w_router, logits, topk_idx, topk_w, workspace, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(logits),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(workspace), _nbytes(workspace),
                           _stream(stream)), "moe_route")


def moe_permute(cfg, topk_idx, x, ring, slot, counts, offsets, row_src, tk_row, workspace,
                stream=None):
    _check(lib().moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(ring),
                             _nbytes(ring), slot, _ptr(counts), _ptr(offsets), _ptr(row_src),
                             _ptr(tk_row), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_permute")


def moe_permute_static(cfg, topk_idx, x, ring, slot, counts, offsets, row_src, tk_row,
                       device_status, stream=None):
    _check(lib().moe_permute_static(ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(ring),
                                    _nbytes(ring), slot, _ptr(counts), _ptr(offsets),
                                    _ptr(row_src), _ptr(tk_row), _ptr(device_status),
                                    _stream(stream)), "moe_permute_static")


def _wq_bytes(wq):
    return 0 if wq is None else _nbytes(wq)


def moe_quantize_weights(cfg, w1, w2, wq, stream=None):
    _check(lib().moe_quantize_weights(ctypes.byref(cfg), _ptr(w1), _ptr(w2), _ptr(wq),
                                      _nbytes(wq), _stream(stream)), "moe_quantize_weights")


def moe_forward(cfg, ring, slot, offsets, tk_row, topk_w, w1, w2, wq, y, saved, workspace,
                stream=None):
    _check(lib().moe_forward(ctypes.byref(cfg), _ptr(ring), _nbytes(ring), slot, _ptr(offsets),
                             _ptr(tk_row), _ptr(topk_w), _ptr(w1), _ptr(w2), _ptr(wq),
                             _wq_bytes(wq), _ptr(y), _ptr(saved), _nbytes(saved),
                             _ptr(workspace), _nbytes(workspace), _stream(stream)), "moe_forward")


def moe_forward_fused(cfg, x, w_router, logits, topk_idx, topk_w, ring, slot, counts, offsets,
                      row_src, tk_row, w1, w2, y, saved, workspace, stream=None):
    _check(lib().moe_forward_fused(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(logits),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(ring), _nbytes(ring), slot,
                                   _ptr(counts), _ptr(offsets), _ptr(row_src), _ptr(tk_row),
                                   _ptr(w1), _ptr(w2), _ptr(y), _ptr(saved), _nbytes(saved),
                                   _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_forward_fused")


def moe_backward(cfg, ring, slot, offsets, row_src, tk_row, topk_idx, topk_w, w_router, w1, w2,
                 wq, saved, dy, dx, dw1, dw2, dwr, d_topk_w, accumulate, workspace, stream=None):
    _check(lib().moe_backward(ctypes.byref(cfg), _ptr(ring), _nbytes(ring), slot, _ptr(offsets),
                              _ptr(row_src), _ptr(tk_row), _ptr(topk_idx), _ptr(topk_w),
                              _ptr(w_router), _ptr(w1), _ptr(w2), _ptr(wq), _wq_bytes(wq),
                              _ptr(saved), _nbytes(saved), _ptr(dy), _ptr(dx), _ptr(dw1), _ptr(dw2),
                              _ptr(dwr), _ptr(d_topk_w), int(accumulate), _ptr(workspace),
                              _nbytes(workspace), _stream(stream)), "moe_backward")
