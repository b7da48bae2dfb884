"""Python binding of libmoe_exl3.so (MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the HIP library
behind the C ABI declared in include/moe_exl3.h.  PyTorch provides device
memory and streams.  There is no fallback: if the library is missing or no
GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_exl3.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_MISALIGNED, ERR_HIP = 0, -1, -2, -3, -4, -5
DT_F32, DT_F16, DT_BF16, DT_FP8 = 0, 1, 2, 3
CB_MCG, CB_MCG_E4M3 = 0, 1
HAS_SHARED, HAS_ROUTER_BIAS, FORCE_GEMV, FORCE_MFMA, FP8_MFMA = 1, 2, 4, 8, 16

# every symbol the header declares
EXPORTS = ("moe_exl3_version", "moe_exl3_strerror", "moe_exl3_workspace_size",
           "moe_exl3_layer", "moe_exl3_layer_profiled", "moe_exl3_route", "moe_exl3_decode")
# launch steps of moe_exl3_layer_profiled (events[i] is recorded before step i)
STEPS = ("route_logits", "topk", "segments", "convert_x", "gemv_gateup", "mfma_gateup",
         "gemv_down", "mfma_down", "shared", "combine")
STEP_END = len(STEPS)


class Desc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("K", C.c_int32), ("codebook", C.c_int32),
                ("mcg", C.c_uint32), ("act_dtype", C.c_int32), ("flags", C.c_uint32),
                ("gemv_max_rows", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [("codes", C.c_void_p * 3), ("suh", C.c_void_p * 3), ("svh", C.c_void_p * 3),
                ("router_w", C.c_void_p), ("router_bias", C.c_void_p),
                ("shared_w", C.c_void_p * 3)]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def lib():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m trellis_quantized_moe_exl3_amd.build`")
        l = C.CDLL(LIB_PATH)
        l.moe_exl3_version.restype = C.c_int
        l.moe_exl3_strerror.argtypes = [C.c_int]
        l.moe_exl3_strerror.restype = C.c_char_p
        l.moe_exl3_workspace_size.argtypes = [C.POINTER(Desc), C.c_int64, C.POINTER(C.c_size_t)]
        l.moe_exl3_layer.argtypes = [C.POINTER(Desc), C.POINTER(Weights), C.c_void_p, C.c_int64,
                                     C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        l.moe_exl3_layer_profiled.argtypes = [
            C.POINTER(Desc), C.POINTER(Weights), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
            C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p), C.c_int]
        l.moe_exl3_route.argtypes = [C.POINTER(Desc), C.POINTER(Weights), C.c_void_p, C.c_int64,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        l.moe_exl3_decode.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_uint32,
                                      C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]
        for f in ("moe_exl3_workspace_size", "moe_exl3_layer", "moe_exl3_layer_profiled",
                  "moe_exl3_route", "moe_exl3_decode"):
            getattr(l, f).restype = C.c_int
        _lib = l
    return _lib


def version() -> int:
    return lib().moe_exl3_version()


def strerror(code: int) -> str:
    return lib().moe_exl3_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise MoeError(rc, what)


def make_desc(hidden, inter, n_experts, top_k, K, codebook=CB_MCG, mcg=0x9E3779B1,
              act_dtype=DT_BF16, flags=0, gemv_max_rows=0) -> Desc:
    return Desc(hidden, inter, n_experts, top_k, K, codebook, mcg & 0xFFFFFFFF, act_dtype, flags,
                gemv_max_rows)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def make_weights(codes: Sequence, suh: Sequence, svh: Sequence, router_w, router_bias=None,
                 shared: Optional[Sequence] = None) -> Weights:
    """Weights struct from device tensors (the tensors must outlive its use)."""
    w = Weights()
    for p in range(3):
        w.codes[p] = _ptr(codes[p])
        w.suh[p] = _ptr(suh[p])
        w.svh[p] = _ptr(svh[p])
        w.shared_w[p] = _ptr(shared[p]) if shared is not None else None
    w.router_w = _ptr(router_w)
    w.router_bias = _ptr(router_bias)
    return w


def workspace_size(desc: Desc, max_tokens: int) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_exl3_workspace_size(C.byref(desc), max_tokens, C.byref(n)), "workspace_size")
    return n.value


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def layer(desc: Desc, weights: Weights, x, out, workspace, stream=None) -> None:
    """out = MoE layer(x); x, out: [T][H] device tensors of the activation dtype."""
    T = x.shape[0]
    _check(lib().moe_exl3_layer(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(out),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "moe_exl3_layer")


def layer_profiled(desc: Desc, weights: Weights, x, out, workspace, events, stream=None) -> None:
    """layer() recording events[i] (hipEvent_t handles) before launch step i."""
    T = x.shape[0]
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().moe_exl3_layer_profiled(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(out),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream), arr, len(events)),
           "moe_exl3_layer_profiled")


def route(desc: Desc, weights: Weights, x, idx, w=None, counts=None, offsets=None,
          sorted_ids=None, pos=None, workspace=None, stream=None) -> None:
    T = x.shape[0]
    _check(lib().moe_exl3_route(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(idx), _ptr(w),
                                _ptr(counts), _ptr(offsets), _ptr(sorted_ids), _ptr(pos),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "moe_exl3_route")


def decode(codes, n_in: int, n_out: int, K: int, mcg: int, codebook: int, dst, dst_dtype: int,
           stream=None) -> None:
    """Dense [n_in][n_out] decode of one trellis-coded matrix into `dst`."""
    _check(lib().moe_exl3_decode(_ptr(codes), n_in, n_out, K, mcg & 0xFFFFFFFF, codebook,
                                 _ptr(dst), dst_dtype, _stream(stream)), "moe_exl3_decode")
