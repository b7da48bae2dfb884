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
DT_F32, DT_F16, DT_BF16, DT_FP8, DT_GEMV_F16, DT_MFMA_BIASED_F16 = 0, 1, 2, 3, 4, 5
CB_MCG, CB_MCG_E4M3 = 0, 1
HAS_SHARED, HAS_ROUTER_BIAS, FORCE_GEMV, FORCE_MFMA, FP8_MFMA = 1, 2, 4, 8, 16
DEBUG_CHECKS, DETERMINISTIC_COMBINE = 32, 64
HADAMARD, SHARED_TRELLIS, PER_TENSOR_K = 128, 256, 512
# status word of a workspace (int32 at byte STATUS_OFFSET)
STATUS_OFFSET = 8
(STATUS_BAD_INDEX, STATUS_TILE_OVERFLOW, STATUS_ACT_RANGE, STATUS_COUNTS, STATUS_TABLES,
 STATUS_NONFINITE_X, STATUS_BAD_WIDTH) = (1, 2, 4, 8, 16, 32, 64)

# every symbol the header declares
EXPORTS = ("moe_exl3_version", "moe_exl3_strerror", "moe_exl3_workspace_size",
           "moe_exl3_layer", "moe_exl3_layer_profiled", "moe_exl3_route", "moe_exl3_decode",
           "moe_exl3_repack", "moe_exl3_expand_block_scales", "moe_exl3_layer_noalloc")
SCRATCH_BYTES = 64 << 20
ORDER_ROWMAJOR, ORDER_COLMAJOR, ORDER_COLGROUPS128 = 0, 1, 2
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
                ("shared_w", C.c_void_p * 3), ("signs", C.c_void_p), ("code_tab", C.c_void_p),
                ("k_tab", C.c_void_p)]


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
        l.moe_exl3_layer_noalloc.argtypes = [C.POINTER(Desc), C.POINTER(Weights), C.c_void_p, C.c_int64,
                                             C.c_void_p, C.c_void_p]
        l.moe_exl3_repack.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_void_p]
        l.moe_exl3_expand_block_scales.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                                   C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.c_void_p]
        for f in ("moe_exl3_workspace_size", "moe_exl3_layer", "moe_exl3_layer_profiled",
                  "moe_exl3_route", "moe_exl3_decode", "moe_exl3_repack", "moe_exl3_expand_block_scales",
                  "moe_exl3_layer_noalloc"):
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
                 shared: Optional[Sequence] = None, signs=None, code_tab=None, k_tab=None) -> Weights:
    """Weights struct from device tensors (the tensors must outlive its use).
    signs: int8 [2][H]; code_tab: int64 [3][EA] device addresses of the
    per-tensor codes; k_tab: int32 [3][EA] widths."""
    w = Weights()
    w.signs = _ptr(signs)
    w.code_tab = _ptr(code_tab)
    w.k_tab = _ptr(k_tab)
    for p in range(3):
        w.codes[p] = _ptr(codes[p]) if codes is not None else None
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


def _check_acts(desc: Desc, what: str, *tensors) -> None:
    """x and out must be contiguous 2-D device tensors [T][hidden] of a 2-byte
    dtype (bf16 or fp16 data, raw int16 accepted) matching act_dtype, all of
    the same shape: the kernels index them as such."""
    import torch
    want = {DT_BF16: (torch.bfloat16, torch.int16), DT_F16: (torch.float16, torch.int16)}[desc.act_dtype]
    shape = None
    for t in tensors:
        if t.dim() != 2 or t.shape[1] != desc.hidden:
            raise ValueError(f"{what}: expected [T][{desc.hidden}], got {tuple(t.shape)}")
        if t.dtype not in want:
            raise ValueError(f"{what}: dtype {t.dtype} does not match act_dtype {desc.act_dtype}")
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{what}: tensors must be contiguous and on the GPU")
        if shape is not None and t.shape != shape:
            raise ValueError(f"{what}: x and out shapes differ")
        shape = t.shape


def _check_ws(workspace) -> None:
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")


def status(workspace) -> int:
    """The status word of the last call that used `workspace` (synchronises)."""
    import torch
    torch.cuda.synchronize()
    return int(workspace.view(torch.uint8)[STATUS_OFFSET:STATUS_OFFSET + 4].cpu().view(torch.int32).item())


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def layer(desc: Desc, weights: Weights, x, out, workspace, stream=None) -> None:
    """out = MoE layer(x); x, out: [T][H] device tensors of the activation dtype."""
    _check_acts(desc, "layer", x, out)
    _check_ws(workspace)
    T = x.shape[0]
    _check(lib().moe_exl3_layer(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(out),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "moe_exl3_layer")


def layer_noalloc(desc: Desc, weights: Weights, x, out, stream=None) -> None:
    """layer() with the library's own per-GPU scratch array as the workspace
    (moe_exl3_layer_noalloc): allocates nothing."""
    _check_acts(desc, "layer_noalloc", x, out)
    T = x.shape[0]
    _check(lib().moe_exl3_layer_noalloc(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(out),
                                        _stream(stream)), "moe_exl3_layer_noalloc")


def layer_profiled(desc: Desc, weights: Weights, x, out, workspace, events, stream=None) -> None:
    """layer() recording events[i] (hipEvent_t handles) before launch step i."""
    _check_acts(desc, "layer_profiled", x, out)
    _check_ws(workspace)
    T = x.shape[0]
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().moe_exl3_layer_profiled(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(out),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream), arr, len(events)),
           "moe_exl3_layer_profiled")


def route(desc: Desc, weights: Weights, x, idx, w=None, counts=None, offsets=None,
          sorted_ids=None, pos=None, workspace=None, stream=None) -> None:
    """Routing tables of x (moe_exl3_route); outputs are int32/fp32 device
    tensors of T*k (idx, w, sorted_ids, pos), E (counts) or E+1 (offsets)
    elements, or None (idx is required)."""
    _check_acts(desc, "route", x)
    _check_ws(workspace)
    T = x.shape[0]
    n, E = T * desc.top_k, desc.n_experts
    for t, size, what in ((idx, n, "idx"), (w, n, "w"), (counts, E, "counts"), (offsets, E + 1, "offsets"),
                          (sorted_ids, n, "sorted_ids"), (pos, n, "pos")):
        if t is None:
            if what == "idx":
                raise ValueError("route: idx is required")
            continue
        if not t.is_cuda or not t.is_contiguous() or t.numel() < size or t.element_size() != 4:
            raise ValueError(f"route: {what} must be a contiguous 4-byte GPU tensor of >= {size} elements")
    _check(lib().moe_exl3_route(C.byref(desc), C.byref(weights), _ptr(x), T, _ptr(idx), _ptr(w),
                                _ptr(counts), _ptr(offsets), _ptr(sorted_ids), _ptr(pos),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "moe_exl3_route")


def decode(codes, n_in: int, n_out: int, K: int, mcg: int, codebook: int, dst, dst_dtype: int,
           stream=None) -> None:
    """Dense [n_in][n_out] decode of one trellis-coded matrix into `dst`."""
    nbytes = n_in * n_out * (4 if dst_dtype == DT_F32 else 1 if dst_dtype == DT_FP8 else 2)
    words = (n_in // 16) * (n_out // 16) * 16 * K
    if not (dst.is_cuda and codes.is_cuda and dst.is_contiguous() and codes.is_contiguous()):
        raise ValueError("decode: codes and dst must be contiguous GPU tensors")
    if dst.numel() * dst.element_size() < nbytes or codes.numel() * codes.element_size() < 2 * words:
        raise ValueError("decode: codes or dst smaller than the matrix")
    _check(lib().moe_exl3_decode(_ptr(codes), n_in, n_out, K, mcg & 0xFFFFFFFF, codebook,
                                 _ptr(dst), dst_dtype, _stream(stream)), "moe_exl3_decode")


def repack(src, dst, count: int, n_in: int, n_out: int, K: int, src_order: int, stream=None) -> None:
    """Reorder the tile grids of `count` trellis tensors from `src_order` into
    the kernels' row-major grid (moe_exl3_repack)."""
    words = count * (n_in // 16) * (n_out // 16) * 16 * K
    for t, what in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < 2 * words:
            raise ValueError(f"repack: {what} must be a contiguous GPU tensor of >= {2 * words} bytes")
    _check(lib().moe_exl3_repack(_ptr(src), _ptr(dst), count, n_in, n_out, K, src_order, _stream(stream)),
           "moe_exl3_repack")


def expand_block_scales(block, n_trellis: int, hidden: int, inter: int, suh: Sequence, svh: Sequence,
                        stream=None) -> None:
    """Per-channel side vectors from the block table [n_trellis][3][hidden/128]
    (moe_exl3_expand_block_scales)."""
    if block.numel() < n_trellis * 3 * (hidden // 128):
        raise ValueError("expand_block_scales: block table too small")
    for p in range(3):
        n_in, n_out = (hidden, inter) if p < 2 else (inter, hidden)
        if suh[p].numel() < n_trellis * n_in or svh[p].numel() < n_trellis * n_out:
            raise ValueError("expand_block_scales: side vector too small")
    sp = (C.c_void_p * 3)(*[_ptr(t) for t in suh])
    vp = (C.c_void_p * 3)(*[_ptr(t) for t in svh])
    _check(lib().moe_exl3_expand_block_scales(_ptr(block), n_trellis, hidden, inter, sp, vp, _stream(stream)),
           "moe_exl3_expand_block_scales")
