"""CPU oracle for the EXL3 trellis-coded MoE layer -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  The product path never touches it.  The
arithmetic lives in `oracle.c` (plain C, built with gcc); this module only
builds it and marshals numpy arrays.  It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle_moe.so")

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (strict IEEE: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        l = C.CDLL(build())
        l.orc_mcg_value.argtypes = [C.c_uint32, C.c_uint32]
        l.orc_mcg_value.restype = C.c_int
        l.orc_stream_states.argtypes = [_u16p, C.c_int, C.c_int, _u16p]
        l.orc_e4m3_rne.argtypes = [C.c_double]
        l.orc_e4m3_rne.restype = C.c_double
        l.orc_codebook_value.argtypes = [C.c_uint32, C.c_uint32, C.c_int]
        l.orc_codebook_value.restype = C.c_double
        l.orc_decode_tile.argtypes = [_u16p, C.c_int, C.c_uint32, C.c_int, _f32p]
        l.orc_decode_matrix.argtypes = [_u16p, C.c_int, C.c_int, C.c_int, C.c_uint32, C.c_int, _f32p]
        l.orc_router_logits.argtypes = [_u16p, C.c_int, C.c_int64, C.c_int, _u16p, C.c_void_p,
                                        C.c_int, _f32p]
        l.orc_topk_softmax.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, _i32p, _f64p]
        l.orc_segments.argtypes = [_i32p, C.c_int64, C.c_int, C.c_int, _i32p, _i32p, _i32p, _i32p]
        l.orc_layer.argtypes = [
            C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_uint32, C.c_int, C.c_int,
            _u16p, _i64p, C.c_int64, _u16p, C.c_void_p,
            C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
            C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, _i32p, _f64p, _f64p, C.c_int]
        l.orc_tile_position.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int]
        l.orc_tile_position.restype = C.c_int64
        l.orc_decode_matrix_order.argtypes = [_u16p, C.c_int, C.c_int, C.c_int, C.c_uint32, C.c_int,
                                              C.c_int, _f32p]
        l.orc_decode_matrix_order.restype = C.c_int
        l.orc_expand_block_scales.argtypes = [_u16p, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_void_p),
                                              C.POINTER(C.c_void_p)]
        l.orc_sylvester.argtypes = [C.c_int, np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")]
        l.orc_rotate.argtypes = [_f64p, C.c_int, C.c_void_p]
        l.orc_layer.restype = C.c_int
        l.orc_f16_to_double.argtypes = [C.c_uint16]
        l.orc_f16_to_double.restype = C.c_double
        l.orc_bf16_to_double.argtypes = [C.c_uint16]
        l.orc_bf16_to_double.restype = C.c_double
        _lib = l
    return _lib


def _u16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16) if a.dtype != np.uint16 else np.ascontiguousarray(a)


# --------------------------------------------------------------------- decode
def mcg_value(state: int, mcg: int) -> int:
    return lib().orc_mcg_value(state, mcg)


def value_table(mcg: int) -> np.ndarray:
    """v(s) for all 65536 states (int32)."""
    l = lib()
    return np.array([l.orc_mcg_value(s, mcg) for s in range(65536)], dtype=np.int32)


def stream_states(words: np.ndarray, K: int) -> np.ndarray:
    w = _u16(words)
    n = 16 * w.size // K
    out = np.zeros(n, dtype=np.uint16)
    lib().orc_stream_states(w, w.size, K, out)
    return out


def e4m3_rne(x: float) -> float:
    return lib().orc_e4m3_rne(float(x))


def codebook_value(state: int, mcg: int, codebook: int) -> float:
    return lib().orc_codebook_value(state, mcg, codebook)


def decode_tile(words: np.ndarray, K: int, mcg: int, codebook: int = 0) -> np.ndarray:
    out = np.zeros(256, dtype=np.float32)
    lib().orc_decode_tile(_u16(words), K, mcg, codebook, out)
    return out


def decode_matrix(codes: np.ndarray, n_in: int, n_out: int, K: int, mcg: int,
                  codebook: int = 0) -> np.ndarray:
    """Dense [in][out] fp32 matrix of decoded values (before side vectors)."""
    c = _u16(codes).reshape(-1)
    assert c.size == (n_in // 16) * (n_out // 16) * 16 * K
    out = np.zeros((n_in, n_out), dtype=np.float32)
    lib().orc_decode_matrix(c, n_in, n_out, K, mcg, codebook, out)
    return out


def tile_position(order: int, n_in: int, n_out: int, tk: int, tn: int) -> int:
    """Position (in tiles) of tile (tk, tn) in a stored tile order."""
    return lib().orc_tile_position(order, n_in, n_out, tk, tn)


def decode_matrix_order(codes: np.ndarray, n_in: int, n_out: int, K: int, mcg: int,
                        codebook: int, order: int) -> np.ndarray:
    """Dense [in][out] fp32 matrix of a projection stored in tile `order`."""
    c = _u16(codes).reshape(-1)
    assert c.size == (n_in // 16) * (n_out // 16) * 16 * K
    out = np.zeros((n_in, n_out), dtype=np.float32)
    if lib().orc_decode_matrix_order(c, n_in, n_out, K, mcg, codebook, order, out) != 0:
        raise ValueError("unknown tile order or shape")
    return out


def expand_block_scales(block: np.ndarray, H: int, I: int):
    """(suh[3], svh[3]) fp16 side vectors from an fp16 block table
    [EA][3][H/128] (exlr8 "Index slices" reading)."""
    b = np.ascontiguousarray(block, dtype=np.float16)
    EA = b.shape[0]
    assert b.shape == (EA, 3, H // 128)
    suh = [np.zeros((EA, H), np.float16), np.zeros((EA, H), np.float16), np.zeros((EA, I), np.float16)]
    svh = [np.zeros((EA, I), np.float16), np.zeros((EA, I), np.float16), np.zeros((EA, H), np.float16)]
    sp = (C.c_void_p * 3)(*[a.ctypes.data for a in suh])
    vp = (C.c_void_p * 3)(*[a.ctypes.data for a in svh])
    lib().orc_expand_block_scales(_u16(b), EA, H, I, sp, vp)
    return suh, svh


# ------------------------------------------------------------------ rotation
def sylvester(n: int) -> np.ndarray:
    """The n x n Hadamard matrix by Sylvester's construction (int8)."""
    h = np.zeros((n, n), dtype=np.int8)
    lib().orc_sylvester(n, h)
    return h


def rotate(v: np.ndarray, signs: Optional[np.ndarray] = None) -> np.ndarray:
    """Block rotation (128-blocks, orthonormal) of each row of v, after an
    optional elementwise sign vector."""
    a = np.array(v, dtype=np.float64, order="C", copy=True)
    rows = a.reshape(-1, a.shape[-1])
    s = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    for r in rows:
        lib().orc_rotate(r, r.size, None if s is None else s.ctypes.data)
    return a


# -------------------------------------------------------------------- routing
def router_logits(x_bits: np.ndarray, act_dtype: int, router_w: np.ndarray,
                  bias: Optional[np.ndarray]) -> np.ndarray:
    x = _u16(x_bits)
    T, H = x.shape
    E = router_w.shape[0]
    out = np.zeros((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().orc_router_logits(x, act_dtype, T, H, _u16(router_w),
                            None if b is None else b.ctypes.data, E, out)
    return out


def topk_softmax(logits: np.ndarray, k: int):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    lib().orc_topk_softmax(lg, T, E, k, idx, w)
    return idx, w


def segments(idx: np.ndarray, E: int):
    i = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = i.shape
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_ids = np.zeros(T * k, dtype=np.int32)
    pos = np.zeros(T * k, dtype=np.int32)
    lib().orc_segments(i, T, k, E, counts, offsets, sorted_ids, pos)
    return counts, offsets, sorted_ids, pos


# ---------------------------------------------------------------------- layer
def layer(inp, tokens: Optional[Sequence[int]] = None, nthreads: int = 0,
          codes: Optional[Sequence] = None, present=None):
    """Layer output (fp64) for the given token subset of a `workloads.LayerInputs`.

    Returns (idx [n][k] int32, w [n][k] fp64, out [n][H] fp64).  `codes`
    overrides inp.codes: 3 sequences indexed by expert ([E][words] arrays or
    lists of per-expert arrays) or 3 dicts {expert: words}.  Experts missing
    from a dict, or outside `present`, are passed as NULL and routing a
    selected token to one of them is an error.  With per-tensor widths
    (inp.ktab), sign vectors (inp.signs) or a trellis shared expert
    (cfg.shared_trellis, expert index E) the oracle applies them.
    """
    cfg = inp.cfg
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    EA = cfg.n_trellis
    T = inp.x.shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    assert tok.size == 0 or (tok.min() >= 0 and tok.max() < T)
    cds = inp.codes if codes is None else codes
    ptrs = (C.c_void_p * (3 * EA))()
    keep = []
    for p in range(3):
        arr = cds[p]
        for e in range(EA):
            if present is not None and e not in present and e < E:
                continue
            if isinstance(arr, dict):
                if e not in arr:
                    continue
                row = np.ascontiguousarray(arr[e], dtype=np.uint16)
            else:
                row = arr[e]
                assert row.dtype == np.uint16 and row.flags.c_contiguous
            assert row.size == cfg.words_of(p, e, inp.ktab)
            keep.append(row)
            ptrs[p * EA + e] = row.ctypes.data
    suh = [np.ascontiguousarray(a) for a in inp.suh]
    svh = [np.ascontiguousarray(a) for a in inp.svh]
    for p in range(3):
        assert suh[p].shape[0] == EA and svh[p].shape[0] == EA
    suh_p = (C.c_void_p * 3)(*[a.ctypes.data for a in suh])
    svh_p = (C.c_void_p * 3)(*[a.ctypes.data for a in svh])
    shared_arr = None
    shared_p = None
    if inp.shared is not None:
        shared_arr = [np.ascontiguousarray(a) for a in inp.shared]
        shared_p = (C.c_void_p * 3)(*[a.ctypes.data for a in shared_arr])
    ktab = None if inp.ktab is None else np.ascontiguousarray(inp.ktab, dtype=np.int32)
    if ktab is not None:
        assert ktab.shape == (3, EA)
    signs = None if inp.signs is None else np.ascontiguousarray(inp.signs, dtype=np.int8)
    if signs is not None:
        assert signs.shape == (2, H)
    idx = np.zeros((tok.size, k), dtype=np.int32)
    w = np.zeros((tok.size, k), dtype=np.float64)
    out = np.zeros((tok.size, H), dtype=np.float64)
    bias = None if inp.router_bias is None else np.ascontiguousarray(inp.router_bias, np.float32)
    rc = lib().orc_layer(
        H, I, E, k, cfg.K, cfg.mcg, cfg.codebook, cfg.act_dtype,
        _u16(inp.x), tok, tok.size, _u16(inp.router_w),
        None if bias is None else bias.ctypes.data,
        ptrs, suh_p, svh_p,
        C.cast(shared_p, C.c_void_p) if shared_p is not None else None,
        None if ktab is None else ktab.ctypes.data,
        None if signs is None else signs.ctypes.data,
        1 if cfg.shared_trellis else 0,
        idx, w, out, nthreads)
    if rc != 0:
        raise RuntimeError("oracle layer: codes of a needed expert are missing, or a width is invalid")
    return idx, w, out


def route_tokens(inp, tokens: Sequence[int]):
    """Oracle routing (idx, w) for a token subset, without the expert math."""
    x = _u16(inp.x)[np.asarray(tokens, dtype=np.int64)]
    lg = router_logits(x, inp.cfg.act_dtype, inp.router_w, inp.router_bias)
    return topk_softmax(lg, inp.cfg.top_k)
