"""The C-ABI library loads, exports every symbol the header declares, and its
host-side checks reject bad arguments before any launch (no GPU needed: every
call here returns from argument validation)."""
import ctypes as C
import os
import re

import pytest

import trellis_quantized_moe_exl3_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_exl3.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_exl3_\w+)\s*\(", text, re.M)))


def test_header_declares_binding_exports():
    assert _declared() == sorted(M.EXPORTS)


def test_library_exports_every_declared_symbol():
    l = C.CDLL(M.LIB_PATH)
    for name in _declared():
        assert hasattr(l, name), name


def test_version_and_strerror():
    assert M.version() == 2
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(M.strerror(code), str) and M.strerror(code)


def _desc(**kw):
    base = dict(hidden=4096, inter=2048, n_experts=288, top_k=8, K=2, act_dtype=M.DT_BF16,
                flags=M.HAS_SHARED | M.HAS_ROUTER_BIAS)
    base.update(kw)
    return M.make_desc(**base)


def test_workspace_size_monotone_and_sane():
    d = _desc()
    s0, s1, s2 = M.workspace_size(d, 0), M.workspace_size(d, 8), M.workspace_size(d, 7168)
    assert 0 < s0 <= s1 <= s2
    # the per-slot buffers alone are T*k*I bf16 (h rows) + T*k*H bf16 (down rows)
    assert s2 >= 7168 * 8 * (2048 * 2 + 4096 * 2)
    assert s2 < 4 * 2 ** 30


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), M.ERR_INVALID_ARG),
    (dict(inter=96), M.ERR_INVALID_ARG),
    (dict(n_experts=0), M.ERR_INVALID_ARG),
    (dict(n_experts=12), M.ERR_INVALID_ARG),
    (dict(K=5), M.ERR_UNSUPPORTED),
    (dict(K=1), M.ERR_UNSUPPORTED),
    (dict(top_k=17), M.ERR_UNSUPPORTED),
    (dict(act_dtype=M.DT_F32), M.ERR_UNSUPPORTED),
    (dict(codebook=7), M.ERR_UNSUPPORTED),
    (dict(flags=M.FORCE_GEMV | M.FORCE_MFMA), M.ERR_INVALID_ARG),
    (dict(gemv_max_rows=-1), M.ERR_INVALID_ARG),
])
def test_bad_desc_rejected(kw, code):
    n = C.c_size_t(0)
    assert M.lib().moe_exl3_workspace_size(C.byref(_desc(**kw)), 8, C.byref(n)) == code


def _fake_weights(align=256, shared=True):
    w = M.Weights()
    for p in range(3):
        w.codes[p] = 0x10000 + align * (p + 1)
        w.suh[p] = 0x20000 + align * (p + 1)
        w.svh[p] = 0x30000 + align * (p + 1)
        w.shared_w[p] = (0x40000 + align * (p + 1)) if shared else None
    w.router_w = 0x50000
    w.router_bias = 0x60000
    return w


def _layer(desc, w, x=0x100000, T=8, out=0x200000, ws=0x300000, ws_bytes=1 << 40):
    return M.lib().moe_exl3_layer(C.byref(desc), C.byref(w) if w is not None else None,
                                  x, T, out, ws, ws_bytes, None)


def test_layer_argument_checks_without_launch():
    d = _desc()
    w = _fake_weights()
    assert _layer(d, w, T=-1) == M.ERR_INVALID_ARG
    assert _layer(d, None) == M.ERR_INVALID_ARG
    assert _layer(d, w, x=None) == M.ERR_INVALID_ARG
    assert _layer(d, w, out=None) == M.ERR_INVALID_ARG
    assert _layer(d, w, ws=None) == M.ERR_INVALID_ARG
    assert _layer(d, w, x=0x100008) == M.ERR_MISALIGNED
    assert _layer(d, w, ws=0x300010) == M.ERR_MISALIGNED
    assert _layer(d, w, ws_bytes=1024) == M.ERR_WORKSPACE
    assert _layer(d, w, out=0x100000) == M.ERR_INVALID_ARG        # out aliases x
    assert _layer(d, _fake_weights(align=8)) == M.ERR_MISALIGNED
    assert _layer(d, _fake_weights(shared=False)) == M.ERR_INVALID_ARG
    w2 = _fake_weights()
    w2.router_bias = None
    assert _layer(d, w2) == M.ERR_INVALID_ARG
    assert _layer(_desc(flags=M.FP8_MFMA), w) == M.ERR_UNSUPPORTED
    assert _layer(_desc(), w, T=0) == M.OK                          # no-op, no launch
    assert _layer(_desc(), w, T=2 ** 28) == M.ERR_UNSUPPORTED       # T*k >= 2^31


def test_route_and_decode_argument_checks():
    d = _desc()
    w = _fake_weights()
    l = M.lib()
    assert l.moe_exl3_route(C.byref(d), C.byref(w), 0x100000, 8, None, None, None, None, None,
                            None, 0x300000, 1 << 40, None) == M.ERR_INVALID_ARG
    assert l.moe_exl3_route(C.byref(d), C.byref(w), 0x100000, 8, 0x400000, None, None, None,
                            None, None, 0x300000, 16, None) == M.ERR_WORKSPACE
    assert l.moe_exl3_decode(0x1000, 48, 64, 5, 1, 0, 0x2000, 0, None) == M.ERR_UNSUPPORTED
    assert l.moe_exl3_decode(0x1000, 40, 64, 2, 1, 0, 0x2000, 0, None) == M.ERR_INVALID_ARG
    assert l.moe_exl3_decode(0x1000, 48, 64, 2, 1, 0, 0x2004, 0, None) == M.ERR_MISALIGNED
    assert l.moe_exl3_decode(0x1000, 48, 64, 2, 1, 0, 0x2000, 9, None) == M.ERR_UNSUPPORTED
    # the one-block MFMA operand mode exists for the mcg codebook only
    assert l.moe_exl3_decode(0x1000, 48, 64, 2, 1, 1, 0x2000, M.DT_MFMA_BIASED_F16, None) == M.ERR_UNSUPPORTED


def test_bench_event_helper_declares_pointer_arguments():
    # the benchmark's HIP event calls take event and stream handles; without
    # declared argument types ctypes passes a Python int as a 32-bit C int,
    # which truncates the handles (a graph-timing call made before any eager
    # timing call crashed that way)
    import bench
    try:
        hip = bench.Hip()
    except OSError:
        pytest.skip("HIP runtime library not loadable here")
    assert hip.l.hipEventRecord.argtypes == [C.c_void_p, C.c_void_p]
    assert hip.l.hipEventElapsedTime.argtypes == [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    assert hip.l.hipEventDestroy.argtypes == [C.c_void_p]
