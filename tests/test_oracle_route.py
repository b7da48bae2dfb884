"""Pins of the oracle's routing (fp32 logits in a fixed order, top-k, softmax)
and segment tables, against hand-derived values, library routines and
invariants."""
import numpy as np
import pytest

import oracle
import workloads as W

F16_ONE = 0x3C00
F16_TINY = 0x0001          # 2^-24, the smallest fp16 subnormal
BF16_ONE = 0x3F80
BF16_TINY = 0x3380         # 2^-24 in bf16


def _one_expert_w(H):
    return np.full((1, H), 1.0, dtype=np.float16)


@pytest.mark.parametrize("dt,one,tiny", [(W.DT_F16, F16_ONE, F16_TINY), (W.DT_BF16, BF16_ONE, BF16_TINY)])
def test_fixed_order_hand_cases(dt, one, tiny):
    H = 128
    Wr = _one_expert_w(H)
    # x[0] = 1, x[1] = x[3] = 2^-24.  The tree adds lanes 1 and 3 first
    # (d = 2: 2^-23), then lane 1 into lane 0 (d = 1): 1 + 2^-23 exactly.
    # A left-to-right sum would round 1 + 2^-24 back to 1 twice.
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, 0], x[0, 1], x[0, 3] = one, tiny, tiny
    lg = oracle.router_logits(x, dt, Wr, None)
    assert lg[0, 0] == np.float32(1 + 2 ** -23)
    # x[0] = x[64] = 2^-24 share lane 0 (i = 0, 1): 2^-23; x[1] = 1 in lane 1;
    # d = 1 gives 1 + 2^-23.
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, 0], x[0, 64], x[0, 1] = tiny, tiny, one
    lg = oracle.router_logits(x, dt, Wr, None)
    assert lg[0, 0] == np.float32(1 + 2 ** -23)
    # x[0] = 1, x[64] = 2^-24 in lane 0: the running sum 1 + 2^-24 is a tie and
    # rounds to even (1.0); x[32] = 2^-24 joins at d = 32: again a tie -> 1.0
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, 0], x[0, 64], x[0, 32] = one, tiny, tiny
    lg = oracle.router_logits(x, dt, Wr, np.array([0.5], dtype=np.float32))
    assert lg[0, 0] == np.float32(1.5)


def _libm_fmaf():
    import ctypes
    import ctypes.util
    libm = ctypes.CDLL(ctypes.util.find_library("m"))
    f = libm.fmaf
    f.restype = ctypes.c_float
    f.argtypes = [ctypes.c_float] * 3
    return f


@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_F16])
def test_fused_steps_match_libm_fmaf(dt):
    # Every accumulation step is one fused multiply-add.  Reference: the C
    # library's fmaf (correctly rounded x * w + p) in the same order, then the
    # fp32 halving tree, on activations and weights that make products normal,
    # fp32-subnormal (where a separately rounded product would differ),
    # overflowing, infinite and NaN.
    fmaf = _libm_fmaf()
    rng = np.random.default_rng(11)
    H, E = 128, 5
    xf = rng.standard_normal((6, H)).astype(np.float32)
    xf[1] *= np.float32(2.0 ** -120 if dt == W.DT_BF16 else 2.0 ** -12)
    xf[2] *= np.float32(2.0 ** -130 if dt == W.DT_BF16 else 2.0 ** -14)
    xf[3] *= np.float32(2.0 ** 100 if dt == W.DT_BF16 else 2.0 ** 10)
    if dt == W.DT_BF16:
        x = W.f32_to_bf16_bits(xf)
        inf, nan = 0x7F80, 0x7FC0
    else:
        x = xf.astype(np.float16).view(np.uint16).copy()
        inf, nan = 0x7C00, 0x7E00
    x[4, 17] = inf
    x[5, 90] = nan
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float16)
    Wr[1] = (Wr[1].astype(np.float32) * np.float32(2.0 ** -12)).astype(np.float16)   # fp16 subnormals
    Wr[2, ::3] = np.float16(65504.0)
    lg = oracle.router_logits(x, dt, Wr, None)
    xv = W.act_bits_to_f32(x, dt)
    wv = Wr.astype(np.float32)
    ref = np.zeros_like(lg)
    differs = 0
    for t in range(x.shape[0]):
        for e in range(E):
            p = [0.0] * 64
            q = np.zeros(64, dtype=np.float32)   # separately rounded product, for contrast
            for i in range(H // 64):
                for l in range(64):
                    a, b = float(xv[t, 64 * i + l]), float(wv[e, 64 * i + l])
                    p[l] = fmaf(a, b, p[l])
                    with np.errstate(all="ignore"):
                        q[l] = np.float32(q[l] + np.float32(np.float32(a) * np.float32(b)))
            v = np.array(p, dtype=np.float32)
            d = 32
            while d >= 1:
                with np.errstate(all="ignore"):
                    v[:d] = v[:d] + v[d:2 * d]
                    q[:d] = q[:d] + q[d:2 * d]
                d //= 2
            ref[t, e] = v[0]
            differs += int(not (np.isnan(q[0]) and np.isnan(v[0])) and q[0].view(np.uint32) != v[0].view(np.uint32))
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(lg), nan)
    np.testing.assert_array_equal(lg[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert nan.any() and np.isinf(ref).any()
    if dt == W.DT_BF16:
        # bf16 activations reach products below fp32's normal range, where a
        # separately rounded product parts from the fused step
        assert differs > 0
    else:
        # fp16 x fp16 products are at least 2^-48: always exact in fp32, so
        # the two readings coincide
        assert differs == 0


def test_logits_close_to_exact_dot():
    cfg = W.CONFIGS[1]
    x = W.gen_x(cfg)[:4]
    Wr = W.gen_router_w(cfg)
    b = np.random.default_rng(0).standard_normal(cfg.n_experts).astype(np.float32)
    lg = oracle.router_logits(x, cfg.act_dtype, Wr, b)
    xf = W.act_bits_to_f32(x, cfg.act_dtype).astype(np.float64)
    prod = xf @ Wr.astype(np.float64).T
    bound = (np.abs(xf) @ np.abs(Wr.astype(np.float64)).T) * 2.0 ** -24 * 80
    assert (np.abs(lg - (prod + b)) <= bound + np.abs(prod + b) * 2.0 ** -23).all()


def test_topk_matches_stable_argsort_and_ties():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 40)).astype(np.float32)
    lg[:, 5] = lg[:, 7] = lg[:, 30] = 10.0   # a three-way tie at the top
    idx, w = oracle.topk_softmax(lg, 6)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :6]
    np.testing.assert_array_equal(idx, ref)
    assert (idx[:, :3] == [5, 7, 30]).all()
    # weights: sum to one, follow the logit order, ratios are exp differences
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (np.diff(w, axis=1) <= 1e-15).all()
    l_sel = np.take_along_axis(lg, idx, axis=1).astype(np.float64)
    np.testing.assert_allclose(w[:, 1:] / w[:, :1], np.exp(l_sel[:, 1:] - l_sel[:, :1]), rtol=1e-12)


def test_zero_input_routes_to_first_experts():
    cfg = W.CONFIGS[0]
    x = np.zeros((3, cfg.hidden), dtype=np.uint16)
    lg = oracle.router_logits(x, cfg.act_dtype, W.gen_router_w(cfg), None)
    assert (lg == 0).all()
    idx, w = oracle.topk_softmax(lg, cfg.top_k)
    assert (idx == np.arange(cfg.top_k)).all()
    assert (w == 1.0 / cfg.top_k).all()


def test_segments_match_library_sort():
    rng = np.random.default_rng(2)
    E, T, k = 37, 301, 5
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[idx == 3] = 4  # experts with zero rows exist; duplicates inside a row are allowed here
    counts, offsets, sorted_ids, pos = oracle.segments(idx, E)
    flat = idx.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(sorted_ids, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(pos[sorted_ids], np.arange(T * k))
    assert counts[3] == 0


def test_routing_of_workloads_is_skewed_with_bias():
    cfg = W.CONFIGS[2]
    x = W.gen_x(cfg)[:512]
    lg = oracle.router_logits(x, cfg.act_dtype, W.gen_router_w(cfg), W.gen_router_bias(cfg))
    idx, _ = oracle.topk_softmax(lg, cfg.top_k)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
    assert counts.max() > 8 * np.median(counts[counts > 0])
