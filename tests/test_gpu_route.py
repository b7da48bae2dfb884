"""Bit-exact parity of the HIP routing and segment tables with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer, dev

pytestmark = pytest.mark.gpu


def _check(dl: DevLayer, x_bits: np.ndarray, x_dev=None):
    cfg = dl.inp.cfg
    idx, w, counts, offsets, sorted_ids, pos = dl.route(x_dev)
    lg = oracle.router_logits(x_bits, cfg.act_dtype, dl.inp.router_w, dl.inp.router_bias)
    ridx, rw = oracle.topk_softmax(lg, cfg.top_k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    rc, ro, rs, rp = oracle.segments(ridx, cfg.n_experts)
    np.testing.assert_array_equal(counts, rc)
    np.testing.assert_array_equal(offsets, ro)
    np.testing.assert_array_equal(sorted_ids, rs)
    np.testing.assert_array_equal(pos, rp)
    return idx


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "fp8"])
def test_route_configs(name):
    cfg = W.BY_NAME[name]
    inp = W.gen_layer(cfg, experts=[])
    dl = DevLayer(inp)
    _check(dl, inp.x)


# up to 64 tokens (one segment chunk) one block runs top-k and the segment
# tables; 65 tokens and more take the multi-launch path
@pytest.mark.parametrize("T", [1, 13, 64, 65, 300])
def test_route_ragged_token_counts(T):
    cfg = W.BY_NAME["decode"].replace(tokens=T, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    _check(DevLayer(inp), inp.x)


def test_route_small_path_wide_topk():
    # 64 tokens x top-16 = 1024 slots in the single-block routing tail
    cfg = W.BY_NAME["decode"].replace(tokens=64, top_k=16, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    _check(DevLayer(inp), inp.x)


def test_route_zero_input_and_forced_expert():
    cfg = W.BY_NAME["decode"].replace(tokens=40, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    inp.x = np.zeros_like(inp.x)
    dl = DevLayer(inp)
    idx = _check(dl, inp.x)
    # zero input: logits = bias, every token picks the same k experts
    assert (idx == idx[0]).all()
    # no bias, zero input: ties everywhere -> experts 0..k-1
    cfg2 = cfg.replace(router_bias=False)
    inp2 = W.gen_layer(cfg2, experts=[])
    inp2.x = np.zeros_like(inp2.x)
    idx2 = _check(DevLayer(inp2), inp2.x)
    assert (idx2 == np.arange(cfg.top_k)).all()


def test_route_deterministic():
    cfg = W.BY_NAME["prefill"]
    inp = W.gen_layer(cfg, experts=[])
    dl = DevLayer(inp)
    a = dl.route()
    b = dl.route()
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# The routing entry leaves the fp32 logits in its workspace right after the
# 256-byte header (an internal layout this test reads on purpose).  They must
# equal the oracle's fixed-order sums bit for bit: up to 64 tokens on the
# 32-lanes-per-pair kernel, above that on the matrix-core one (16-token x
# 32-expert tiles, ragged in tokens and, in the tiny config's 8 experts and
# 256 channels, in experts and with fewer 128-channel steps than its LDS ring
# has stages); bf16 activations at the real shapes, fp16 in the tiny config.
_LOGITS_AT = 256


def _device_logits(dl, T):
    cfg = dl.inp.cfg
    k, E = cfg.top_k, cfg.n_experts
    outs = [torch.empty(T * k, dtype=dt, device="cuda") for dt in (torch.int32, torch.float32)]
    tabs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    ws = dl.workspace(T)
    M.route(dl.desc, dl.weights, dl.x, *outs, *tabs, ws)
    torch.cuda.synchronize()
    return ws[_LOGITS_AT:_LOGITS_AT + 4 * T * E].cpu().numpy().view(np.float32).reshape(T, E)


@pytest.mark.parametrize("T", [1, 8, 13, 64, 65, 300])
@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_route_logits_bit_exact(name, T):
    cfg = W.BY_NAME[name].replace(tokens=T, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    dl = DevLayer(inp)
    got = _device_logits(dl, T)
    ref = oracle.router_logits(inp.x, cfg.act_dtype, inp.router_w, inp.router_bias)
    assert got.view(np.uint32).tolist() == ref.view(np.uint32).tolist()


@pytest.mark.parametrize("T", [79, 80, 81, 129])
@pytest.mark.parametrize("E,H", [(40, 512), (296, 1024)])
def test_route_logits_bit_exact_ragged_tiles(E, H, T):
    # the matrix-core router's ragged edges: 40 experts = one full 32-expert
    # tile and one of 8, 296 = nine full tiles and one of 8; token counts on
    # both sides of a 16-token tile boundary; 4 and 8 128-channel steps
    cfg = W.BY_NAME["decode"].replace(tokens=T, n_experts=E, hidden=H, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    got = _device_logits(DevLayer(inp), T)
    ref = oracle.router_logits(inp.x, cfg.act_dtype, inp.router_w, inp.router_bias)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name", ["prefill", "mixed_k3"])
def test_route_logits_bit_exact_prefill_shapes(name):
    # every logit of the 7168- and 2048-token layers (448 and 128 token tiles
    # of 16, 9 expert tiles of 32)
    inp = W.gen_layer(W.BY_NAME[name], experts=[])
    dl = DevLayer(inp)
    got = _device_logits(dl, inp.cfg.tokens)
    ref = oracle.router_logits(inp.x, inp.cfg.act_dtype, inp.router_w, inp.router_bias)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def _edge_inputs(T):
    """bf16 activations and fp16 router weights at the edges of the number
    formats: products in fp32's subnormal range, fp16 subnormal weights,
    products that overflow, infinities and NaN."""
    cfg = W.BY_NAME["decode"].replace(tokens=T)     # no bias: the sums are the logits
    inp = W.gen_layer(cfg, experts=[])
    rng = np.random.default_rng(5)
    H = cfg.hidden
    xf = W.bf16_bits_to_f32(inp.x).copy()
    xf[0:4] *= np.float32(2.0 ** -128)          # x * w far below fp32's normal range
    xf[4:6] *= np.float32(2.0 ** -100)
    xf[6:8] *= np.float32(2.0 ** 110)           # x * w beyond fp32's range for large w
    x = W.f32_to_bf16_bits(xf)
    x[8, rng.integers(0, H)] = 0x7F80           # +inf
    x[9, rng.integers(0, H)] = 0xFF80           # -inf
    x[10, rng.integers(0, H)] = 0x7FC0          # NaN
    x[11, :] = 0x8000                           # -0
    inp.x = x
    w = inp.router_w.copy()
    w[0:3] = (w[0:3].astype(np.float32) * np.float32(2.0 ** -10)).astype(np.float16)   # subnormal fp16
    w[3, :] = np.float16(65504.0)
    w[4, ::2] = np.float16(-65504.0)
    inp.router_w = w
    return inp


@pytest.mark.parametrize("T", [40, 96])
def test_route_logits_edge_values(T):
    # T = 40: the few-token kernel; T = 96: the matrix-core kernel.  Equal bit
    # for bit where the oracle's logit is a number, NaN where it is NaN.
    inp = _edge_inputs(T)
    got = _device_logits(DevLayer(inp), T)
    ref = oracle.router_logits(inp.x, inp.cfg.act_dtype, inp.router_w, inp.router_bias)
    nan = np.isnan(ref)
    sub = (ref != 0) & (np.abs(ref) < np.finfo(np.float32).tiny)
    assert nan.any() and np.isinf(ref).any() and sub.sum() > 100
    print(f"T={T}: {int(nan.sum())} NaN, {int(np.isinf(ref).sum())} inf, {int(sub.sum())} subnormal logits")
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
