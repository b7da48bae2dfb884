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
# 32-lanes-per-pair kernel, above that on the register-tiled one; bf16
# activations at the real shapes, fp16 in the tiny config.
_LOGITS_AT = 256


@pytest.mark.parametrize("T", [1, 8, 13, 64, 65, 300])
@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_route_logits_bit_exact(name, T):
    cfg = W.BY_NAME[name].replace(tokens=T, router_bias=True)
    inp = W.gen_layer(cfg, experts=[])
    dl = DevLayer(inp)
    k, E = cfg.top_k, cfg.n_experts
    outs = [torch.empty(T * k, dtype=dt, device="cuda")
            for dt in (torch.int32, torch.float32)]
    tabs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    ws = dl.workspace(T)
    M.route(dl.desc, dl.weights, dl.x, *outs, *tabs, ws)
    torch.cuda.synchronize()
    got = ws[_LOGITS_AT:_LOGITS_AT + 4 * T * E].cpu().numpy().view(np.float32).reshape(T, E)
    ref = oracle.router_logits(inp.x, cfg.act_dtype, inp.router_w, inp.router_bias)
    assert got.view(np.uint32).tolist() == ref.view(np.uint32).tolist()
