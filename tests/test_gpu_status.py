"""The status word and the routing of non-finite logits, through the C ABI.

The NaN cases run the fixed top-k code (a NaN logit ranks as -inf); the host
model in test_topk_lane_model.py shows on the CPU that this selection always
yields a valid expert."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer, dev, poisoned_workspace, rel_err

pytestmark = pytest.mark.gpu


def _route_and_status(dl, x):
    T = x.shape[0]
    cfg = dl.inp.cfg
    n = T * cfg.top_k
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    w = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = poisoned_workspace(dl.desc, T)
    M.route(dl.desc, dl.weights, x, idx, w, None, None, None, None, ws)
    return idx.cpu().numpy().reshape(T, -1), w.cpu().numpy().reshape(T, -1), M.status(ws)


@pytest.mark.parametrize("T", [8, 300])
def test_nan_router_row_ranks_last(T):
    # expert 5's router row holds a NaN: its logit is NaN for every token and
    # it is never chosen; the few-token (T = 8) and many-token paths agree
    # with the oracle bit for bit
    cfg = W.BY_NAME["decode"].replace(tokens=T)
    inp = W.gen_layer(cfg, experts=[])
    inp.router_w = inp.router_w.copy()
    inp.router_w[5, 17] = np.float16(np.nan)
    dl = DevLayer(inp)
    idx, w, st = _route_and_status(dl, dl.x)
    ref_idx, ref_w = oracle.route_tokens(inp, list(range(T)))
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(w, ref_w, rtol=2e-6)
    assert not (idx == 5).any()
    assert st == 0


@pytest.mark.parametrize("T", [8, 300])
def test_nan_activation_row_gets_valid_experts(T):
    # token 3 holds a NaN: every logit of it is NaN, its experts are 0..k-1
    # (the -inf tie goes to the lower index) and its weights NaN; the other
    # tokens route as usual.  Every index stays inside [0, E).
    cfg = W.BY_NAME["decode"].replace(tokens=T)
    inp = W.gen_layer(cfg, experts=[])
    x = inp.x.copy()
    x[3, 100] = 0x7FC0   # bf16 NaN
    inp = dataclasses.replace(inp, x=x)
    dl = DevLayer(inp)
    idx, w, st = _route_and_status(dl, dl.x)
    assert ((idx >= 0) & (idx < cfg.n_experts)).all()
    ref_idx, ref_w = oracle.route_tokens(inp, list(range(T)))
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_array_equal(idx[3], np.arange(cfg.top_k))
    assert np.isnan(w[3]).all()
    ok = np.arange(T) != 3
    np.testing.assert_allclose(w[ok], ref_w[ok], rtol=2e-6)
    assert st == 0


def test_status_clear_after_normal_layer_with_debug_checks():
    # DEBUG_CHECKS adds the table and finiteness checks; a normal layer leaves
    # the (poisoned) status word cleared, at both routing paths
    for T in (8, 300):
        inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=T))
        dl = DevLayer(inp, flags=M.DEBUG_CHECKS)
        out = torch.empty_like(dl.x)
        ws = dl.workspace(T)
        M.layer(dl.desc, dl.weights, dl.x, out, ws)
        assert M.status(ws) == 0, T


@pytest.mark.parametrize("T", [8, 300])
def test_bf16_beyond_fp16_range_is_flagged(T):
    cfg = W.BY_NAME["decode"].replace(tokens=T, K=2)
    inp = W.gen_layer(cfg)
    routed = dataclasses.replace(inp, shared=None)
    dl = DevLayer(routed)
    x = dl.x.clone()
    out = torch.empty_like(x)
    ws = dl.workspace(T)
    M.layer(dl.desc, dl.weights, x, out, ws)
    assert M.status(ws) == 0
    x[2, 7] = int(W.f32_to_bf16_bits(np.array([1.0e5], dtype=np.float32))[0].astype(np.int16))
    M.layer(dl.desc, dl.weights, x, out, ws)
    assert M.status(ws) & M.STATUS_ACT_RANGE


def test_debug_checks_flag_nonfinite_x():
    inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=40))
    dl = DevLayer(inp, flags=M.DEBUG_CHECKS)
    x = dl.x.clone()
    x[5, 9] = 0x7C00     # fp16 inf
    out = torch.empty_like(x)
    ws = dl.workspace(40)
    M.layer(dl.desc, dl.weights, x, out, ws)
    st = M.status(ws)
    assert st & M.STATUS_NONFINITE_X
    assert not st & (M.STATUS_TABLES | M.STATUS_COUNTS | M.STATUS_BAD_INDEX)


def test_debug_checks_leave_outputs_unchanged():
    inp = W.gen_layer(W.BY_NAME["tiny"])
    a = DevLayer(inp).run()
    b = DevLayer(inp, flags=M.DEBUG_CHECKS).run()
    np.testing.assert_array_equal(a, b)
    _, _, ref = oracle.layer(inp)
    assert rel_err(b, ref) <= 2e-2
