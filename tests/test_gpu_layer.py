"""Layer parity of the HIP path (moe_exl3_layer through the C ABI) with the
fp64 oracle, max |out - ref| / max |ref| <= 2e-2 (fp16/bf16 arithmetic) or
<= 6e-2 with the routed GEMMs in fp8 (the activations are then rounded to
E4M3 with a per-row scale, which the oracle does not do).

With the synthetic side vectors (~1/64 on both sides) the routed experts add
about 1e-5 of what the shared expert adds, so a whole-output comparison would
not see routed errors: the routed part is checked on its own (layer without
the shared expert) and the full layer is checked as well.
"""
import numpy as np
import pytest
import torch

import oracle
import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer, dev, rel_err
from margins import record

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_FP8 = 6e-2


def _routed_only(inp):
    import dataclasses
    return dataclasses.replace(inp, shared=None)


@pytest.mark.parametrize("flags", [0, M.FORCE_GEMV, M.FORCE_MFMA])
def test_tiny_full(flags):
    inp = W.gen_layer(W.BY_NAME["tiny"])
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"tiny flags={flags} err={err:.3e}")
    record(f"tiny flags={flags}", err, TOL)
    assert err <= TOL


@pytest.mark.parametrize("T", [1, 37, 300])
@pytest.mark.parametrize("flags", [0, M.FORCE_MFMA])
def test_tiny_ragged(T, flags):
    inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=T))
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp)
    assert rel_err(out, ref) <= TOL


def test_tiny_one_expert_takes_every_token():
    # a huge bias on expert 3: all 600 slots of expert 3 -> three MFMA row tiles
    cfg = W.BY_NAME["tiny"].replace(tokens=600, router_bias=True)
    inp = W.gen_layer(cfg)
    inp.router_bias = np.zeros(cfg.n_experts, dtype=np.float32)
    inp.router_bias[3] = 100.0
    dl = DevLayer(inp)
    idx = dl.route()[0]
    assert (idx[:, 0] == 3).all()
    out = dl.run()
    _, _, ref = oracle.layer(inp)
    assert rel_err(out, ref) <= TOL


def test_decode_eight_rows_on_one_expert():
    # a huge bias on expert 3: all 8 tokens route to it.  Up to 8 tokens every
    # expert runs on the GEMV path (no expert can get more rows than there
    # are tokens), so expert 3 takes its 8 rows in four passes over its codes
    cfg = W.BY_NAME["decode"].replace(router_bias=True)
    inp = W.gen_layer(cfg)
    inp.router_bias = np.zeros(cfg.n_experts, dtype=np.float32)
    inp.router_bias[3] = 100.0
    routed = _routed_only(inp)
    dl = DevLayer(routed)
    idx = dl.route()[0]
    assert (idx[:, 0] == 3).all()
    out = dl.run()
    _, _, ref = oracle.layer(routed)
    err = rel_err(out, ref)
    print(f"decode eight rows on one expert err={err:.3e}")
    assert err <= TOL


def test_zero_tokens_is_noop():
    inp = W.gen_layer(W.BY_NAME["tiny"])
    dl = DevLayer(inp)
    x = dl.x[:0]
    out = torch.empty_like(x)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    M.layer(dl.desc, dl.weights, x, out, ws)
    torch.cuda.synchronize()


def test_decode_step():
    inp = W.gen_layer(W.BY_NAME["decode"])
    routed = _routed_only(inp)
    out_r = DevLayer(routed).run()
    _, _, ref_r = oracle.layer(routed)
    err_r = rel_err(out_r, ref_r)
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"decode routed err={err_r:.3e} full err={err:.3e}")
    record("decode routed", err_r, TOL)
    record("decode full", err, TOL)
    assert err_r <= TOL and err <= TOL


@pytest.mark.parametrize("K,codebook", [(3, W.CB_MCG), (4, W.CB_MCG), (4, W.CB_MCG_E4M3)])
def test_decode_step_code_widths(K, codebook):
    # the 8-token step at 3 and 4 bits per weight and with the E4M3 codebook:
    # every routed expert on the GEMV path or a small MFMA tile, the shared
    # expert's GEMV blocks inside the routed GEMV launches
    # (the full layer, dominated by the shared expert, on two tokens: the
    # oracle then decodes only the experts those two route to)
    inp = W.gen_layer(W.BY_NAME["decode"].replace(K=K, codebook=codebook))
    routed = _routed_only(inp)
    out_r = DevLayer(routed).run()
    _, _, ref_r = oracle.layer(routed)
    sample = [0, 7]
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp, sample)
    err_r, err = rel_err(out_r, ref_r), rel_err(out[sample], ref)
    print(f"decode K={K} cb={codebook} routed err={err_r:.3e} full err={err:.3e}")
    record(f"decode K={K} cb={codebook} routed", err_r, TOL)
    assert err_r <= TOL and err <= TOL
    assert np.isfinite(out).all() and np.isfinite(out_r).all()


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("name,K,codebook", [("decode", 2, W.CB_MCG), ("decode", 4, W.CB_MCG_E4M3),
                                             ("mixed_k34", None, None)])
def test_verify_batch_sizes(name, K, codebook, T):
    # 1-4 tokens at the real shapes (the verify batches of speculative
    # decoding): so few experts that the GEMV launches split each expert's
    # columns into narrower blocks and its input rows into ranges, to fill
    # the GPU; every token checked, routed-only and with the shared expert
    cfg = W.BY_NAME[name].replace(tokens=T)
    if K is not None:
        cfg = cfg.replace(K=K, codebook=codebook)
    inp = W.gen_layer(cfg)
    routed = _routed_only(inp)
    out_r = DevLayer(routed).run()
    _, _, ref_r = oracle.layer(routed)
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp)
    err_r, err = rel_err(out_r, ref_r), rel_err(out, ref)
    print(f"verify batch {name} T={T} K={cfg.K} cb={cfg.codebook} routed err={err_r:.3e} full err={err:.3e}")
    record(f"verify batch {name} T={T} K={cfg.K} cb={cfg.codebook} routed", err_r, TOL)
    assert err_r <= TOL and err <= TOL
    assert np.isfinite(out).all() and np.isfinite(out_r).all()


def routing_sample(dl, gemv_rows=2, n_min=64, seed=0):
    """Tokens chosen from the layer's own segment tables so that the sample
    reaches every kernel path: the first and last token; in the heaviest
    expert, rows 0, 255 and 256 (the end of a full 256-row tile and the start
    of the next) and its last row (the ragged last tile); for every MFMA tile
    size class (up to 32, 64, 128, 192 and 256 rows: the (NMB, CM) variants of
    the kernels) the last row of one expert's last tile in that class; one
    token on an expert at the GEMV threshold; then seeded random tokens up to
    n_min.  Returns (sorted token list, description)."""
    cfg = dl.inp.cfg
    T, k = dl.x.shape[0], cfg.top_k
    idx, _, counts, offsets, sorted_ids, _ = dl.route()
    tok = lambda p: int(sorted_ids[p]) // k
    pick, what = {0, T - 1}, []
    heavy = int(np.argmax(counts))
    o, c = int(offsets[heavy]), int(counts[heavy])
    for r in (0, 255, 256, c - 1):
        if 0 <= r < c:
            pick.add(tok(o + r))
    what.append(f"heaviest expert {heavy} ({c} rows)")
    classes = [(1, 32), (33, 64), (65, 128), (129, 192), (193, 256)]
    for lo, hi in classes:
        for e in np.argsort(-counts, kind="stable"):
            ce = int(counts[e])
            if ce <= gemv_rows:
                continue
            last = ce - 256 * ((ce - 1) // 256)   # rows in the expert's last tile
            if lo <= last <= hi:
                pick.add(tok(int(offsets[e]) + ce - 1))
                what.append(f"{lo}-{hi} rows: expert {int(e)}")
                break
    on_gemv = [int(e) for e in range(cfg.n_experts) if 0 < counts[e] <= gemv_rows]
    if on_gemv:
        e = max(on_gemv, key=lambda e: (int(counts[e]), -e))
        pick.add(tok(int(offsets[e])))
        what.append(f"GEMV expert {e} ({int(counts[e])} rows)")
    rng = np.random.default_rng(seed)
    while len(pick) < n_min:
        pick.add(int(rng.integers(0, T)))
    return sorted(pick), "; ".join(what)


def _sampled(name, flags=0, tol=TOL, n_min=64, n_full=8):
    """Routed-only parity on a routing-table sample of >= n_min tokens, and
    the full layer (shared expert included) on n_full of them."""
    cfg = W.BY_NAME[name]
    inp = W.gen_layer(cfg)
    routed = _routed_only(inp)
    dlr = DevLayer(routed, flags=flags)
    sample, what = routing_sample(dlr, n_min=n_min)
    out_r = dlr.run()
    _, _, ref_r = oracle.layer(routed, sample)
    err_r = rel_err(out_r[sample], ref_r)
    full = sample[:: max(1, len(sample) // n_full)][:n_full]
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp, full)
    err = rel_err(out[full], ref)
    print(f"{name} flags={flags} {len(sample)} tokens ({what}) routed err={err_r:.3e} full err={err:.3e}")
    record(f"{name} flags={flags} routed ({len(sample)} tokens)", err_r, tol)
    record(f"{name} flags={flags} full ({len(full)} tokens)", err, tol)
    assert err_r <= tol and err <= tol
    assert np.isfinite(out).all() and np.isfinite(out_r).all()


@pytest.mark.parametrize("T", [64, 65])
def test_decode_sized_layer_boundary(T):
    # 64 tokens: the single-block routing tail also writes the fp16 copy of the
    # bf16 activations; 65 tokens: the multi-launch routing and the separate copy
    cfg = W.BY_NAME["decode"].replace(tokens=T, router_bias=True)
    inp = W.gen_layer(cfg)
    sample = [0, T // 2, T - 1]
    routed = _routed_only(inp)
    out_r = DevLayer(routed).run()
    _, _, ref_r = oracle.layer(routed, sample)
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp, sample)
    err_r, err = rel_err(out_r[sample], ref_r), rel_err(out[sample], ref)
    print(f"decode-sized T={T} sampled routed err={err_r:.3e} full err={err:.3e}")
    assert err_r <= TOL and err <= TOL
    assert np.isfinite(out).all() and np.isfinite(out_r).all()


def test_prefill_sampled():
    _sampled("prefill")


@pytest.mark.parametrize("name", ["mixed_k3", "mixed_k4"])
def test_mixed_width_sampled(name):
    _sampled(name)


def test_tp2_rank_prefill_sampled():
    # the 7168-token layer at I = 1024, one tensor-parallel rank's share
    _sampled("prefill_tp2", n_min=32, n_full=2)


@pytest.mark.parametrize("name,n_min", [("tiles_full", 64), ("tiles_mid", 24), ("tiles_small", 24)])
def test_tile_class_routings_sampled(name, n_min):
    # the routings that isolate one row-tile class for measurement: every
    # tile full (4096 tokens on 8 experts), every tile 35-79 rows, every tile
    # 5-31 rows
    _sampled(name, n_min=n_min, n_full=1)


def test_e4m3_codebook_sampled():
    _sampled("fp8")


def test_e4m3_fp8_mfma_sampled():
    _sampled("fp8", flags=M.FP8_MFMA, tol=TOL_FP8)


def _tiny_e4m3(T):
    # the fp8 GEMMs need hidden and inter in whole 256-channel rounds
    return W.BY_NAME["tiny"].replace(tokens=T, inter=256, codebook=W.CB_MCG_E4M3)


@pytest.mark.parametrize("T", [1, 37, 300])
def test_tiny_fp8_mfma(T):
    inp = W.gen_layer(_tiny_e4m3(T))
    for part in (_routed_only(inp), inp):
        out = DevLayer(part, flags=M.FORCE_MFMA | M.FP8_MFMA).run()
        _, _, ref = oracle.layer(part)
        err = rel_err(out, ref)
        print(f"tiny fp8 T={T} shared={part.shared is not None} err={err:.3e}")
        assert err <= TOL_FP8 and np.isfinite(out).all()


@pytest.mark.parametrize("T", [37, 300])
def test_tiny_fp8_mfma_with_fp16_shared_expert(T):
    # above 16 tokens the dense fp16 shared expert's tiles run on the 16-bit
    # MFMA path inside the fp8 launches (300 tokens: two 256-row dense tiles,
    # the second ragged)
    inp = W.gen_layer(_tiny_e4m3(T).replace(shared=True))
    assert inp.shared is not None
    out = DevLayer(inp, flags=M.FORCE_MFMA | M.FP8_MFMA).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"tiny fp8 + fp16 shared T={T} err={err:.3e}")
    record(f"tiny fp8 + fp16 shared T={T}", err, TOL_FP8)
    assert err <= TOL_FP8 and np.isfinite(out).all()


def test_tiny_fp8_one_expert_takes_every_token():
    # 600 slots on expert 3: the fp8 GEMMs run three row tiles, the last one
    # ragged (88 rows), for the same expert
    cfg = _tiny_e4m3(600).replace(router_bias=True)
    inp = W.gen_layer(cfg)
    inp.router_bias = np.zeros(cfg.n_experts, dtype=np.float32)
    inp.router_bias[3] = 100.0
    routed = _routed_only(inp)
    out = DevLayer(routed, flags=M.FP8_MFMA).run()
    _, _, ref = oracle.layer(routed)
    err = rel_err(out, ref)
    print(f"tiny fp8 one expert err={err:.3e}")
    assert err <= TOL_FP8


@pytest.mark.parametrize("T,flags", [(1, 0), (3, 0), (8, 0), (9, 0), (16, 0), (3, M.FORCE_MFMA)])
def test_shared_expert_gemv_token_counts(T, flags):
    # up to 16 tokens the shared expert runs on its GEMV code, which works on
    # a power-of-two token count (3 -> 4 with one padding token); up to 8 its
    # blocks run inside the routed GEMV launches (T = 8 the last such count,
    # T = 9 the first in launches of its own), unless no expert is on the GEMV
    # path (forced MFMA).  The full output is dominated by the shared expert.
    inp = W.gen_layer(W.BY_NAME["decode"].replace(tokens=T))
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"shared gemv T={T} flags={flags} err={err:.3e}")
    assert err <= TOL and np.isfinite(out).all()


def test_shared_expert_ragged_row_tile():
    # 300 tokens at the real shapes: the shared expert runs on the MFMA path
    # (more than 16 tokens) with a last row tile of 44 rows, so one of its two
    # row halves is empty; the full output is dominated by the shared expert
    cfg = W.BY_NAME["decode"].replace(tokens=300)
    inp = W.gen_layer(cfg)
    sample = [0, 127, 128, 255, 256, 299]
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp, sample)
    err = rel_err(out[sample], ref)
    print(f"shared ragged err={err:.3e}")
    assert err <= TOL
    assert np.isfinite(out).all()


# The largest hidden and intermediate sizes the descriptor accepts (16384),
# each with a small other dimension so the oracle stays quick.  Past hidden
# 8192 the routed experts all run on MFMA tiles (the gate/up GEMV keeps two
# projections' activation rows in LDS up to that size), so the forced-GEMV
# case checks that fallback; at inter 16384 the down GEMV holds 64 KiB of h
# rows in LDS.  The shared expert takes its GEMV at T = 5.  The activations are bf16: the
# generator's side vectors scale as 1/sqrt(H), which at H = 16384 leaves the
# layer output near 2e-7, inside fp16's subnormal range (spacing 2^-24), where
# an fp16 output would keep only two or three significant bits.
_MAX_SHAPES = [(16384, 128), (256, 16384)]


@pytest.mark.parametrize("T,flags", [(5, 0), (300, 0), (300, M.FORCE_GEMV)])
@pytest.mark.parametrize("H,I", _MAX_SHAPES)
def test_largest_hidden_and_inter_routed(H, I, T, flags):
    cfg = W.BY_NAME["tiny"].replace(hidden=H, inter=I, tokens=T, act_dtype=W.DT_BF16)
    inp = W.gen_layer(cfg)
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"H={H} I={I} T={T} flags={flags} err={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("T", [5, 300])
@pytest.mark.parametrize("H,I", _MAX_SHAPES)
def test_largest_hidden_and_inter_shared(H, I, T):
    # T = 5: shared-expert GEMV; T = 300: its tiles inside the routed launches
    cfg = W.BY_NAME["tiny"].replace(hidden=H, inter=I, tokens=T, shared=True, act_dtype=W.DT_BF16)
    inp = W.gen_layer(cfg)
    out = DevLayer(inp).run()
    _, _, ref = oracle.layer(inp)
    err = rel_err(out, ref)
    print(f"H={H} I={I} T={T} shared err={err:.3e}")
    assert err <= TOL
