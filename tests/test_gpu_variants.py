"""Layer parity of the format variants through the C ABI, against the oracle:
the rotated basis with sign vectors (HADAMARD), the trellis-coded shared
expert (SHARED_TRELLIS) and per-tensor widths (PER_TENSOR_K), on their own
and together (the exlr8 v2 layout at real shapes), on every kernel path."""
import dataclasses

import numpy as np
import pytest

import oracle
import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer, rel_err
from margins import record
from test_gpu_layer import routing_sample

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_FP8 = 6e-2
PATHS = [0, M.FORCE_GEMV, M.FORCE_MFMA]


def _check(name, inp, flags=0, tokens=None, tol=TOL):
    out = DevLayer(inp, flags=flags).run()
    _, _, ref = oracle.layer(inp, tokens)
    got = out if tokens is None else out[tokens]
    err = rel_err(got, ref)
    print(f"{name} flags={flags} err={err:.3e}")
    record(f"{name} flags={flags}", err, tol)
    assert err <= tol and np.isfinite(out).all()
    return out


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("T", [1, 37, 300])
def test_tiny_rotated(T, flags):
    inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=T, hadamard=True))
    _check(f"tiny rotated T={T}", inp, flags)


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("T", [1, 37, 300])
@pytest.mark.parametrize("hadamard", [False, True])
def test_tiny_trellis_shared_expert(T, flags, hadamard):
    cfg = W.BY_NAME["tiny"].replace(tokens=T, K=4, shared_trellis=True, hadamard=hadamard)
    _check(f"tiny shared-trellis rot={hadamard} T={T}", W.gen_layer(cfg), flags)


def test_rotated_bf16_with_fp16_shared_expert():
    # the dense fp16 shared expert reads x while the trellis experts read R(s0 x)
    cfg = W.BY_NAME["decode"].replace(tokens=5, hadamard=True)
    inp = W.gen_layer(cfg)
    _check("decode-shape rotated + fp16 shared T=5", inp)
    _check("decode-shape rotated routed T=5", dataclasses.replace(inp, shared=None))


def test_exlr8_decode_step():
    # 8 tokens at real shapes: K4 E4M3 codebook, rotated, trellis shared
    # expert (expert 288, on the GEMV path with every routed expert)
    inp = W.gen_layer(W.BY_NAME["exlr8_decode"])
    _check("exlr8 decode-8", inp)


@pytest.mark.parametrize("flags,tol", [(0, TOL), (M.FP8_MFMA, TOL_FP8)])
def test_exlr8_prefill_sampled(flags, tol):
    # 2048 tokens: the trellis shared expert takes 2048 rows (eight full MFMA
    # row tiles) next to the routed experts; sampled from the routing table
    inp = W.gen_layer(W.BY_NAME["exlr8_prefill"])
    dl = DevLayer(inp, flags=flags)
    sample, what = routing_sample(dl)
    out = dl.run()
    _, _, ref = oracle.layer(inp, sample)
    err = rel_err(out[sample], ref)
    print(f"exlr8 prefill flags={flags} {len(sample)} tokens ({what}) err={err:.3e}")
    record(f"exlr8 prefill-2048 flags={flags} ({len(sample)} tokens)", err, tol)
    assert err <= tol and np.isfinite(out).all()


# ------------------------------------------------------- per-tensor widths
@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("T", [1, 37, 300])
def test_tiny_per_tensor_widths(T, flags):
    # every (projection, expert) tensor K3 or K4, on its own allocation
    inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=T, mixed_k=True))
    assert set(np.unique(inp.ktab)) == {3, 4}
    _check(f"tiny per-tensor K T={T}", inp, flags)


def test_tiny_per_tensor_widths_with_rotation_and_trellis_shared():
    cfg = W.BY_NAME["tiny"].replace(tokens=300, mixed_k=True, hadamard=True, shared_trellis=True)
    _check("tiny per-tensor K + rotation + trellis shared T=300", W.gen_layer(cfg))


def test_mixed_k34_prefill_sampled():
    # the 2048-token prefill with every tensor independently K3 or K4
    inp = W.gen_layer(W.BY_NAME["mixed_k34"])
    routed = dataclasses.replace(inp, shared=None)
    dl = DevLayer(routed)
    sample, what = routing_sample(dl)
    out = dl.run()
    _, _, ref = oracle.layer(routed, sample)
    err = rel_err(out[sample], ref)
    print(f"mixed_k34 {len(sample)} tokens ({what}) routed err={err:.3e}")
    record(f"mixed_k34 prefill-2048 routed ({len(sample)} tokens)", err, TOL)
    assert err <= TOL and np.isfinite(out).all()


def test_bad_width_is_flagged_and_reads_nothing():
    import torch
    inp = W.gen_layer(W.BY_NAME["tiny"].replace(tokens=40, mixed_k=True))
    dl = DevLayer(inp)
    kt = dl.k_tab.clone()
    kt[1, 3] = 7
    w = M.make_weights(dl.codes, dl.suh, dl.svh, dl.router_w, dl.bias, dl.shared, dl.signs, dl.code_tab, kt)
    out = torch.empty_like(dl.x)
    ws = dl.workspace(40)
    M.layer(dl.desc, w, dl.x, out, ws)
    assert M.status(ws) & M.STATUS_BAD_WIDTH
    M.layer(dl.desc, dl.weights, dl.x, out, ws)
    assert M.status(ws) == 0


# ------------------------------------------------------------ load layout
@pytest.mark.parametrize("order,n_in,n_out", [(M.ORDER_ROWMAJOR, 48, 64), (M.ORDER_COLMAJOR, 48, 64),
                                              (M.ORDER_COLMAJOR, 4096, 2048),
                                              (M.ORDER_COLGROUPS128, 4096, 2048),
                                              (M.ORDER_COLGROUPS128, 32, 384)])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_repack_then_decode_bit_exact(order, n_in, n_out, K):
    # the stored layout decoded by the oracle's order definition equals the
    # kernels' decode of the repacked tensor, bit for bit; three tensors in one
    # call (a stacked expert dimension)
    import torch
    from gpu_util import dev
    count = 3
    rng = np.random.default_rng(order * 10 + K)
    words = (n_in // 16) * (n_out // 16) * 16 * K
    src = rng.integers(0, 1 << 16, count * words, dtype=np.uint16)
    dsrc = dev(src)
    dst = torch.full_like(dsrc, -1)
    M.repack(dsrc, dst, count, n_in, n_out, K, order)
    for i in [0, count - 1]:
        ref = oracle.decode_matrix_order(src[i * words:(i + 1) * words], n_in, n_out, K, W.MCG_DEFAULT, 0, order)
        got = torch.empty((n_in, n_out), dtype=torch.float32, device="cuda")
        M.decode(dst[i * words:(i + 1) * words], n_in, n_out, K, W.MCG_DEFAULT, 0, got, M.DT_F32)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_expand_block_scales_bit_exact():
    import torch
    from gpu_util import dev
    EA, H, I = 289, 4096, 2048
    rng = np.random.default_rng(9)
    block = rng.uniform(0.5, 1.5, (EA, 3, H // 128)).astype(np.float16)
    suh, svh = oracle.expand_block_scales(block, H, I)
    dsuh = [torch.full((EA, n), -1, dtype=torch.int16, device="cuda") for n in (H, H, I)]
    dsvh = [torch.full((EA, n), -1, dtype=torch.int16, device="cuda") for n in (I, I, H)]
    M.expand_block_scales(dev(block), EA, H, I, dsuh, dsvh)
    torch.cuda.synchronize()
    for p in range(3):
        np.testing.assert_array_equal(dsuh[p].cpu().numpy().view(np.uint16), suh[p].view(np.uint16))
        np.testing.assert_array_equal(dsvh[p].cpu().numpy().view(np.uint16), svh[p].view(np.uint16))


def test_exlr8_layout_loaded_end_to_end():
    # an exlr8-v2-style layer stored as on the pages' layout (gate/up in
    # 128-column halves, block scales) goes through the load-time entries and
    # then the layer; the oracle reads the same stored bytes by its own
    # definitions of the order and of the block table
    import torch
    from gpu_util import dev
    cfg = W.BY_NAME["tiny"].replace(tokens=37, K=4, inter=256, codebook=W.CB_MCG_E4M3, hadamard=True,
                                    shared_trellis=True)
    inp = W.gen_layer(cfg)
    EA, H, I, K = cfg.n_trellis, cfg.hidden, cfg.inter, cfg.K
    rng = np.random.default_rng(17)
    block = (rng.uniform(0.5, 1.5, (EA, 3, H // 128)) / 16).astype(np.float16)
    suh, svh = oracle.expand_block_scales(block, H, I)
    stored = []
    for p in range(3):
        n_in, n_out = cfg.proj_shape(p)
        stored.append(np.ascontiguousarray(inp.codes[p]))   # read as COLGROUPS128 (gate/up) / ROWMAJOR (down)
    ref_codes = []
    for p in range(3):
        n_in, n_out = cfg.proj_shape(p)
        order = M.ORDER_COLGROUPS128 if p < 2 else M.ORDER_ROWMAJOR
        # the oracle's own reorder: position of tile (tk, tn) in the stored order
        ntk, ntn = n_in // 16, n_out // 16
        perm = np.array([oracle.tile_position(order, n_in, n_out, tk, tn)
                         for tk in range(ntk) for tn in range(ntn)])
        tiles = stored[p].reshape(EA, ntk * ntn, 16 * K)
        ref_codes.append(np.ascontiguousarray(tiles[:, perm, :].reshape(EA, -1)))
    ref_inp = dataclasses.replace(inp, codes=ref_codes, suh=suh, svh=svh)
    dl = DevLayer(ref_inp)
    # replace the device codes and side vectors by the load-time entries' output
    for p in range(3):
        n_in, n_out = cfg.proj_shape(p)
        order = M.ORDER_COLGROUPS128 if p < 2 else M.ORDER_ROWMAJOR
        M.repack(dev(stored[p]), dl.codes[p], EA, n_in, n_out, K, order)
        dl.suh[p].fill_(-1)
        dl.svh[p].fill_(-1)
    M.expand_block_scales(dev(block), EA, H, I, dl.suh, dl.svh)
    torch.cuda.synchronize()
    out = dl.run()
    _, _, ref = oracle.layer(ref_inp)
    err = rel_err(out, ref)
    record("exlr8 layout loaded end to end T=37", err, TOL)
    assert err <= TOL and np.isfinite(out).all()
