"""Pins of the oracle's format variants: the Hadamard rotation with sign
vectors, per-tensor widths, the trellis-coded shared expert, the stored tile
orders, NaN ranking in top-k and the bf16 conversion.  Each is checked against
a library routine (scipy's Hadamard matrix, torch's bfloat16, numpy matmul and
stable argsort), a hand-derived table or an invariant, never against itself."""
import dataclasses

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import workloads as W


def _silu(z):
    return z / (1.0 + np.exp(-z))


# ------------------------------------------------------------------ bf16
def test_bf16_conversion_matches_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    lib = oracle.lib()
    got = np.array([lib.orc_bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------- NaN ranking
def test_topk_ranks_nan_as_minus_infinity():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((40, 24)).astype(np.float32)
    lg[rng.random(lg.shape) < 0.3] = np.nan
    lg[3, :] = np.nan                    # a token with no number at all
    lg[5, 2] = -np.inf                   # -inf ties with NaN, lower index first
    lg[5, 1] = np.nan
    k = 6
    idx, w = oracle.topk_softmax(lg, k)
    key = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    ref = np.argsort(-key, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref)
    assert ((idx >= 0) & (idx < lg.shape[1])).all()
    np.testing.assert_array_equal(idx[3], np.arange(k))
    assert np.isnan(w[3]).all()          # softmax of k values of -inf
    # a NaN chosen after a finite logit weighs nothing
    fin = np.isfinite(np.take_along_axis(key, idx, axis=1))
    rows = fin[:, 0]
    assert (w[rows][~fin[rows]] == 0).all()
    np.testing.assert_allclose(w[rows].sum(axis=1), 1.0, rtol=0, atol=1e-12)


# -------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy_and_is_orthogonal(n):
    h = oracle.sylvester(n).astype(np.int64)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(n))
    np.testing.assert_array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


def test_rotation_is_blockwise_scaled_hadamard_and_an_involution():
    rng = np.random.default_rng(3)
    H = 512
    v = rng.standard_normal((5, H))
    s = (rng.integers(0, 2, H) * 2 - 1).astype(np.int8)
    R = np.kron(np.eye(H // 128), scipy.linalg.hadamard(128)) / np.sqrt(128.0)
    np.testing.assert_allclose(oracle.rotate(v), v @ R.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.rotate(v, s), (v * s) @ R.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.rotate(oracle.rotate(v)), v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(oracle.rotate(v), axis=1), np.linalg.norm(v, axis=1),
                               rtol=1e-13)
    # a unit vector maps to a signed column of H_128 in its own block only
    e = np.zeros(H)
    e[130] = 1.0
    r = oracle.rotate(e)
    assert (r[:128] == 0).all() and (r[256:] == 0).all()
    np.testing.assert_allclose(r[128:256] * np.sqrt(128.0), scipy.linalg.hadamard(128)[:, 2], atol=1e-13)


def _dense_mats(inp, e, ktab=None):
    """suh[k] c[k][n] svh[n] of expert e's three projections (fp64)."""
    cfg = inp.cfg
    mats = []
    for p in range(3):
        a, b = cfg.proj_shape(p)
        K = cfg.K if ktab is None else int(ktab[p][e])
        c = oracle.decode_matrix(inp.codes[p][e], a, b, K, cfg.mcg, cfg.codebook).astype(np.float64)
        mats.append(inp.suh[p][e].astype(np.float64)[:, None] * c * inp.svh[p][e].astype(np.float64)[None, :])
    return mats


def _mlp(x, mats):
    return (_silu(x @ mats[0]) * (x @ mats[1])) @ mats[2]


def test_rotated_single_expert_equals_rotated_dense_mlp():
    # one expert, top-1: the layer is s1 * R(mlp(R(s0 * x))), R from scipy
    cfg = W.BY_NAME["tiny"].replace(n_experts=1, top_k=1, K=4, hadamard=True)
    inp = W.gen_layer(cfg, tokens=9)
    assert set(np.unique(inp.signs)) == {-1, 1}
    _, w, out = oracle.layer(inp)
    assert (w == 1.0).all()
    H = cfg.hidden
    R = np.kron(np.eye(H // 128), scipy.linalg.hadamard(128)) / np.sqrt(128.0)
    x = W.act_bits_to_f32(inp.x, cfg.act_dtype).astype(np.float64)
    s0, s1 = inp.signs.astype(np.float64)
    ref = ((_mlp((x * s0) @ R.T, _dense_mats(inp, 0))) @ R.T) * s1
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_rotation_leaves_router_and_fp16_shared_expert_on_x():
    cfg = W.BY_NAME["tiny"].replace(hadamard=True, shared=True, tokens=7)
    inp = W.gen_layer(cfg)
    plain = dataclasses.replace(inp, signs=None)
    idx_r, w_r, out_r = oracle.layer(inp)
    idx_p, w_p, _ = oracle.layer(plain)
    np.testing.assert_array_equal(idx_r, idx_p)
    np.testing.assert_array_equal(w_r, w_p)
    # the fp16 shared expert adds shared(x) to the rotated expert sum
    _, _, routed = oracle.layer(dataclasses.replace(inp, shared=None))
    x = W.act_bits_to_f32(inp.x, cfg.act_dtype).astype(np.float64)
    g, u, d = (a.astype(np.float64) for a in inp.shared)
    shared = (_silu(x @ g.T) * (x @ u.T)) @ d.T
    np.testing.assert_allclose(out_r - routed, shared, rtol=1e-9, atol=1e-12 * np.abs(shared).max())


# ------------------------------------------------------- per-tensor widths
def test_per_tensor_widths_single_expert_dense_mlp():
    cfg = W.BY_NAME["tiny"].replace(n_experts=1, top_k=1, mixed_k=True)
    inp = W.gen_layer(cfg, tokens=6)
    inp.ktab = np.array([[3], [4], [2]], dtype=np.int32)   # gate K3, up K4, down K2
    inp.codes = [[W.gen_codes_expert(cfg, p, 0, int(inp.ktab[p][0]))] for p in range(3)]
    assert [c[0].size for c in inp.codes] == [cfg.words_per_expert(p, int(inp.ktab[p][0])) for p in range(3)]
    _, _, out = oracle.layer(inp)
    x = W.act_bits_to_f32(inp.x, cfg.act_dtype).astype(np.float64)
    ref = _mlp(x, _dense_mats(inp, 0, inp.ktab))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_per_tensor_widths_equal_uniform_width_when_all_equal():
    cfg = W.BY_NAME["tiny"].replace(K=3)
    inp = W.gen_layer(cfg)
    _, _, ref = oracle.layer(inp)
    tab = dataclasses.replace(inp, ktab=np.full((3, cfg.n_experts), 3, dtype=np.int32))
    _, _, out = oracle.layer(tab)
    np.testing.assert_array_equal(out, ref)


def test_per_tensor_width_table_is_used_and_validated():
    cfg = W.BY_NAME["tiny"].replace(mixed_k=True)
    inp = W.gen_layer(cfg)
    assert set(np.unique(inp.ktab)) == {3, 4}
    bad = dataclasses.replace(inp, ktab=np.where(inp.ktab == 3, 5, inp.ktab).astype(np.int32))
    with pytest.raises((RuntimeError, AssertionError)):
        oracle.layer(bad)


# ------------------------------------------------- trellis shared expert
@pytest.mark.parametrize("hadamard", [False, True])
def test_trellis_shared_expert_adds_its_mlp_with_weight_one(hadamard):
    cfg = W.BY_NAME["tiny"].replace(shared_trellis=True, hadamard=hadamard, K=4, tokens=11)
    inp = W.gen_layer(cfg)
    E = cfg.n_experts
    idx, _, out = oracle.layer(inp)
    assert ((idx >= 0) & (idx < E)).all()   # the shared expert is never routed
    # the same layer without the shared expert: drop expert E from every tensor
    rcfg = cfg.replace(shared_trellis=False)
    routed_inp = dataclasses.replace(
        inp, cfg=rcfg, codes=[c[:E] for c in inp.codes], suh=[a[:E] for a in inp.suh],
        svh=[a[:E] for a in inp.svh])
    _, _, routed = oracle.layer(routed_inp)
    x = W.act_bits_to_f32(inp.x, cfg.act_dtype).astype(np.float64)
    mats = _dense_mats(inp, E)
    if hadamard:
        H = cfg.hidden
        R = np.kron(np.eye(H // 128), scipy.linalg.hadamard(128)) / np.sqrt(128.0)
        s0, s1 = inp.signs.astype(np.float64)
        ref = (_mlp((x * s0) @ R.T, mats) @ R.T) * s1
    else:
        ref = _mlp(x, mats)
    np.testing.assert_allclose(out - routed, ref, rtol=1e-8, atol=1e-11 * np.abs(ref).max())


# ------------------------------------------------------------ tile orders
def test_tile_positions_hand_derived():
    # a 32 x 48 projection: 2 x 3 tiles
    rowmajor = {(0, 0): 0, (0, 1): 1, (0, 2): 2, (1, 0): 3, (1, 1): 4, (1, 2): 5}
    colmajor = {(0, 0): 0, (1, 0): 1, (0, 1): 2, (1, 1): 3, (0, 2): 4, (1, 2): 5}
    for (tk, tn), p in rowmajor.items():
        assert oracle.tile_position(0, 32, 48, tk, tn) == p
    for (tk, tn), p in colmajor.items():
        assert oracle.tile_position(1, 32, 48, tk, tn) == p
    # a 32 x 256 projection in groups of 128 columns (8 tiles): group 0 holds
    # tiles (0, 0..7) then (1, 0..7); group 1 starts at 16 with (0, 8..15)
    groups = {(0, 0): 0, (0, 7): 7, (1, 0): 8, (1, 7): 15, (0, 8): 16, (0, 15): 23,
              (1, 8): 24, (1, 9): 25, (1, 15): 31}
    for (tk, tn), p in groups.items():
        assert oracle.tile_position(2, 32, 256, tk, tn) == p
    assert oracle.tile_position(7, 32, 48, 0, 0) == -1


@pytest.mark.parametrize("order,n_in,n_out", [(0, 48, 64), (1, 48, 64), (1, 64, 32), (2, 32, 256),
                                              (2, 64, 384)])
def test_tile_positions_are_a_permutation(order, n_in, n_out):
    pos = [oracle.tile_position(order, n_in, n_out, tk, tn)
           for tk in range(n_in // 16) for tn in range(n_out // 16)]
    assert sorted(pos) == list(range(len(pos)))


@pytest.mark.parametrize("order", [1, 2])
def test_decode_by_order_reads_each_tile_from_its_position(order):
    # every stored tile is a distinct random tile; decoding the stored layout
    # must give, at grid cell (tk, tn), the tile stored at its position
    n_in, n_out, K, mcg = 48, 256, 3, W.MCG_DEFAULT
    ntk, ntn = n_in // 16, n_out // 16
    rng = np.random.default_rng(order)
    stored = rng.integers(0, 1 << 16, (ntk * ntn, 16 * K), dtype=np.uint16)
    got = oracle.decode_matrix_order(stored.ravel(), n_in, n_out, K, mcg, 0, order)
    for tk in range(ntk):
        for tn in range(ntn):
            p = oracle.tile_position(order, n_in, n_out, tk, tn)
            tile = oracle.decode_tile(stored[p], K, mcg)
            block = got[16 * tk:16 * tk + 16, 16 * tn:16 * tn + 16]
            # state j sits at row j % 16, column j / 16 of its tile
            np.testing.assert_array_equal(block, tile.reshape(16, 16).T)
    # order 0 is the layout decode_matrix reads
    flat = stored.ravel()
    np.testing.assert_array_equal(oracle.decode_matrix_order(flat, n_in, n_out, K, mcg, 0, 0),
                                  oracle.decode_matrix(flat, n_in, n_out, K, mcg))


def test_exlr8_half_sizes():
    # a 4096 x 128 gate/up half at width K is 65,536 K bytes (exlr8 "Loading")
    for K in (2, 3, 4):
        assert (4096 // 16) * (128 // 16) * 16 * K * 2 == 65536 * K


# ---------------------------------------------------------- block scales
def test_block_scale_expansion_matches_numpy_repeat():
    rng = np.random.default_rng(5)
    EA, H, I = 3, 512, 256
    block = rng.uniform(0.5, 1.5, (EA, 3, H // 128)).astype(np.float16)
    suh, svh = oracle.expand_block_scales(block, H, I)
    np.testing.assert_array_equal(suh[0], np.repeat(block[:, 0, :], 128, axis=1))
    np.testing.assert_array_equal(suh[1], np.repeat(block[:, 1, :], 128, axis=1))
    np.testing.assert_array_equal(svh[2], np.repeat(block[:, 2, :], 128, axis=1))
    for a in (svh[0], svh[1], suh[2]):
        assert a.shape == (EA, I) and (a == np.float16(1.0)).all()
