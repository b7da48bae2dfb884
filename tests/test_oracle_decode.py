"""Pins of the oracle's trellis decode against facts fixed outside the oracle.

The pages define the storage (packed 16-bit words, 16/K weights per word, a
`mcg` codebook multiplier, 16x16 tiles) but not the bit-level decode; the
reading used here is stated in oracle/oracle.c.  These tests pin that reading
with hand-derived values, closed forms of special multipliers, an inverse
(re-encode) map, brute-force search and a library FP8 conversion.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MCG = 0x9E3779B1


def _words_p1(K):
    return np.array([(0x1234 * i + 0xBEEF) & 0xFFFF for i in range(16 * K)], dtype=np.uint16)


def test_value_map_hand_examples():
    # h = 0 -> every field 0 -> v = -254
    assert oracle.mcg_value(0, MCG) == -254
    # s = 1: h = 0x9E3779B1, bytes B1 79 37 9E, fields (byte >> 1) 88 60 27 79, sum 254
    assert oracle.mcg_value(1, MCG) == 0
    # s = 2: h = 0x3C6EF362, bytes 62 F3 6E 3C -> 49 121 55 30, sum 255
    assert oracle.mcg_value(2, MCG) == 1
    # s = 3: h = 0xDAA66D13, bytes 13 6D A6 DA -> 9 54 83 109, sum 255
    assert oracle.mcg_value(3, MCG) == 1
    # s = 0xFFFF: h = 0x79B10000 - 0x9E3779B1 mod 2^32 = 0xDB79864F -> 39 67 60 109
    assert oracle.mcg_value(0xFFFF, MCG) == 21
    # s = 8: h = 0xF1BBCD88, bytes 88 CD BB F1 -> 68 102 93 120, sum 383
    assert oracle.mcg_value(8, MCG) == 129


def test_value_map_closed_forms():
    s = np.arange(65536)
    # mcg = 1: h = s, upper two fields are zero
    v1 = oracle.value_table(1)
    np.testing.assert_array_equal(v1, ((s >> 1) & 127) + ((s >> 9) & 127) - 254)
    assert len(np.unique(v1)) == 255 and v1.min() == -254 and v1.max() == 0
    # mcg = 0: every state maps to the minimum
    assert (oracle.value_table(0) == -254).all()
    # mcg = 2: h = 2s, fields are bits 0..6 and 8..14 of s
    np.testing.assert_array_equal(oracle.value_table(2), (s & 127) + ((s >> 8) & 127) - 254)
    # mcg = 2^16: h = s << 16, fields move to the top two bytes -> same as mcg = 1
    np.testing.assert_array_equal(oracle.value_table(1 << 16), v1)
    # mcg = 2^32 - 1: h = -s mod 2^32; s = 1 gives all-ones -> four fields of 127
    assert oracle.mcg_value(1, 0xFFFFFFFF) == 254


def test_value_map_enumeration():
    with open(os.path.join(GOLDEN, "value_map_enumeration.txt")) as f:
        line = [l for l in f if l.strip() and not l.startswith("#")][0]
    s1, s2, lo, hi, nd = map(int, line.split())
    v = oracle.value_table(MCG).astype(np.int64)
    assert v.sum() == s1 and (v * v).sum() == s2
    assert v.min() == lo and v.max() == hi and len(np.unique(v)) == nd
    # uniform random words decode to states that are uniform on 16 bits, so the
    # decoded histogram converges to the table's
    rng = np.random.default_rng(5)
    words = rng.integers(0, 1 << 16, 16 * 2 * 4096, dtype=np.uint16)
    st = oracle.stream_states(words, 2)
    dec = v[st]
    assert abs(dec.mean() - v.mean()) < 0.05 * v.std()


def test_worked_example():
    with open(os.path.join(GOLDEN, "decode_worked_example.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for row in rows:
        parts = [p.split() for p in row.split("|")]
        K = int(parts[0][0])
        s_head = [int(t, 16) for t in parts[1]]
        v_head = [int(t) for t in parts[2]]
        v_tail = [int(t) for t in parts[3]]
        s_last = int(parts[4][0], 16)
        st = oracle.stream_states(_words_p1(K), K)
        assert st.size == 256
        assert list(st[:4]) == s_head
        assert st[255] == s_last
        vals = oracle.decode_tile(_words_p1(K), K, MCG)
        np.testing.assert_array_equal(vals[:8] * 64, v_head)
        np.testing.assert_array_equal(vals[254:] * 64, v_tail)
        assert [oracle.mcg_value(int(s), MCG) for s in st[:8]] == v_head


@pytest.mark.parametrize("K", [2, 3, 4])
def test_trellis_consistency_and_reencode(K):
    rng = np.random.default_rng(K)
    words = rng.integers(0, 1 << 16, 16 * K, dtype=np.uint16)
    st = oracle.stream_states(words, K).astype(np.int64)
    # the first state is word 0 (the first 16 stream bits)
    assert st[0] == words[0]
    # each state shifts in K fresh bits: s_{j+1} >> K == s_j & (2^(16-K) - 1), cyclically
    nxt = np.roll(st, -1)
    np.testing.assert_array_equal(nxt >> K, st & ((1 << (16 - K)) - 1))
    # inverse map: write every state's K fresh (low) bits at stream bits
    # jK+16-K .. jK+15 (mod B), most significant first, and rebuild the words
    B = 256 * K
    bits = np.zeros(B, dtype=np.int64)
    for j, s in enumerate(st):
        for t in range(K):
            p = (j * K + 16 - K + t) % B
            bits[p] = (s >> (K - 1 - t)) & 1
    rebuilt = np.zeros(16 * K, dtype=np.int64)
    for p in range(B):
        rebuilt[p // 16] |= bits[p] << (15 - p % 16)
    np.testing.assert_array_equal(rebuilt, words.astype(np.int64))


def test_tile_grid_and_inner_order():
    # a 48 x 64 matrix (3 x 4 tiles) at K = 4; zero words decode to state 0
    # (v = -254); all-ones words decode to state 0xFFFF (v = 21)
    K, n_in, n_out = 4, 48, 64
    codes = np.zeros((n_in // 16) * (n_out // 16) * 16 * K, dtype=np.uint16)
    tk, tn = 1, 2
    t0 = (tk * (n_out // 16) + tn) * 16 * K
    codes[t0:t0 + 16 * K] = 0xFFFF
    dense = oracle.decode_matrix(codes, n_in, n_out, K, MCG) * 64
    expect = np.full((n_in, n_out), -254.0)
    expect[16 * tk:16 * tk + 16, 16 * tn:16 * tn + 16] = 21.0
    np.testing.assert_array_equal(dense, expect)
    # inside a tile: one set bit at stream position 100 touches the states
    # j = 22..25 (window start 4j <= 100 < 4j + 16); state j sits at input
    # row j % 16 and output column j // 16 of the tile
    tile = np.zeros(16 * K, dtype=np.uint16)
    tile[100 // 16] = 1 << (15 - 100 % 16)
    codes = np.zeros(16 * K, dtype=np.uint16)
    codes[:] = tile
    dense = oracle.decode_matrix(codes, 16, 16, K, MCG) * 64
    expect = np.full((16, 16), -254.0)
    for j in (22, 23, 24, 25):
        s = 1 << (15 - (100 - 4 * j))
        expect[j % 16, j // 16] = oracle.mcg_value(s, MCG)
    np.testing.assert_array_equal(dense, expect)
    assert expect[6, 1] == 129  # j = 22 holds state 8, derived by hand above


def test_e4m3_against_library_and_spec():
    c = np.arange(-254, 255) / 64.0
    ours = np.array([oracle.e4m3_rne(v) for v in c])
    lib = torch.tensor(c, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, lib)
    spot = {17: 16, 18: 18, 19: 20, 33: 32, 35: 36, 100: 96, 127: 128, 254: 256}
    for a, b in spot.items():
        assert oracle.e4m3_rne(a / 64) == b / 64
        assert oracle.e4m3_rne(-a / 64) == -b / 64
    assert int((ours != c).sum()) == 414
    # saturation at the largest finite value (the library cast gives NaN there)
    assert oracle.e4m3_rne(1000.0) == 448.0 and oracle.e4m3_rne(-460.0) == -448.0
    assert oracle.e4m3_rne(464.0) == 448.0
    # subnormals: spacing 2^-9, ties to even
    assert oracle.e4m3_rne(1.5 * 2 ** -9) == 2 ** -8
    assert oracle.e4m3_rne(2 ** -10) == 0.0
    assert oracle.e4m3_rne(3 * 2 ** -10) == 2 ** -8


def test_e4m3_codebook_matrix():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 1 << 16, 4 * 4 * 16 * 3, dtype=np.uint16)
    a = oracle.decode_matrix(codes, 64, 64, 3, MCG, 0)
    b = oracle.decode_matrix(codes, 64, 64, 3, MCG, 1)
    lib = torch.tensor(a).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    np.testing.assert_array_equal(b, lib)


def test_bruteforce_reencode_single_word():
    # one 16-bit word at K = 2 is a tail-biting stream of 8 states; an
    # exhaustive minimum-squared-error search over all 2^16 words must find
    # zero error for any decodable target and reproduce its values
    v = oracle.value_table(MCG).astype(np.float64)
    all_words = np.arange(65536, dtype=np.uint16)
    states = np.stack([oracle.stream_states(all_words[i:i + 1], 2) for i in range(65536)])
    vals = v[states.astype(np.int64)]                      # [65536][8]
    rng = np.random.default_rng(3)
    for w in rng.integers(0, 65536, 8):
        target = vals[w]
        err = ((vals - target) ** 2).sum(axis=1)
        best = int(np.argmin(err))
        assert err[best] == 0.0
        np.testing.assert_array_equal(vals[best], target)
    # single-word window: state j is the word rotated left by 2j bits
    w = 0xBEEF
    st = oracle.stream_states(np.array([w], dtype=np.uint16), 2)
    rot = [((w << (2 * j)) | (w >> (16 - 2 * j))) & 0xFFFF for j in range(8)]
    assert list(st) == rot
