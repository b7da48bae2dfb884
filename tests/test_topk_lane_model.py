"""A host model of the wavefront top-k selection in the routing kernel
(topk_token): 64 lanes, lane l holding experts l, l + 64, ...; each round every
lane offers its best remaining (logit, expert), a wave maximum picks the
value, a ballot of the lanes holding it names the winner (the lowest expert
among several).  The model shows on the CPU that the selection with NaN logits
ranked as -inf always yields a valid expert and agrees with the oracle, and
that the selection without that step (fmax ignores NaN, the ballot then finds
no lane) yields the out-of-range sentinel for a token whose logits are all NaN.
"""
import numpy as np
import pytest

import oracle

NO_EXPERT = 0x7FFFFFFF


def _fmax(a, b):
    # IEEE maxNum, as v_max_f32: a NaN operand yields the other operand
    if np.isnan(a):
        return b
    if np.isnan(b):
        return a
    return max(a, b)


def lane_topk(logits_row, k, nan_as_minus_inf=True):
    E = logits_row.size
    nper = (E + 63) // 64
    v = np.full((64, nper), -np.inf, dtype=np.float32)
    key = np.full((64, nper), NO_EXPERT, dtype=np.int64)
    for l in range(64):
        for i in range(nper):
            e = l + 64 * i
            if e < E:
                x = logits_row[e]
                v[l, i] = -np.inf if (nan_as_minus_inf and np.isnan(x)) else x
                key[l, i] = e
    chosen = []
    for _ in range(k):
        bv = np.full(64, -np.inf, dtype=np.float32)
        bi = np.full(64, NO_EXPERT, dtype=np.int64)
        for l in range(64):
            for i in range(nper):
                if key[l, i] != NO_EXPERT and (bi[l] == NO_EXPERT or v[l, i] > bv[l]):
                    bv[l], bi[l] = v[l, i], key[l, i]
        m = -np.inf
        for l in range(64):
            m = _fmax(m, -np.inf if bi[l] == NO_EXPERT else bv[l])
        tie = [l for l in range(64) if bi[l] != NO_EXPERT and bv[l] == m]
        win = int(bi[tie[0]]) if len(tie) == 1 else min([int(bi[l]) for l in tie], default=NO_EXPERT)
        chosen.append(win)
        if win != NO_EXPERT:
            l = win & 63
            key[l][key[l] == win] = NO_EXPERT
    return np.array(chosen)


def _rows(E, rng):
    rows = [rng.standard_normal(E).astype(np.float32) for _ in range(6)]
    r = rng.standard_normal(E).astype(np.float32)
    r[rng.random(E) < 0.5] = np.nan
    rows.append(r)
    rows.append(np.full(E, np.nan, dtype=np.float32))
    r = np.full(E, -np.inf, dtype=np.float32)
    r[::7] = np.nan
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32)
    r[5 % E] = r[70 % E] = r[200 % E] = 9.0  # ties across lanes
    r[3 % E] = np.inf
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("E,k", [(8, 2), (288, 8), (300, 16), (64, 16)])
def test_lane_model_with_nan_ranking_matches_oracle(E, k):
    rng = np.random.default_rng(E + k)
    lg = _rows(E, rng)
    ref, _ = oracle.topk_softmax(lg, k)
    for t in range(lg.shape[0]):
        got = lane_topk(lg[t], k)
        assert ((got >= 0) & (got < E)).all()
        np.testing.assert_array_equal(got, ref[t])


def test_lane_model_without_nan_ranking_loses_the_winner():
    # the defect the NaN ranking removes: an all-NaN token gets no valid expert
    lg = np.full(288, np.nan, dtype=np.float32)
    got = lane_topk(lg, 8, nan_as_minus_inf=False)
    assert (got == NO_EXPERT).all()
    np.testing.assert_array_equal(lane_topk(lg, 8), np.arange(8))
