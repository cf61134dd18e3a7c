"""Pins for the parity rules themselves: the oracle's error scale (score_magnitude), which sets
the absolute half of every score tolerance and tie band, and the selection checker
(tests/parity.check_selection), which must reject every kind of wrong output row. CPU only."""
import numpy as np
import pytest

import oracle
from parity import REL, check_selection, gamma, score_tol

# The hand case of test_oracle_dense: H=2, D=2, q heads (2,-1) and (1,3), w = (0.5, 2).
#   A[s] = sum_h |w_h| sum_d |q_hd k_sd|
#   key (1,0):  h0 |2|+0 = 2,  h1 |1|+0 = 1   ->  0.5*2 + 2*1 = 3
#   key (0,1):  h0 0+|-1| = 1, h1 0+|3| = 3   ->  0.5*1 + 2*3 = 6.5
#   key (1,1):  h0 2+1 = 3,    h1 1+3 = 4     ->  0.5*3 + 2*4 = 9.5
#   key (-1,2): h0 2+2 = 4,    h1 1+6 = 7     ->  0.5*4 + 2*7 = 16
HQ = np.array([[2.0, -1.0], [1.0, 3.0]])
HW = np.array([0.5, 2.0])
HK = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 2.0]])
HA = [3.0, 6.5, 9.5, 16.0]


def test_score_magnitude_hand_case():
    assert oracle.score_magnitude(HQ, HW, HK).tolist() == HA


def test_score_magnitude_takes_absolute_values_of_every_factor():
    # negating the weights, a query head, or a key component leaves A unchanged
    assert oracle.score_magnitude(HQ, -HW, HK).tolist() == HA
    q2 = HQ.copy()
    q2[1] *= -1
    assert oracle.score_magnitude(q2, HW, HK).tolist() == HA
    assert oracle.score_magnitude(HQ, HW, -HK).tolist() == HA
    # a single term: |w| |q| |k| with w = -3, q = 2, k = -5  ->  30
    assert oracle.score_magnitude(np.array([[2.0]]), np.array([-3.0]), np.array([[-5.0]])).tolist() == [30.0]


def test_score_magnitude_bounds_the_score():
    # |I[s]| <= A[s] for every key (each ReLU term is at most the sum of absolute products)
    rng = np.random.default_rng(5)
    q, w, k = rng.normal(size=(8, 16)), rng.normal(size=8), rng.normal(size=(50, 16))
    assert (np.abs(oracle.index_scores(q, w, k)) <= oracle.score_magnitude(q, w, k) + 1e-12).all()


def test_score_tol_formula():
    # 1e-3 relative plus D * 2^-23 times the magnitude
    assert gamma(128) == 128 * 2.0 ** -23
    np.testing.assert_allclose(score_tol(np.array([-2.0, 0.0]), np.array([4.0, 1.0]), 64),
                               [2e-3 + 64 * 2.0 ** -23 * 4.0, 64 * 2.0 ** -23])


# A synthetic row: 40 tokens of a universe with gaps, well separated scores except for a near-tie
# at the k-th place, small magnitudes (so that the band is about 1e-3 * |tau|).
D = 128
K = 8


def _row():
    universe = np.arange(0, 80, 2, dtype=np.int64)           # 40 even tokens
    rng = np.random.default_rng(0)
    ref = np.linspace(10.0, 1.0, len(universe))[rng.permutation(len(universe))]
    mag = np.full(len(universe), 0.5)
    order = np.lexsort((universe, -ref))
    # make the (K+1)-th score a near-tie of the K-th one (inside the band)
    tau = ref[order[K - 1]]
    ref[order[K]] = tau - 0.2 * REL * abs(tau)
    return universe, ref, mag, order


def _out(tokens, scores, k=K):
    idx = np.full(k, -1, np.int64)
    sc = np.full(k, -np.inf)
    idx[:len(tokens)] = tokens
    sc[:len(tokens)] = scores
    return idx, sc


def _exact(universe, ref, order, k=K):
    sel = order[:k]
    return _out(universe[sel], ref[sel], k)


def test_accepts_the_oracle_selection_in_any_order():
    universe, ref, mag, order = _row()
    gi, gs = _exact(universe, ref, order)
    assert check_selection(gi, gs, universe, ref, mag, K, D) == 0
    p = np.random.default_rng(1).permutation(K)
    assert check_selection(gi[p], gs[p], universe, ref, mag, K, D) == 0


def test_accepts_a_swap_inside_the_tie_band():
    universe, ref, mag, order = _row()
    gi, gs = _exact(universe, ref, order)
    gi[K - 1], gs[K - 1] = universe[order[K]], ref[order[K]]
    assert check_selection(gi, gs, universe, ref, mag, K, D) == 1


def test_rejects_a_swap_ten_bands_below_tau():
    universe, ref, mag, order = _row()
    tau = ref[order[K - 1]]
    band = REL * abs(tau) + gamma(D) * 2 * 0.5
    far = order[K + 1]
    ref[far] = tau - 10 * band
    gi, gs = _exact(universe, ref, order)
    gi[K - 1], gs[K - 1] = universe[far], ref[far]
    with pytest.raises(AssertionError, match="tie band"):
        check_selection(gi, gs, universe, ref, mag, K, D)


def test_rejects_a_score_off_by_2e_3_relative():
    universe, ref, mag, order = _row()
    gi, gs = _exact(universe, ref, order)
    gs[3] *= 1 + 2e-3
    with pytest.raises(AssertionError, match="scores off"):
        check_selection(gi, gs, universe, ref, mag, K, D)
    # the same error on a score of a row without scores passes (only the set is checked)
    assert check_selection(gi, None, universe, ref, mag, K, D) == 0


def test_rejects_a_repeated_token():
    universe, ref, mag, order = _row()
    gi, gs = _exact(universe, ref, order)
    gi[5], gs[5] = gi[4], gs[4]
    with pytest.raises(AssertionError, match="repeated"):
        check_selection(gi, gs, universe, ref, mag, K, D)


def test_rejects_a_token_outside_the_universe():
    universe, ref, mag, order = _row()
    gi, gs = _exact(universe, ref, order)
    gi[2] = universe[order[2]] + 1                            # odd token: not in the universe
    with pytest.raises(AssertionError, match="outside"):
        check_selection(gi, gs, universe, ref, mag, K, D)


def test_rejects_wrong_padding():
    universe, ref, mag, order = _row()
    # a row of 5 candidates: 5 selections, then -1 / -inf
    u5, r5, m5 = universe[:5], ref[:5], mag[:5]
    o5 = np.lexsort((u5, -r5))
    gi, gs = _out(u5[o5], r5[o5])
    assert check_selection(gi, gs, u5, r5, m5, K, D) == 0
    bad = gi.copy()
    bad[6] = 0
    with pytest.raises(AssertionError, match="padding must be -1"):
        check_selection(bad, gs, u5, r5, m5, K, D)
    bad_s = gs.copy()
    bad_s[7] = 0.0
    with pytest.raises(AssertionError, match="padding scores"):
        check_selection(gi, bad_s, u5, r5, m5, K, D)
    short = gi.copy()
    short[4] = -1                                             # one selection missing
    with pytest.raises(AssertionError, match="missing"):
        check_selection(short, gs, u5, r5, m5, K, D)
