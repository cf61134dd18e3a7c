"""Parity rules between the HIP indexer and the oracle (test helpers, no GPU needed to import).

Scores: |gpu - ref| <= 1e-3 * |ref| + D * 2^-23 * A, where A = sum_h |w_h| sum_d |q_hd k_d| is the
a-priori fp32 dot-product error scale (D * 2^-23 = twice the round-to-nearest bound of a D-term
fp32 sum, so that it also covers truncating accumulation) and 1e-3 relative is the stated score
tolerance.

Index sets: the GPU's set must hold min(k, |universe|) distinct members (in any order) of the
row's universe (the tokens the method lets it choose from). Where it differs from the oracle's
selection, each differing token's oracle score must lie within the tie band of the row's k-th
oracle score tau: |ref_i - tau| <= 1e-3 * |tau| + D * 2^-23 * (A_i + A_tau).

Where several results are correct (ties inside the band), the unique part is compared and the
rest is checked for validity with the oracle's scores.
"""
from __future__ import annotations

import numpy as np

REL = 1e-3


def gamma(D: int) -> float:
    return D * 2.0 ** -23


def score_tol(ref, mag, D):
    return REL * np.abs(ref) + gamma(D) * mag


def kth_largest(scores: np.ndarray, n: int):
    """Index (into scores) of the n-th largest value (n >= 1)."""
    order = np.argsort(-scores, kind="stable")
    return order[n - 1]


def check_selection(gpu_idx, gpu_sc, universe, ref_scores, mag, k, D, ctx="",
                    oracle_sel=None):
    """gpu_idx/gpu_sc: one output row (length k). universe: sorted token ids the row may choose
    from, ref_scores/mag aligned with it (oracle values). oracle_sel: the oracle's own selection
    over the same universe (defaults to its top-k by ref_scores, lower index first on ties)."""
    universe = np.asarray(universe, np.int64)
    n_exp = min(k, len(universe))
    gi = np.asarray(gpu_idx, np.int64)
    gs = np.asarray(gpu_sc, np.float64) if gpu_sc is not None else None
    assert (gi[n_exp:] == -1).all(), f"{ctx}: padding must be -1 beyond {n_exp}"
    if gs is not None:
        assert np.isneginf(gs[n_exp:]).all(), f"{ctx}: padding scores must be -inf"
    sel = gi[:n_exp]
    assert (sel >= 0).all(), f"{ctx}: {np.sum(sel < 0)} missing selections (expected {n_exp})"
    order = np.argsort(sel, kind="stable")      # the row is a set; its order is unspecified
    sel = sel[order]
    if gs is not None:
        gs = np.concatenate([gs[:n_exp][order], gs[n_exp:]])
    assert (np.diff(sel) > 0).all(), f"{ctx}: repeated token in the selection"
    if n_exp == 0:
        return 0
    pos = np.searchsorted(universe, sel)
    assert (pos < len(universe)).all() and (universe[np.minimum(pos, len(universe) - 1)] == sel).all(), \
        f"{ctx}: selection outside the row's universe"
    if gs is not None:
        r, m = ref_scores[pos], mag[pos]
        err = np.abs(gs[:n_exp] - r)
        tol = score_tol(r, m, D)
        bad = err > tol
        assert not bad.any(), (f"{ctx}: {bad.sum()} scores off, worst err {err.max():.3e} "
                               f"at ref {r[np.argmax(err - tol)]:.6e}")
    if oracle_sel is None:
        order = np.lexsort((universe, -ref_scores))[:n_exp]
        oracle_sel = universe[order]
    kth = kth_largest(ref_scores, n_exp)
    tau, mtau = ref_scores[kth], mag[kth]
    diff = np.setxor1d(sel, oracle_sel)
    if len(diff):
        dp = np.searchsorted(universe, diff)
        band = REL * abs(tau) + gamma(D) * (mag[dp] + mtau)
        far = np.abs(ref_scores[dp] - tau) > band
        assert not far.any(), (f"{ctx}: {far.sum()} selection differences outside the tie band "
                               f"(tau {tau:.6e}; e.g. token {diff[far][0]} ref "
                               f"{ref_scores[dp][far][0]:.6e})")
    return len(diff) // 2

