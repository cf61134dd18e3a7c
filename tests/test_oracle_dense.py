"""Pins for the oracle's dense indexer: hand-computed cases, brute force on tiny inputs, and the
invariants the method fixes (causal prefix, k clamp, head and key symmetries, scaling)."""
import itertools
import math

import numpy as np
import pytest

import oracle
import workloads as W


def _prob(q, k, w, q_pos, k_len=None, k_dtype=W.F32, k_scale=None):
    q = np.asarray(q, np.float32)
    k = np.asarray(k)
    w = np.asarray(w, np.float32)
    if q.ndim == 2:                     # one query [H,D]
        q, w = q[None, None], w[None, None]
    if k.ndim == 2:
        k = k[None]
        if k_scale is not None:
            k_scale = np.asarray(k_scale, np.float32)[None]
    q_pos = np.asarray(q_pos, np.int32).reshape(q.shape[0], q.shape[1])
    if k_len is None:
        k_len = np.full(q.shape[0], k.shape[1], np.int32)
    return W.Problem(q, W.F32, k if k_dtype != W.F32 else np.asarray(k, np.float32), k_dtype,
                     k_scale, w, q_pos, np.asarray(k_len, np.int32))


# hand case: H=2, D=2, q heads (2,-1) and (1,3), w = (0.5, 2)
#   key      h0 dot  h1 dot   score = 0.5*relu(h0) + 2*relu(h1)
#   (1, 0)     2       1      1 + 2  = 3.0
#   (0, 1)    -1       3      0 + 6  = 6.0
#   (1, 1)     1       4      0.5 + 8 = 8.5
#   (-1, 2)   -4       5      0 + 10 = 10.0
HQ = [[2.0, -1.0], [1.0, 3.0]]
HW = [0.5, 2.0]
HK = [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 2.0]]
HS = [3.0, 6.0, 8.5, 10.0]


def test_hand_scores():
    inp = oracle.Inputs(_prob(HQ, HK, HW, 3))
    r = oracle.dense_row(inp, 0, 0, 4)
    assert r["all_scores"].tolist() == HS


@pytest.mark.parametrize("pos,k,ids,scores", [
    (3, 2, [3, 2], [10.0, 8.5]),
    (3, 3, [3, 2, 1], [10.0, 8.5, 6.0]),
    (1, 2, [1, 0], [6.0, 3.0]),       # causal: keys 2 and 3 are in the future
    (0, 2, [0], [3.0]),               # own token is visible; k clamped to the prefix
    (-1, 2, [], []),                  # empty prefix
    (2, 4, [2, 1, 0], [8.5, 6.0, 3.0]),
])
def test_hand_selection(pos, k, ids, scores):
    out_idx, out_sc = oracle.dense(_prob(HQ, HK, HW, pos), k)
    n = len(ids)
    assert out_idx[0, 0, :n].tolist() == ids
    assert out_sc[0, 0, :n].tolist() == scores
    assert (out_idx[0, 0, n:] == -1).all() and np.isneginf(out_sc[0, 0, n:]).all()


def test_hand_ties_prefer_lower_index():
    # H=1, D=1, w=1, q=1: scores are relu(key) = 1, 2, 2, 2, 0
    p = _prob([[1.0]], [[1.0], [2.0], [2.0], [2.0], [-1.0]], [1.0], 4)
    assert oracle.dense(p, 2)[0][0, 0].tolist() == [1, 2]
    assert oracle.dense(p, 4)[0][0, 0].tolist() == [1, 2, 3, 0]
    assert oracle.dense(p, 5)[0][0, 0].tolist() == [1, 2, 3, 0, 4]


def test_hand_negative_weight():
    # q heads (1) and (-1), w = (1, -2): key 3 -> 3 + 0 = 3; key -2 -> 0 - 2*2 = -4; key 0 -> 0
    p = _prob([[1.0], [-1.0]], [[3.0], [-2.0], [0.0]], [1.0, -2.0], 2)
    idx, sc = oracle.dense(p, 3)
    assert idx[0, 0].tolist() == [0, 2, 1] and sc[0, 0].tolist() == [3.0, 0.0, -4.0]


def test_hand_fp8_scale():
    # E4M3 byte 0x38 = 1.0, 0x40 = 2.0, 0xb8 = -1.0; per-token scales 0.5 and 3
    k8 = np.array([[0x38, 0x40], [0xb8, 0x38]], np.uint8)
    p = _prob([[1.0, 1.0]], k8, [1.0], 1, k_dtype=W.FP8_E4M3, k_scale=[0.5, 3.0])
    # real keys (0.5, 1.0) and (-3, 3): dots 1.5 and 0
    r = oracle.dense_row(oracle.Inputs(p), 0, 0, 2)
    assert r["all_scores"].tolist() == [1.5, 0.0]


def _brute_scores(q, w, keys):
    out = []
    for key in keys:
        tot = []
        for h in range(len(w)):
            x = math.fsum(float(q[h][d]) * float(key[d]) for d in range(len(key)))
            tot.append(float(w[h]) * max(x, 0.0))
        out.append(math.fsum(tot))
    return out


def test_brute_force_scores_and_topk():
    rng = np.random.default_rng(3)
    for trial in range(20):
        H, D, N = rng.integers(1, 5), rng.integers(1, 6), rng.integers(1, 8)
        q = rng.standard_normal((H, D)).astype(np.float32)
        w = (rng.standard_normal(H)).astype(np.float32)
        keys = rng.standard_normal((N, D)).astype(np.float32)
        pos = int(rng.integers(0, N))
        p = _prob(q, keys, w, pos)
        r = oracle.dense_row(oracle.Inputs(p), 0, 0, 0)
        ref = _brute_scores(q, w, keys[: pos + 1])
        assert np.allclose(r["all_scores"], ref, rtol=1e-12, atol=1e-12)
        for k in range(0, pos + 3):
            sel = oracle.dense_row(oracle.Inputs(p), 0, 0, k)["ids"]
            kk = min(k, pos + 1)
            best = max(itertools.combinations(range(pos + 1), kk),
                       key=lambda c: (math.fsum(ref[i] for i in c), [-i for i in c]))
            assert sorted(sel.tolist()) == sorted(best)


@pytest.fixture(scope="module")
def tiny():
    return W.make_tiny(0, L=256)


def test_invariants_tiny(tiny):
    k = 64
    idx, sc = oracle.dense(tiny, k)
    inp = oracle.Inputs(tiny)
    for t in range(tiny.T):
        n = min(k, t + 1)
        sel = idx[0, t, :n]
        assert (idx[0, t, n:] == -1).all()
        assert len(set(sel.tolist())) == n
        assert sel.max() <= t                       # never a future token
        if t + 1 <= k:
            assert sorted(sel.tolist()) == list(range(t + 1))
        r = oracle.dense_row(inp, 0, t, k)
        unsel = np.setdiff1d(np.arange(t + 1), sel)
        if len(unsel):
            assert r["all_scores"][sel].min() >= r["all_scores"][unsel].max()


def test_head_permutation_invariance(tiny):
    perm = np.random.default_rng(5).permutation(tiny.H)
    p2 = W.Problem(tiny.q[:, :, perm], tiny.q_dtype, tiny.k, tiny.k_dtype, None,
                   tiny.w[:, :, perm], tiny.q_pos, tiny.k_len)
    a, sa = oracle.dense(tiny, 32)
    b, sb = oracle.dense(p2, 32)
    for t in range(tiny.T):
        assert set(a[0, t].tolist()) == set(b[0, t].tolist())
    assert np.allclose(sa, sb, rtol=1e-12, atol=0)


def test_weight_scaling(tiny):
    p2 = W.Problem(tiny.q, tiny.q_dtype, tiny.k, tiny.k_dtype, None, tiny.w * np.float32(2.0),
                   tiny.q_pos, tiny.k_len)
    a, sa = oracle.dense(tiny, 16)
    b, sb = oracle.dense(p2, 16)
    assert np.array_equal(a, b)
    fin = np.isfinite(sa)
    assert np.array_equal(sb[fin], 2 * sa[fin])


def test_fp8_scale_scales_scores():
    p = W.make_decode(1, 512, T=2, H=4, D=32, seed=2)
    sc2 = p.k_scale.copy()
    c = np.where(np.arange(512) % 3 == 0, 2.0, 0.5).astype(np.float32)
    sc2[0] *= c
    p2 = W.Problem(p.q, p.q_dtype, p.k, p.k_dtype, sc2, p.w, p.q_pos, p.k_len)
    r1 = oracle.dense_row(oracle.Inputs(p), 0, 1, 10)
    r2 = oracle.dense_row(oracle.Inputs(p2), 0, 1, 10)
    assert np.array_equal(r2["all_scores"], r1["all_scores"] * c)


def test_key_permutation_equivariance():
    rng = np.random.default_rng(7)
    N, H, D = 40, 3, 8
    q = rng.standard_normal((1, 3, H, D)).astype(np.float32)
    keys = rng.standard_normal((1, N, D)).astype(np.float32)
    w = rng.random((1, 3, H)).astype(np.float32)
    pos = np.full((1, 3), N - 1, np.int32)
    p1 = W.Problem(q, W.F32, keys, W.F32, None, w, pos, np.array([N], np.int32))
    perm = rng.permutation(N)
    p2 = W.Problem(q, W.F32, keys[:, perm], W.F32, None, w, pos, np.array([N], np.int32))
    a, _ = oracle.dense(p1, 10)
    b, _ = oracle.dense(p2, 10)
    for t in range(3):
        assert set(perm[b[0, t]].tolist()) == set(a[0, t].tolist())


def test_decode_row_equals_prefill_row():
    # the decode queries at positions N-2, N-1 are prefill rows of the same cache
    pre = W.make_prefill(96, 4, 32, seed=4, k_dtype=W.BF16)
    dec = W.Problem(pre.q[:, 94:96], pre.q_dtype, pre.k, pre.k_dtype, None, pre.w[:, 94:96],
                    pre.q_pos[:, 94:96], pre.k_len)
    a, sa = oracle.dense(pre, 20)
    b, sb = oracle.dense(dec, 20)
    assert np.array_equal(a[:, 94:96], b) and np.array_equal(sa[:, 94:96], sb)


def test_k_len_limits_prefix():
    p = W.make_prefill(64, 2, 16, seed=6, q_dtype=W.F32, k_dtype=W.F32)
    p.k_len[:] = 40
    idx, _ = oracle.dense(p, 64)
    assert idx.max() == 39
    assert (idx[0, 50] >= 0).sum() == 40
