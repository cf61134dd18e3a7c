"""Pins for the oracle's group-shared scan (proxy + refine) and block-pooled coarse filter: hand
cases for the proxy and the pooled keys, and the reductions in which each variant must give
exactly the dense indexer's result."""
import numpy as np
import pytest

import oracle
import workloads as W


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# -------------------------------------------------------------------------- proxy query

def test_proxy_identical_members_is_member():
    p = W.make_prefill(32, 4, 32, seed=1, rho=0.0)
    p.q[0, 8:16] = p.q[0, 8]
    # weights with few significant bits, so that their fp32 partial sums are exact
    p.w[0, 8:16] = (np.round(p.w[0, 8] * 256) / 256).astype(np.float32)
    qb, wb, pos = oracle.proxy_query(p, 0, 1, 8)
    assert np.array_equal(qb, p.q[0, 8]) and np.array_equal(wb, p.w[0, 8]) and pos == 15


def test_proxy_hand_mean():
    # members 1, 2, 4 (bf16 exact): fp32 sum 7, 7/3 = 0x40155555 -> bf16 0x4015 (2.328125)
    H, D = 1, 2
    q = np.array([[1.0, -1.0], [2.0, 1.0], [4.0, 0.0]], np.float32).reshape(1, 3, H, D)
    qb = W.f32_to_bf16_bits(q)
    w = np.array([0.5, 0.25, 1.0], np.float32).reshape(1, 3, 1)
    p = W.Problem(qb, W.BF16, W.f32_to_bf16_bits(np.zeros((1, 4, D), np.float32)), W.BF16, None,
                  w, np.array([[1, 2, 3]], np.int32), np.array([4], np.int32))
    pq, pw, pos = oracle.proxy_query(p, 0, 0, 4)
    assert pq[0].tolist() == [0x4015, 0x0000]     # mean(-1, 1, 0) = 0
    assert pw[0] == np.float32(np.float32(1.75) / np.float32(3.0))
    assert pos == 3


def test_proxy_opposite_members_cancel():
    p = W.make_prefill(4, 2, 16, seed=2, q_dtype=W.F32, k_dtype=W.F32)
    p.q[0, 1] = -p.q[0, 0]
    qb, _, _ = oracle.proxy_query(p, 0, 0, 2)
    assert (qb == 0).all()


# -------------------------------------------------------------------------- group reductions

@pytest.fixture(scope="module")
def pre():
    return W.make_prefill(160, 4, 32, seed=11, rho=0.9)


def test_group_full_candidates_equals_dense(pre):
    k = 24
    d_idx, d_sc = oracle.dense(pre, k)
    for G in (1, 5, 16):
        g_idx, g_sc, _ = oracle.group(pre, k, G, pre.N)      # candidates = whole prefix
        for t in range(pre.T):
            assert set(g_idx[0, t].tolist()) == set(d_idx[0, t].tolist())
        assert np.array_equal(np.sort(g_sc, -1), np.sort(d_sc, -1))


def test_group_singletons_equal_dense(pre):
    k = 24
    d_idx, _ = oracle.dense(pre, k)
    g_idx, _, _ = oracle.group(pre, k, 1, k)                # G=1: proxy == query, C = k
    for t in range(pre.T):
        assert set(g_idx[0, t].tolist()) == set(d_idx[0, t].tolist())


def test_group_outputs_within_candidates(pre):
    k, G, C = 16, 8, 40
    g_idx, _, cands = oracle.group(pre, k, G, C)
    for t in range(pre.T):
        g = t // G
        cand = cands[(0, g)]
        gl = min(pre.T, (g + 1) * G) - 1
        assert len(cand) == min(C, gl + 1)
        sel = g_idx[0, t][g_idx[0, t] >= 0]
        assert set(sel.tolist()) <= set(cand.tolist())
        vis = cand[cand <= t]
        assert len(sel) == min(k, len(vis))


def test_reuse_singletons_equal_dense(pre):
    # G=1: the proxy is the query itself (mean of one value, bf16 of a bf16 value), so sharing
    # its top-k is the dense indexer, scores included
    k = 24
    d_idx, d_sc = oracle.dense(pre, k)
    r_idx, r_sc, _ = oracle.group_reuse(pre, k, 1)
    assert np.array_equal(r_idx, d_idx)
    assert np.array_equal(r_sc, d_sc)


def test_reuse_members_share_the_proxy_topk(pre):
    k, G = 16, 8
    r_idx, r_sc, scans = oracle.group_reuse(pre, k, G)
    inp = oracle.Inputs(pre)
    for (b, g), ps in scans.items():
        mem = list(oracle.group_members(pre.T, G, g))
        top = ps["cand_by_rank"]
        assert len(top) == min(k, ps["P"])
        # the proxy's top-k over its own prefix, ties to the lower token
        ref, _ = oracle.select_topk(ps["proxy_scores"], np.arange(ps["P"]), k)
        assert np.array_equal(top, ref)
        last = max(mem, key=lambda t: pre.q_pos[b, t])
        assert np.array_equal(r_idx[b, last, :len(top)], top)       # the furthest member: all of it
        for t in mem:                                              # the others: its part in their prefix
            sel = r_idx[b, t][r_idx[b, t] >= 0]
            assert np.array_equal(sel, top[top < inp.P(b, t)])
            assert np.array_equal(r_sc[b, t, :len(sel)], ps["proxy_scores"][sel])
            assert (r_idx[b, t, len(sel):] == -1).all()


def test_group_partial_last_group():
    p = W.make_prefill(37, 2, 16, seed=3)
    _, _, cands = oracle.group(p, 8, 16, 20)
    assert sorted(cands) == [(0, 0), (0, 1), (0, 2)]
    qb, wb, pos = oracle.proxy_query(p, 0, 2, 16)             # members 32..36
    assert pos == 36


# -------------------------------------------------------------------------- block pooling

def test_pool_hand_mean_partial_block():
    # block size 3, k_len 5: blocks {1,2,3} -> 2 and {4,8} -> 6 (partial), per dim
    k = np.array([[1, 0], [2, 0], [3, 3], [4, -1], [8, 1], [100, 100]], np.float32)[None]
    p = W.Problem(np.zeros((1, 1, 1, 2), np.float32), W.F32, k, W.F32, None,
                  np.ones((1, 1, 1), np.float32), np.array([[4]], np.int32),
                  np.array([5], np.int32))
    pk = oracle.pool_keys(p, 0, 3)
    assert pk.tolist() == [[2.0, 1.0], [6.0, 0.0]]


def test_pool_block_size_one_is_identity():
    p = W.make_prefill(50, 2, 32, seed=4)
    assert np.array_equal(oracle.pool_keys(p, 0, 1), p.k[0])


def test_pool_constant_block():
    p = W.make_prefill(64, 2, 32, seed=5)
    p.k[0, 16:32] = p.k[0, 16]
    pk = oracle.pool_keys(p, 0, 16)
    assert np.array_equal(pk[1], p.k[0, 16])


def test_block_hand_eligibility():
    # D=1, H=1, w=1, q=1, block size 2, keys 0..5 = 1,1,5,5,9,9 ; pooled 1,5,9
    k = np.array([1, 1, 5, 5, 9, 9], np.float32).reshape(1, 6, 1)
    q = np.ones((1, 2, 1, 1), np.float32)
    p = W.Problem(q, W.F32, k, W.F32, None, np.ones((1, 2, 1), np.float32),
                  np.array([[2, 4]], np.int32), np.array([6], np.int32))
    pooled = oracle.pool_keys(p, 0, 2)
    inp = oracle.Inputs(p)
    # pos 2: blocks 0 and 1 eligible (block 1 starts at 2); keep 1 -> block 1, token 3 is future
    r = oracle.block_row(inp, 0, 0, 4, 2, 1, pooled)
    assert r["blocks"].tolist() == [1] and r["ids"].tolist() == [2]
    # pos 4: block 2 (start 4) eligible and best; only token 4 visible
    r = oracle.block_row(inp, 0, 1, 4, 2, 1, pooled)
    assert r["blocks"].tolist() == [2] and r["ids"].tolist() == [4]
    r = oracle.block_row(inp, 0, 1, 2, 2, 2, pooled)
    assert r["blocks"].tolist() == [1, 2] and r["ids"].tolist() == [4, 2]


@pytest.fixture(scope="module")
def hier():
    return W.make_hier(512, 48, H=4, D=32, seed=7, n_regions=4, region=32)


def test_block_keep_all_equals_dense(hier):
    k = 40
    d_idx, d_sc = oracle.dense(hier, k)
    for bs in (7, 32):
        b_idx, b_sc, _ = oracle.block(hier, k, bs, 10 ** 6)
        for t in range(hier.T):
            assert set(b_idx[0, t].tolist()) == set(d_idx[0, t].tolist())
        assert np.array_equal(np.sort(b_sc, -1), np.sort(d_sc, -1))


def test_block_size_one_keep_k_equals_dense(hier):
    k = 40
    d_idx, _ = oracle.dense(hier, k)
    b_idx, _, _ = oracle.block(hier, k, 1, k)
    for t in range(hier.T):
        assert set(b_idx[0, t].tolist()) == set(d_idx[0, t].tolist())


def test_block_outputs_within_kept_blocks(hier):
    k, bs, keep = 64, 16, 6
    b_idx, _, blks = oracle.block(hier, k, bs, keep)
    for t in range(hier.T):
        kept = blks[0, t][blks[0, t] >= 0]
        assert len(kept) == min(keep, hier.q_pos[0, t] // bs + 1)
        sel = b_idx[0, t][b_idx[0, t] >= 0]
        assert set((sel // bs).tolist()) <= set(kept.tolist())
        assert sel.max() <= hier.q_pos[0, t]


# -------------------------------------------------------------------------- block-filtered proxy

def test_group_block_singletons_equal_block(hier):
    # G=1: the proxy is the query itself, so the result is the hierarchical indexer's
    k, Bs, keep = 16, 8, 5
    b_idx, b_sc = oracle.block(hier, k, Bs, keep)[:2]
    g_idx, g_sc, _ = oracle.group_block(hier, k, 1, Bs, keep)
    assert np.array_equal(g_idx, b_idx)
    assert np.array_equal(g_sc, b_sc)


def test_group_block_keep_all_equals_dense(hier):
    # every eligible block kept: the candidates hold each member's whole prefix
    k = 16
    d_idx, d_sc = oracle.dense(hier, k)
    for G in (1, 6):
        g_idx, g_sc, _ = oracle.group_block(hier, k, G, 8, 10 ** 6)
        for t in range(hier.T):
            assert set(g_idx[0, t].tolist()) == set(d_idx[0, t].tolist())
        assert np.array_equal(np.sort(g_sc, -1), np.sort(d_sc, -1))


def test_group_block_candidates_are_kept_blocks(hier):
    k, G, Bs, keep = 12, 4, 8, 3
    g_idx, _, scans = oracle.group_block(hier, k, G, Bs, keep)
    for (b, g), gs in scans.items():
        assert len(gs["blocks"]) == min(keep, len(gs["block_scores"]))
        assert set((gs["tokens"] // Bs).tolist()) == set(gs["blocks"].tolist())
        for t in oracle.group_members(hier.T, G, g):
            sel = g_idx[b, t][g_idx[b, t] >= 0]
            assert set(sel.tolist()) <= set(gs["tokens"].tolist())


# ---------------------------------------------------------------- FP8 key caches in the block paths

def test_pool_fp8_unit_scales_equal_bf16_pool():
    # every E4M3 value is a bf16 value: with unit scales the FP8 cache pools to exactly what the
    # bf16 cache of the same values pools to
    rng = np.random.default_rng(31)
    p8 = W.make_decode(1, 300, T=2, seed=32)
    b8 = rng.integers(0, 256, size=p8.k.shape).astype(np.uint8)
    p8.k = np.where((b8 & 0x7F) == 0x7F, 0x38, b8).astype(np.uint8)
    p8.k_scale = np.ones_like(p8.k_scale)
    vals = oracle.e4m3fn_bits_to_f64(p8.k).astype(np.float32)
    pb = W.Problem(p8.q, p8.q_dtype, oracle.f32_to_bf16_bits_rne(vals).reshape(p8.k.shape), W.BF16, None,
                   p8.w, p8.q_pos, p8.k_len)
    for Bs in (1, 7, 128):
        assert np.array_equal(oracle.pool_keys(p8, 0, Bs), oracle.pool_keys(pb, 0, Bs))


def test_pool_fp8_hand_block():
    # tokens (1, 2) * 0.5 and (-1, 2) * 3 -> fp32 values (0.5, 1) and (-3, 6): mean (-1.25, 3.5)
    p = W.make_decode(1, 2, T=1, H=1, D=2, seed=33)
    p.k = np.array([[[0x38, 0x40], [0xb8, 0x40]]], np.uint8)
    p.k_scale = np.array([[0.5, 3.0]], np.float32)
    got = oracle.bf16_bits_to_f64(oracle.pool_keys(p, 0, 2))
    assert got.tolist() == [[-1.25, 3.5]]


def test_fp8_block_keep_all_is_dense():
    p = W.make_decode(2, 700, T=2, seed=34, k_len=[700, 333])
    k = 100
    inp = oracle.Inputs(p)
    for b in range(2):
        pooled = oracle.pool_keys(p, b, 16)
        for t in range(2):
            r = oracle.block_row(inp, b, t, k, 16, 10 ** 4, pooled)
            d = oracle.dense_row(inp, b, t, k)
            assert np.array_equal(np.sort(r["ids"]), np.sort(d["ids"]))


def test_fp8_group_block_keep_all_is_dense():
    p = W.make_decode(1, 900, T=2, seed=35)
    k = 64
    out, _, _ = oracle.group_block(p, k, 2, 32, 10 ** 4)
    ref, _ = oracle.dense(p, k)
    for t in range(2):
        assert set(out[0, t].tolist()) == set(ref[0, t].tolist())
