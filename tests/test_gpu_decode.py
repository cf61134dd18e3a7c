"""GPU parity of the decode-shaped indexer (idx_score_topk with T <= 4 queries per sequence over a
long cache: the streaming scan and the multi-work-group selector) against the oracle.

Covers every FP8 E4M3 code through the in-register conversion (exact scores), exact ties at the
k-th score (lowest token index first) including the selector's candidate-list overflow paths,
odd T, head counts that are not multiples of 16, D = 64, bf16 keys, empty and clamped prefixes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection

pytestmark = pytest.mark.gpu


def run(prob, k):
    t = dev(prob)
    oi, osc = idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"],
                             k_scale=t["k_scale"])
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy()


def exact_rows(prob, k, gi, gs, rows, name):
    """Scores that are exact in fp32: the selected set must be the oracle's (ties to the lowest
    index) and every score must be bit-equal."""
    inp = oracle.Inputs(prob)
    for b, t in rows:
        r = oracle.dense_row(inp, b, t, k)
        n = len(r["ids"])
        sel = gi[b, t, :n]
        order = np.argsort(sel)
        assert (gi[b, t, n:] == -1).all() and np.isneginf(gs[b, t, n:]).all(), f"{name} b{b} t{t}"
        assert np.array_equal(sel[order], np.sort(r["ids"])), f"{name} b{b} t{t}: selection differs"
        ref = r["all_scores"][np.searchsorted(r["universe"], sel[order])]
        assert np.array_equal(gs[b, t, :n][order].astype(np.float64), ref), f"{name} b{b} t{t}: scores"


def fp8_code_problem(N=4096):
    """Key i holds E4M3 code i % 256 (the NaN codes replaced by zero) at every position, scaled
    by 2^(i // 256 - 8); query 0 is +e_0, query 1 is -e_0 on head 0, so their scores are
    relu(+-value) * scale exactly."""
    H, D = 4, 64
    codes = (np.arange(N) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    k = np.repeat(codes[:, None], D, axis=1)[None].copy()
    scale = np.exp2(np.arange(N) // 256 - 8).astype(np.float32)[None]
    q = np.zeros((1, 2, H, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 1, 0, 0] = -1.0
    qb = W.f32_to_bf16_bits(q)
    w = np.ones((1, 2, H), np.float32)
    q_pos = np.full((1, 2), N - 1, np.int32)
    return W.Problem(qb, W.BF16, k, W.FP8_E4M3, scale, w, q_pos, np.array([N], np.int32))


@pytest.mark.parametrize("k", [4096, 2500, 1000])
def test_decode_every_fp8_code_exact(k):
    p = fp8_code_problem()
    say(f"case decode fp8 every code, k={k} (exact scores, tie resolution)")
    gi, gs = run(p, k)
    exact_rows(p, k, gi, gs, [(0, 0), (0, 1)], f"fp8-codes-k{k}")


def test_decode_all_scores_equal_overflow():
    # zero head weights: every score is 0, so the k-th score's bin holds the whole row; rows of
    # 40000 slots overflow the candidate list, rows of 10000 keep it in global memory
    p = W.make_decode(2, 40000, T=2, seed=41, k_len=[40000, 10000])
    p.w[:] = 0.0
    say("case decode all-equal scores B=2 N=40000 (candidate overflow, index ties)")
    gi, gs = run(p, 2048)
    for b in range(2):
        for t in range(2):
            assert np.array_equal(np.sort(gi[b, t]), np.arange(2048)), f"b{b} t{t}"
            assert (gs[b, t] == 0).all()


@pytest.mark.parametrize("H,D,T,kd", [(20, 64, 3, W.BF16), (64, 128, 1, W.FP8_E4M3),
                                      (33, 128, 2, W.BF16), (64, 64, 4, W.FP8_E4M3)])
def test_decode_shapes(H, D, T, kd):
    p = W.make_decode(2, 6000, T=T, H=H, D=D, seed=42 + H + T, k_dtype=kd, k_len=[6000, 2345])
    say(f"case decode shapes H={H} D={D} T={T} k_dtype={kd}")
    gi, gs = run(p, 700)
    inp = oracle.Inputs(p)
    for b in range(2):
        for t in range(T):
            r = oracle.dense_row(inp, b, t, 700)
            check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"],
                            700, D, ctx=f"decode H{H} D{D} T{T} b{b} t{t}", oracle_sel=r["ids"])


def test_decode_empty_and_clamped_prefixes():
    p = W.make_decode(3, 3000, T=2, seed=43, k_len=[3000, 3000, 2500])
    p.k_len[0] = 0                           # empty cache
    p.q_pos[1, 0] = -1                       # empty prefix
    p.q_pos[1, 1] = 10                       # 11 visible keys
    p.q_pos[2, :] = 5000                     # beyond the cache: clamped to k_len
    say("case decode empty cache, empty prefix, short prefix, clamp, k > prefix")
    gi, gs = run(p, 2600)
    inp = oracle.Inputs(p)
    for b in range(3):
        for t in range(2):
            r = oracle.dense_row(inp, b, t, 2600)
            check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"],
                            2600, p.D, ctx=f"decode-empty b{b} t{t}", oracle_sel=r["ids"])
    assert (gi[0] == -1).all() and (gi[1, 0] == -1).all()
    assert (gi[1, 1] >= 0).sum() == 11 and (gi[2] >= 0).sum(-1).tolist() == [2500, 2500]


def test_decode_repeatable_sets():
    p = W.make_decode(4, 8192, T=2, seed=44)
    say("case decode repeatability (sets and scores)")
    a = run(p, 2048)
    b = run(p, 2048)
    for x, y in ((a, b),):
        oa = np.argsort(x[0], axis=-1)
        ob = np.argsort(y[0], axis=-1)
        assert np.array_equal(np.take_along_axis(x[0], oa, -1), np.take_along_axis(y[0], ob, -1))
        assert np.array_equal(np.take_along_axis(x[1], oa, -1).view(np.uint32),
                              np.take_along_axis(y[1], ob, -1).view(np.uint32))


def test_decode_many_segments_streaming_select():
    # one sequence: the scan cuts the cache into ~1K-key sub-chunks, more than the selector's
    # chunk table holds (64 segments), so the selector streams the candidates in batches
    p = W.make_decode(1, 70000, T=2, seed=45)
    say("case decode B=1 N=70000 (69 sub-chunks, streaming selector)")
    gi, gs = run(p, 2048)
    inp = oracle.Inputs(p)
    for t in range(2):
        r = oracle.dense_row(inp, 0, t, 2048)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"],
                        2048, p.D, ctx=f"decode-segments t{t}", oracle_sel=r["ids"])
