"""GPU parity of the dense indexer with FP8 queries and FP8 keys (the q.k contraction on the FP8 x
FP8 matrix cores) against the oracle on the dequantised inputs: every row of small prefills, the
head and dimension shapes, degenerate and tied rows, and the full-size workloads on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection

pytestmark = pytest.mark.gpu


def fp8_prefill(L, H, D, seed, **kw):
    return W.make_prefill(L, H, D, seed=seed, q_dtype=W.FP8_E4M3, k_dtype=W.FP8_E4M3, **kw)


def run(prob, k, **kw):
    t = dev(prob)
    oi, osc = idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"],
                             k_scale=t["k_scale"], q_scale=t["q_scale"], **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy()


def check_rows(prob, k, gi, gs, rows, name):
    inp = oracle.Inputs(prob)
    flips = 0
    for b, t in rows:
        r = oracle.dense_row(inp, b, t, k)
        flips += check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"],
                                 k, prob.D, ctx=f"{name} b{b} t{t}", oracle_sel=r["ids"])
    return flips


def test_fp8_prefill_all_rows():
    p = fp8_prefill(700, 64, 128, seed=71)
    say("case fp8 x fp8 prefill L=700 H=64 D=128 k=128, every row")
    gi, gs = run(p, 128)
    check_rows(p, 128, gi, gs, [(0, t) for t in range(p.T)], "fp8-700")


@pytest.mark.parametrize("H,D", [(8, 64), (48, 64), (100, 128), (128, 128), (1, 128), (64, 64)])
def test_fp8_head_and_dim_shapes(H, D):
    p = fp8_prefill(300, H, D, seed=H + D + 70)
    say(f"case fp8 shapes H={H} D={D}")
    gi, gs = run(p, 40)
    check_rows(p, 40, gi, gs, [(0, t) for t in range(p.T)], f"fp8-H{H}D{D}")


def test_fp8_degenerate_and_ragged():
    p = fp8_prefill(90, 64, 128, seed=72, B=2)
    p.q_pos[0, :16] = -1                     # two whole tiles of empty prefixes
    p.k_len[1] = 50                          # ragged cache
    p.q_pos[1, 80:] = 1000                   # beyond the cache
    p.w[0, 30:40] *= -1.0                    # negative head weights
    p.w[1, 20:25] = 0.0                      # all-zero scores (ties)
    p.q_scale[0, 50:60] *= 3.0               # larger query scales
    say("case fp8 degenerate: empty tiles, ragged k_len, negative and zero weights")
    gi, gs = run(p, 64)
    check_rows(p, 64, gi, gs, [(b, t) for b in range(2) for t in range(p.T)], "fp8-degenerate")
    assert (gi[0, :16] == -1).all() and np.isneginf(gs[0, :16]).all()


def test_fp8_exact_ties_keep_lowest_slots():
    p = fp8_prefill(1200, 64, 128, seed=73)
    p.k[0, 300:] = np.tile(p.k[0, :100], (9, 1))
    p.k_scale[0, 300:] = np.tile(p.k_scale[0, :100], 9)      # equal keys, equal scores
    p.w[0, 1000:1005] = 0.0
    k = 300
    say("case fp8 exact ties: repeated keys and all-zero rows, L=1200 k=300")
    gi, gs = run(p, k)
    check_rows(p, k, gi, gs, [(0, t) for t in list(range(299, 1200, 61)) + list(range(1000, 1005))], "fp8-ties")
    for t in range(1000, 1005):
        assert set(gi[0, t].tolist()) == set(range(k)), f"fp8 ties t{t}"


@pytest.mark.timeout(900)
def test_dense16k_fp8_full_size_sampled_rows():
    spec = W.WORKLOADS["dense16k_fp8"]
    p = spec["gen"](0)
    say("case dense16k_fp8 full size (L=16384, H=64, D=128, fp8 x fp8, k=2048)")
    gi, gs = run(p, spec["k"])
    rng = np.random.default_rng(5)
    ts = sorted(set([0, 7, 8, 2047, 2048, 8191, 16383] + [256 * j + int(rng.integers(0, 256)) for j in range(64)]))
    flips = check_rows(p, spec["k"], gi, gs, [(0, t) for t in ts], "dense16k_fp8")
    say(f"dense16k_fp8: {len(ts)} rows checked, {flips} tie-band swaps")
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(spec["k"], np.arange(16384) + 1))
    assert (gi[0].max(-1) <= np.arange(16384)).all()


@pytest.mark.timeout(1200)
def test_dense64k_fp8_full_size_sampled_rows():
    spec = W.WORKLOADS["dense64k_fp8"]
    p = spec["gen"](0)
    say("case dense64k_fp8 full size (L=65536, H=64, D=128, fp8 x fp8, k=2048)")
    gi, gs = run(p, spec["k"])
    rng = np.random.default_rng(6)
    ts = sorted(set([0, 2047, 2048, 65535] + [4096 * j + d for j in range(1, 16, 3) for d in (-1, 0)] +
                    list(rng.integers(0, 65536, 6))))
    flips = check_rows(p, spec["k"], gi, gs, [(0, t) for t in ts], "dense64k_fp8")
    say(f"dense64k_fp8: {len(ts)} rows checked, {flips} tie-band swaps")
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(spec["k"], np.arange(65536) + 1))
