"""GPU parity of the group-shared scan (idx_group_proxy_refine) and the block-pooled
hierarchical indexer (idx_block_coarse_refine) against the oracle. Each stage is compared where
the result is unique: the candidate set / kept blocks against the oracle's proxy / pooled-block
scores (tie band at the n_cand-th / n_keep-th score), and every final row against the oracle's
token scores over the GPU's own candidates. End-to-end agreement with the oracle is reported."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection
from block_checks import check_block

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- group

def run_group(prob, k, G, C):
    t = dev(prob)
    oi, osc, cand = idx.group_proxy_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                           group_size=G, n_cand=C, k_len=t["k_len"],
                                           k_scale=t["k_scale"], return_cand=True)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy(), cand.cpu().numpy()


def check_group(prob, k, G, C, gi, gs, gc, groups, name):
    inp = oracle.Inputs(prob)
    e2e_diff = 0
    e2e_tot = 0
    for b, g in groups:
        ps = oracle.group_proxy_scan(inp, b, g, G, C)
        check_selection(gc[b, g], None, np.arange(ps["P"]), ps["proxy_scores"],
                        ps["proxy_magnitude"], C, prob.D, ctx=f"{name} cand b{b} g{g}",
                        oracle_sel=ps["cand"])
        cand = gc[b, g, :ps["n_cand"]].astype(np.int64)
        assert (np.diff(cand) > 0).all() and (gc[b, g, ps["n_cand"]:] == -1).all()
        for t in oracle.group_members(prob.T, G, g):
            d = oracle.dense_row(inp, b, t, k)
            uni = cand[cand < inp.P(b, t)]
            check_selection(gi[b, t], gs[b, t], uni, d["all_scores"][uni], d["magnitude"][uni],
                            k, prob.D, ctx=f"{name} b{b} t{t}")
            ro = oracle.refine_row(inp, b, t, k, ps["cand"])
            sel = gi[b, t][gi[b, t] >= 0]
            e2e_diff += len(np.setxor1d(sel, ro["ids"])) // 2
            e2e_tot += len(ro["ids"])
    say(f"{name}: end-to-end differences vs oracle {e2e_diff}/{e2e_tot}")


def test_group_small_all_groups():
    p = W.make_prefill(700, 64, 128, seed=21, rho=0.95)
    say("case group L=700 G=16 C=128 k=48")
    gi, gs, gc = run_group(p, 48, 16, 128)
    check_group(p, 48, 16, 128, gi, gs, gc, [(0, g) for g in range(gc.shape[1])], "group-700")


def test_group_ragged_last_group_and_batch():
    p = W.make_prefill(203, 16, 64, seed=22, B=2)
    p.k_len[1] = 150
    say("case group B=2 L=203 G=5 C=60 k=20 (partial last group, k_len < L)")
    gi, gs, gc = run_group(p, 20, 5, 60)
    check_group(p, 20, 5, 60, gi, gs, gc,
                [(b, g) for b in range(2) for g in range(gc.shape[1])], "group-ragged")


def test_group_full_candidates_is_dense():
    p = W.make_prefill(333, 32, 128, seed=23)
    say("case group with n_cand = N (must equal dense)")
    gi, gs, _ = run_group(p, 64, 8, p.N)
    inp = oracle.Inputs(p)
    for t in range(p.T):
        r = oracle.dense_row(inp, 0, t, 64)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"], 64,
                        p.D, ctx=f"full-cand t{t}", oracle_sel=r["ids"])


def test_group_more_candidates_than_cache_is_dense():
    # n_cand = 2N: each proxy keeps its whole prefix, so the result equals the dense indexer's,
    # and out_cand rows hold the prefix in ascending order, then -1 up to n_cand
    p = W.make_prefill(250, 16, 64, seed=25)
    C = 2 * p.N
    say("case group with n_cand = 2N (clamped to each proxy's prefix; must equal dense)")
    gi, gs, gc = run_group(p, 32, 8, C)
    assert gc.shape[-1] == C
    inp = oracle.Inputs(p)
    for g in range(gc.shape[1]):
        P = inp.P(0, min(p.T, 8 * g + 8) - 1)
        assert np.array_equal(gc[0, g, :P], np.arange(P)) and (gc[0, g, P:] == -1).all()
    for t in range(p.T):
        r = oracle.dense_row(inp, 0, t, 32)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"], 32,
                        p.D, ctx=f"cand-2N t{t}", oracle_sel=r["ids"])


def test_group_fp32_and_fp8_inputs():
    for qd, kd in ((W.F32, W.F32), (W.BF16, W.FP8_E4M3)):
        p = W.make_prefill(150, 8, 32, seed=24, q_dtype=qd, k_dtype=kd)
        say(f"case group dtypes q={qd} k={kd}")
        gi, gs, gc = run_group(p, 16, 4, 40)
        check_group(p, 16, 4, 40, gi, gs, gc, [(0, g) for g in range(gc.shape[1])],
                    f"group-q{qd}k{kd}")


@pytest.mark.timeout(1200)
def test_group64k_full_size_sampled_groups():
    spec = W.WORKLOADS["group64k"]
    p = spec["gen"](0)
    G, C, k = spec["group_size"], spec["n_cand"], spec["k"]
    say("case group64k full size (L=65536, G=16, C=8192, k=2048)")
    gi, gs, gc = run_group(p, k, G, C)
    rng = np.random.default_rng(1)
    gs_ = sorted(set([0, 127, 128, 4095] + list(rng.integers(0, 4096, 4))))
    check_group(p, k, G, C, gi, gs, gc, [(0, g) for g in gs_], "group64k")
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(k, np.arange(65536) + 1))


# ----------------------------------------------------------------------------- block

def run_block(prob, k, Bs, keep):
    t = dev(prob)
    oi, osc, blk = idx.block_coarse_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                           block_size=Bs, n_blocks_keep=keep,
                                           k_len=t["k_len"], return_blocks=True)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy(), blk.cpu().numpy()


def test_block_small_all_rows():
    p = W.make_hier(3000, 200, seed=31, n_regions=8, region=64)
    say("case block N=3000 T=200 Bs=64 keep=8 k=128")
    gi, gs, gb = run_block(p, 128, 64, 8)
    check_block(p, 128, 64, 8, gi, gs, gb, [(0, t) for t in range(p.T)], "block-3000")


@pytest.mark.parametrize("Bs,keep", [(7, 30), (100, 3), (1, 64), (33, 1000)])
def test_block_sizes(Bs, keep):
    p = W.make_prefill(500, 16, 64, seed=32 + Bs, B=2)
    p.k_len[1] = 437
    say(f"case block Bs={Bs} keep={keep} (partial blocks, keep-all when keep >= blocks)")
    gi, gs, gb = run_block(p, 48, Bs, keep)
    check_block(p, 48, Bs, keep, gi, gs, gb, [(b, t) for b in range(2) for t in range(p.T)],
                f"block-Bs{Bs}")


@pytest.mark.parametrize("Bs,keep", [(128, 40), (256, 20), (512, 8)])
def test_block_whole_tile_blocks(Bs, keep):
    # blocks of one or more 128-key tiles at H=64, D=128 (the path that takes a tile's keys and
    # kept position per tile), a partial last block, unions of more than 64 tiles
    p = W.make_hier(13000, 96, seed=40 + Bs, n_regions=6, region=Bs)
    say(f"case block Bs={Bs} keep={keep} N=13000 T=96 H=64 D=128")
    gi, gs, gb = run_block(p, 256, Bs, keep)
    check_block(p, 256, Bs, keep, gi, gs, gb, [(0, t) for t in range(p.T)], f"block-big-Bs{Bs}")


def test_block_whole_tile_blocks_d64():
    # D=64 and 32 heads through the whole-tile path (Bs=256), partial last block
    p = W.make_hier(5000, 42, H=32, D=64, seed=45, n_regions=4, region=256)
    say("case block Bs=256 keep=6 N=5000 T=42 H=32 D=64")
    gi, gs, gb = run_block(p, 300, 256, 6)
    check_block(p, 300, 256, 6, gi, gs, gb, [(0, t) for t in range(p.T)], "block-big-d64")


@pytest.mark.parametrize("Bs,keep", [(128, 3), (32, 10)])
def test_block_ragged_tail_tiles(Bs, keep):
    # H=64, D=128: a query count that is not a multiple of the refine's work-group, two sequences
    # with a shorter cache in the second (queries past its end see only the cached keys)
    p = W.make_prefill(1003, 64, 128, seed=60 + Bs, B=2)
    p.k_len[1] = 870
    say(f"case block ragged T=1003 B=2 k_len=(1003, 870) Bs={Bs} keep={keep}")
    gi, gs, gb = run_block(p, 200, Bs, keep)
    check_block(p, 200, Bs, keep, gi, gs, gb, [(b, t) for b in range(2) for t in range(p.T)],
                f"block-ragged-Bs{Bs}")


@pytest.mark.parametrize("N,T,Bs,keep", [(40000, 32, 16, 900), (200000, 16, 128, 500)])
def test_block_union_of_several_rounds(N, T, Bs, keep):
    # uncorrelated queries: the union of a work-group's kept blocks exceeds the 1024 blocks the
    # refine handles per round (counted on the CPU: ~1100 blocks at Bs=128), so it runs in rounds
    p = W.make_hier(N, T, seed=50 + Bs, rho=0.0)
    say(f"case block rounds N={N} T={T} Bs={Bs} keep={keep} H=64 D=128")
    gi, gs, gb = run_block(p, 512, Bs, keep)
    check_block(p, 512, Bs, keep, gi, gs, gb, [(0, t) for t in range(p.T)], f"block-rounds-Bs{Bs}")


def test_block_keep_all_is_dense():
    p = W.make_hier(1500, 100, H=32, D=128, seed=34)
    say("case block keep >= blocks (must equal dense)")
    gi, gs, _ = run_block(p, 256, 32, 10 ** 4)
    inp = oracle.Inputs(p)
    for t in range(p.T):
        r = oracle.dense_row(inp, 0, t, 256)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"], 256,
                        p.D, ctx=f"keep-all t{t}", oracle_sel=r["ids"])


def test_block_fp32_inputs():
    p = W.make_prefill(400, 4, 32, seed=35, q_dtype=W.F32, k_dtype=W.F32)
    say("case block fp32")
    gi, gs, gb = run_block(p, 24, 16, 5)
    check_block(p, 24, 16, 5, gi, gs, gb, [(0, t) for t in range(p.T)], "block-f32")


@pytest.mark.timeout(900)
def test_hier128k_full_size_sampled_rows():
    spec = W.WORKLOADS["hier128k"]
    p = spec["gen"](0)
    Bs, keep, k = spec["block_size"], spec["n_blocks_keep"], spec["k"]
    say("case hier128k full size (N=131072, T=4096, Bs=128, keep=128, k=2048)")
    gi, gs, gb = run_block(p, k, Bs, keep)
    rng = np.random.default_rng(2)
    ts = sorted(set([0, 1, 4095] + list(rng.integers(0, 4096, 9))))
    check_block(p, k, Bs, keep, gi, gs, gb, [(0, t) for t in ts], "hier128k")
    assert ((gi[0] >= 0).sum(-1) == k).all()
