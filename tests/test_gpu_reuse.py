"""GPU parity of PIVOT-Reuse (idx_group_proxy_reuse) against the oracle, and of decode-phase
grouping (a group = one step's multi-token-prediction queries) for both PIVOT variants. The
proxy top-k is compared where it is unique (tie band at the k-th proxy score) on the member that
receives all of it; every other member must hold exactly its part inside the member's prefix,
with the same scores bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection
from test_gpu_variants import run_group, check_group

pytestmark = pytest.mark.gpu


def run_reuse(prob, k, G):
    t = dev(prob)
    oi, osc = idx.group_proxy_reuse(t["q"], t["k"], t["w"], t["q_pos"], topk=k, group_size=G,
                                    k_len=t["k_len"], k_scale=t["k_scale"])
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy()


def check_reuse(prob, k, G, gi, gs, name, groups=None):
    inp = oracle.Inputs(prob)
    NG = (prob.T + G - 1) // G
    if groups is None:
        groups = [(b, g) for b in range(prob.B) for g in range(NG)]
    for b, g in groups:
        mem = list(oracle.group_members(prob.T, G, g))
        ps = oracle.group_proxy_scan(inp, b, g, G, k)
        far = max(mem, key=lambda t: prob.q_pos[b, t])
        check_selection(gi[b, far], gs[b, far], np.arange(ps["P"]), ps["proxy_scores"],
                        ps["proxy_magnitude"], k, prob.D, ctx=f"{name} b{b} g{g} t{far}",
                        oracle_sel=ps["cand"])
        top = gi[b, far][gi[b, far] >= 0]
        sc = dict(zip(top.tolist(), gs[b, far][gi[b, far] >= 0].view(np.uint32).tolist()))
        for t in mem:
            sel = gi[b, t][gi[b, t] >= 0]
            want = top[top < inp.P(b, t)]
            assert set(sel.tolist()) == set(want.tolist()), f"{name} b{b} t{t}"
            assert len(sel) == len(want) and (gi[b, t, len(sel):] == -1).all()
            got = gs[b, t][: len(sel)].view(np.uint32).tolist()
            assert got == [sc[v] for v in sel.tolist()], f"{name} b{b} t{t} scores"
            assert np.isneginf(gs[b, t, len(sel):]).all()


def test_reuse_singletons_equal_dense():
    p = W.make_prefill(300, 64, 128, seed=51)
    k = 40
    say("case reuse G=1: L=300 H=64 D=128 k=40 (must equal the dense indexer)")
    gi, gs = run_reuse(p, k, 1)
    inp = oracle.Inputs(p)
    for t in range(p.T):
        r = oracle.dense_row(inp, 0, t, k)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"], k,
                        p.D, ctx=f"reuse-1 t{t}", oracle_sel=r["ids"])


def test_reuse_prefill_groups_and_ragged_batch():
    p = W.make_prefill(700, 64, 128, seed=52, B=2, rho=0.95)
    p.k_len[1] = 500
    say("case reuse G=16: B=2 L=700 (k_len 500 for b1) k=48")
    gi, gs = run_reuse(p, 48, 16)
    check_reuse(p, 48, 16, gi, gs, "reuse-16")


def test_decode_grouping_fp8_both_variants():
    p = W.make_decode(3, 6000, T=2, seed=53, k_len=[6000, 4321, 100])
    G, k, C = 2, 256, 1024
    say("case decode grouping: B=3 N=6000 T=2 fp8, G=T=2; reuse k=256, refine C=1024")
    gi, gs = run_reuse(p, k, G)
    check_reuse(p, k, G, gi, gs, "decode-reuse")
    ri, rs, rc = run_group(p, k, G, C)
    check_group(p, k, G, C, ri, rs, rc, [(b, 0) for b in range(p.B)], "decode-refine")


def test_reuse_long_proxy_rows_and_ties():
    # ten proxies over prefixes of up to 40000 keys: too few rows for one work-group per row
    # range, so the proxy rows come without a summary and take the long-row selector; one group
    # has all-zero head weights (every proxy score 0: ties keep the lowest tokens)
    p = W.make_prefill(40000, 8, 64, seed=54)
    G, k = 4096, 2048
    p.w[0, 2 * G:3 * G] = 0.0
    say("case reuse long proxy rows: L=40000 H=8 D=64 G=4096 k=2048, one all-zero group")
    gi, gs = run_reuse(p, k, G)
    check_reuse(p, k, G, gi, gs, "reuse-long")
    far = 3 * G - 1
    assert set(gi[0, far].tolist()) == set(range(k)), "ties: lowest tokens"


@pytest.mark.timeout(900)
def test_reuse64k_full_size_sampled_groups():
    # the benchmarked shape: L=65536, H=64, D=128, groups of 16, k=2048; the proxies' prefix
    # scans over up to 65536 keys and the member rows of sampled groups across the prefill
    spec = W.WORKLOADS["reuse64k"]
    p = spec["gen"](0)
    G, k = spec["group_size"], spec["k"]
    say("case reuse64k full size (L=65536, H=64, D=128, G=16, k=2048)")
    gi, gs = run_reuse(p, k, G)
    rng = np.random.default_rng(4)
    groups = sorted(set([0, 127, 128, 2047, 4095] + list(rng.integers(0, 4096, 4))))
    check_reuse(p, k, G, gi, gs, "reuse64k", groups=[(0, g) for g in groups])


@pytest.mark.timeout(900)
def test_decode_grouping_full_size_sampled_sequences():
    # the benchmarked decode-grouping shapes: 32 sequences of 131072 FP8 keys, the 2 MTP queries of
    # a step form one group (the proxies' scan is the decode scan); both variants
    rs, gs_ = W.WORKLOADS["decodereuse128k"], W.WORKLOADS["decodegroup128k"]
    p = rs["gen"](0)
    G, k, C = rs["group_size"], rs["k"], gs_["n_cand"]
    assert gs_["group_size"] == G and gs_["k"] == k
    say("case decodereuse128k / decodegroup128k full size (B=32, N=131072, T=2, G=2, k=2048, C=8192)")
    gi, gsc = run_reuse(p, k, G)
    seqs = [0, 9, 31]
    check_reuse(p, k, G, gi, gsc, "decodereuse128k", groups=[(b, 0) for b in seqs])
    ri, rsc, rc = run_group(p, k, G, C)
    check_group(p, k, G, C, ri, rsc, rc, [(b, 0) for b in seqs], "decodegroup128k")
    assert ((ri >= 0).sum(-1) == k).all()
