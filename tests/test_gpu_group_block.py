"""GPU parity of the block-filtered group proxy (idx_group_block_refine) against the oracle: each
group's kept blocks against the oracle's pooled-block scores of the proxy (tie band at the
n_keep-th score), and every member row against the oracle's token scores over the tokens of the
GPU's kept blocks; keeping every block must reproduce the dense indexer."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection
from block_checks import check_gb

pytestmark = pytest.mark.gpu


def run_gb(prob, k, G, Bs, keep):
    t = dev(prob)
    oi, osc, blk = idx.group_block_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k, group_size=G,
                                          block_size=Bs, n_blocks_keep=keep, k_len=t["k_len"],
                                          return_blocks=True)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy(), blk.cpu().numpy()


def test_group_block_small_ragged_batch():
    p = W.make_prefill(600, 16, 64, seed=61, B=2)
    p.k_len[1] = 450
    G, Bs, keep, k = 8, 16, 6, 40
    say("case group-block: B=2 L=600 (k_len 450) G=8 Bs=16 keep=6 k=40")
    gi, gs, gb = run_gb(p, k, G, Bs, keep)
    NG = gb.shape[1]
    check_gb(p, k, G, Bs, keep, gi, gs, gb, [(b, g) for b in range(2) for g in range(NG)], "gb-small")


def test_group_block_hier_shape():
    p = W.make_hier(8192, 512, seed=62, n_regions=16)
    G, Bs, keep, k = 16, 64, 16, 256
    say("case group-block: N=8192, 512 queries at the end, G=16 Bs=64 keep=16 k=256")
    gi, gs, gb = run_gb(p, k, G, Bs, keep)
    check_gb(p, k, G, Bs, keep, gi, gs, gb, [(0, g) for g in (0, 7, 19, 31)], "gb-hier")


def test_group_block_keep_all_is_dense():
    p = W.make_prefill(300, 32, 128, seed=63)
    k = 48
    say("case group-block keeping every block (must equal dense)")
    gi, gs, _ = run_gb(p, k, 5, 8, 1000)
    inp = oracle.Inputs(p)
    for t in range(p.T):
        r = oracle.dense_row(inp, 0, t, k)
        check_selection(gi[0, t], gs[0, t], r["universe"], r["all_scores"], r["magnitude"], k, p.D,
                        ctx=f"gb-all t{t}", oracle_sel=r["ids"])


@pytest.mark.timeout(900)
def test_gblock128k_full_size_sampled_groups():
    # the benchmarked shape: 4096 queries at the end of a 131072-token context, groups of 16,
    # 128-token blocks, 128 kept blocks, so each member refines rows of 16384 list slots
    spec = W.WORKLOADS["gblock128k"]
    p = spec["gen"](0)
    G, Bs, keep, k = spec["group_size"], spec["block_size"], spec["n_blocks_keep"], spec["k"]
    say("case gblock128k full size (N=131072, 4096 queries, G=16, Bs=128, keep=128, k=2048)")
    gi, gs, gb = run_gb(p, k, G, Bs, keep)
    rng = np.random.default_rng(3)
    groups = sorted(set([0, 1, 128, 255] + list(rng.integers(0, 256, 4))))
    check_gb(p, k, G, Bs, keep, gi, gs, gb, [(0, g) for g in groups], "gblock128k")
    assert ((gi[0] >= 0).sum(-1) == k).all()
