"""GPU parity of the block filter on FP8 key caches and at decode shapes (a few queries per
sequence, where the kept tokens are refined as per-query lists): the pooled block keys bit for
bit against the oracle's, the kept blocks and final rows against the oracle, the caller-pooled
entry points against the ones that pool inside the call (identical outputs), and the full-size
decode workloads on sampled sequences."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from block_checks import check_block, check_gb
from gpu_util import dev, say
from parity import check_selection

pytestmark = pytest.mark.gpu


def run_block(prob, k, Bs, keep, pooled=None):
    t = dev(prob)
    pk = None if pooled is None else pooled(t)
    oi, osc, blk = idx.block_coarse_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k, block_size=Bs,
                                           n_blocks_keep=keep, k_len=t["k_len"], k_scale=t["k_scale"],
                                           return_blocks=True, pooled=pk)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy(), blk.cpu().numpy()


def run_gb(prob, k, G, Bs, keep, pooled=None):
    t = dev(prob)
    pk = None if pooled is None else pooled(t)
    oi, osc, blk = idx.group_block_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k, group_size=G,
                                          block_size=Bs, n_blocks_keep=keep, k_len=t["k_len"],
                                          k_scale=t["k_scale"], return_blocks=True, pooled=pk)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy(), blk.cpu().numpy()


def pool_of(Bs):
    return lambda t: idx.block_pool(t["k"], Bs, k_len=t["k_len"], k_scale=t["k_scale"])


def assert_same_selection(x, y, name):
    """Equal outputs up to the order inside each row (the decode selector emits a row's picks in
    no fixed order): the same tokens with the same scores, and the same kept blocks."""
    (xi, xs, xb), (yi, ys, yb) = x, y
    ox, oy = np.argsort(xi, axis=-1, kind="stable"), np.argsort(yi, axis=-1, kind="stable")
    assert np.array_equal(np.take_along_axis(xi, ox, -1), np.take_along_axis(yi, oy, -1)), f"{name} idx"
    assert np.array_equal(np.take_along_axis(xs, ox, -1), np.take_along_axis(ys, oy, -1)), f"{name} score"
    assert np.array_equal(xb, yb), f"{name} blocks"


@pytest.mark.parametrize("k_dtype", [W.FP8_E4M3, W.BF16, W.F32])
@pytest.mark.parametrize("D,Bs", [(128, 64), (64, 7), (32, 128)])
def test_block_pool_bits_match_oracle(k_dtype, D, Bs):
    p = W.make_decode(3, 1000, 2, H=8, D=D, seed=D + Bs, k_dtype=k_dtype, k_len=[1000, 613, 1])
    say(f"case block_pool k_dtype={W.DTYPE_NAMES[k_dtype]} D={D} Bs={Bs} ragged k_len")
    t = dev(p)
    got = idx.block_pool(t["k"], Bs, k_len=t["k_len"], k_scale=t["k_scale"])
    torch.cuda.synchronize()
    g = got.view(torch.int16).cpu().numpy().view(np.uint16) if got.dtype == torch.bfloat16 else \
        got.cpu().numpy()
    for b in range(p.B):
        ref = oracle.pool_keys(p, b, Bs)
        nb = ref.shape[0]
        assert np.array_equal(g[b, :nb], ref), f"pooled b{b}"
        assert (g[b, nb:] == 0).all(), f"blocks past k_len b{b}"


def test_fp8_block_prefill_all_rows():
    p = W.make_prefill(900, 32, 128, seed=81, k_dtype=W.FP8_E4M3, B=2)
    p.k_len[1] = 700
    say("case fp8 block prefill B=2 L=900 (k_len 700) Bs=32 keep=6 k=64")
    gi, gs, gb = run_block(p, 64, 32, 6)
    check_block(p, 64, 32, 6, gi, gs, gb, [(b, t) for b in range(2) for t in range(p.T)], "fp8-block")


@pytest.mark.parametrize("k_dtype", [W.FP8_E4M3, W.BF16])
def test_block_decode_shape_all_rows(k_dtype):
    p = W.make_decode(6, 6000, 2, seed=82, k_dtype=k_dtype, n_regions=6, region=64,
                      k_len=[6000, 5000, 4097, 129, 2, 64])
    say(f"case block decode B=6 N=6000 T=2 {W.DTYPE_NAMES[k_dtype]} Bs=64 keep=12 k=256")
    gi, gs, gb = run_block(p, 256, 64, 12)
    check_block(p, 256, 64, 12, gi, gs, gb, [(b, t) for b in range(p.B) for t in range(p.T)],
                f"block-decode-{W.DTYPE_NAMES[k_dtype]}")


def test_fp8_block_decode_keep_all_is_dense():
    p = W.make_decode(3, 3000, 3, seed=83, k_len=[3000, 1111, 40])
    say("case fp8 block decode keeping every block (must equal dense)")
    gi, gs, _ = run_block(p, 512, 32, 10 ** 4)
    inp = oracle.Inputs(p)
    for b in range(p.B):
        for t in range(p.T):
            r = oracle.dense_row(inp, b, t, 512)
            check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"], 512,
                            p.D, ctx=f"fp8 keep-all b{b} t{t}", oracle_sel=r["ids"])


@pytest.mark.parametrize("G", [2, 3])
def test_fp8_group_block_decode(G):
    p = W.make_decode(5, 5000, 3, seed=84 + G, n_regions=6, region=64, k_len=[5000, 3000, 2049, 300, 3])
    say(f"case fp8 group-block decode B=5 N=5000 T=3 G={G} Bs=64 keep=10 k=200")
    gi, gs, gb = run_gb(p, 200, G, 64, 10)
    check_gb(p, 200, G, 64, 10, gi, gs, gb, [(b, g) for b in range(p.B) for g in range(gb.shape[1])],
             f"fp8-gb-G{G}")


def test_fp8_group_block_prefill():
    p = W.make_prefill(600, 16, 64, seed=86, k_dtype=W.FP8_E4M3, B=2)
    p.k_len[1] = 450
    say("case fp8 group-block prefill B=2 L=600 (k_len 450) G=8 Bs=16 keep=6 k=40")
    gi, gs, gb = run_gb(p, 40, 8, 16, 6)
    check_gb(p, 40, 8, 16, 6, gi, gs, gb, [(b, g) for b in range(2) for g in range(gb.shape[1])], "fp8-gb")


@pytest.mark.parametrize("k_dtype", [W.FP8_E4M3, W.BF16])
def test_pooled_entry_points_equal_internal_pooling(k_dtype):
    p = W.make_decode(4, 4000, 2, seed=87, k_dtype=k_dtype, n_regions=4, region=64, k_len=[4000, 2500, 700, 65])
    say(f"case pooled entry points vs internal pooling, {W.DTYPE_NAMES[k_dtype]}")
    assert_same_selection(run_block(p, 128, 64, 8), run_block(p, 128, 64, 8, pooled=pool_of(64)), "block")
    assert_same_selection(run_gb(p, 128, 2, 64, 8), run_gb(p, 128, 2, 64, 8, pooled=pool_of(64)), "group-block")


def test_pooled_prefill_union_route_equal_internal_pooling():
    # many query tiles per sequence: the union refine kernel, with the pooled keys passed in
    p = W.make_hier(3000, 600, seed=88, n_regions=8, region=64)
    say("case pooled entry point on a prefill chunk (union refine route)")
    assert_same_selection(run_block(p, 128, 64, 8), run_block(p, 128, 64, 8, pooled=pool_of(64)), "block")


def _full_size(name, rows_of):
    spec = W.WORKLOADS[name]
    p = spec["gen"](0)
    Bs, keep, k = spec["block_size"], spec["n_blocks_keep"], spec["k"]
    if spec["op"] == "block":
        gi, gs, gb = run_block(p, k, Bs, keep, pooled=pool_of(Bs))
        check_block(p, k, Bs, keep, gi, gs, gb, rows_of(p), name)
    else:
        G = spec["group_size"]
        gi, gs, gb = run_gb(p, k, G, Bs, keep, pooled=pool_of(Bs))
        check_gb(p, k, G, Bs, keep, gi, gs, gb, [(b, 0) for b, _ in rows_of(p)], name)
    assert ((gi >= 0).sum(-1) == k).all()


@pytest.mark.timeout(900)
def test_decodeblk128k_full_size_sampled_sequences():
    say("case decodeblk128k full size (B=32, N=131072, T=2, fp8, Bs=128, keep=128, k=2048)")
    _full_size("decodeblk128k", lambda p: [(b, t) for b in (0, 13, 31) for t in range(p.T)])


@pytest.mark.timeout(900)
def test_decodegblk128k_full_size_sampled_sequences():
    say("case decodegblk128k full size (B=32, N=131072, T=2 sharing the filter, fp8, Bs=128, keep=128)")
    _full_size("decodegblk128k", lambda p: [(b, 0) for b in (0, 17, 31)])
