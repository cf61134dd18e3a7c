"""GPU parity of the dense indexer (idx_score_topk) against the oracle: prefill and decode
shapes, every dtype combination, ragged and degenerate cases, and the full-size workloads on
sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection

pytestmark = pytest.mark.gpu


def run_dense(prob, k, **kw):
    t = dev(prob)
    oi, osc = idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"],
                             k_scale=t["k_scale"], **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy()


def check_rows(prob, k, gi, gs, rows, name):
    inp = oracle.Inputs(prob)
    flips = 0
    for b, t in rows:
        r = oracle.dense_row(inp, b, t, k)
        flips += check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"],
                                 r["magnitude"], k, prob.D, ctx=f"{name} b{b} t{t}",
                                 oracle_sel=r["ids"])
    return flips


def all_rows(prob):
    return [(b, t) for b in range(prob.B) for t in range(prob.T)]


def test_tiny_fp32_all_rows():
    p = W.make_tiny(0)
    say("case tiny fp32 L=1024 H=4 D=32 k=64")
    gi, gs = run_dense(p, 64)
    check_rows(p, 64, gi, gs, all_rows(p), "tiny")


def test_bf16_prefill_ragged():
    p = W.make_prefill(1000, 64, 128, seed=1)          # 1000: not a multiple of 8 or 64
    say("case bf16 prefill L=1000 H=64 D=128 k=128")
    gi, gs = run_dense(p, 128)
    check_rows(p, 128, gi, gs, all_rows(p), "bf16-1000")


@pytest.mark.parametrize("H,D", [(4, 32), (16, 64), (48, 64), (64, 32), (100, 128), (128, 128),
                                 (1, 128)])
def test_head_and_dim_shapes(H, D):
    p = W.make_prefill(300, H, D, seed=H + D)
    say(f"case shapes H={H} D={D}")
    gi, gs = run_dense(p, 40)
    check_rows(p, 40, gi, gs, all_rows(p), f"H{H}D{D}")


@pytest.mark.parametrize("qd,kd", [(W.F32, W.BF16), (W.BF16, W.F32), (W.F32, W.FP8_E4M3),
                                   (W.BF16, W.FP8_E4M3), (W.F32, W.F32)])
def test_dtype_combinations(qd, kd):
    p = W.make_prefill(260, 8, 64, seed=5, q_dtype=qd, k_dtype=kd)
    say(f"case dtypes q={qd} k={kd}")
    gi, gs = run_dense(p, 50)
    check_rows(p, 50, gi, gs, all_rows(p), f"q{qd}k{kd}")


def test_decode_fp8_ragged_lengths():
    p = W.make_decode(3, 5000, T=2, seed=3, k_len=[5000, 4321, 100])
    say("case decode fp8 B=3 N=5000 ragged k_len")
    gi, gs = run_dense(p, 2048)
    check_rows(p, 2048, gi, gs, all_rows(p), "decode-small")


def test_decode_bf16_four_mtp_queries():
    p = W.make_decode(2, 3000, T=4, seed=4, k_dtype=W.BF16)
    say("case decode bf16 B=2 N=3000 T=4")
    gi, gs = run_dense(p, 512)
    check_rows(p, 512, gi, gs, all_rows(p), "decode-bf16")


def test_degenerate_cases():
    p = W.make_prefill(70, 64, 128, seed=9, B=2)
    p.q_pos[0, :5] = -1                      # empty prefixes
    p.q_pos[0, 5:9] = 0                      # only token 0
    p.q_pos[1, 60:] = 1000                   # beyond the cache: clamped to k_len
    p.k_len[1] = 64
    p.w[0, 20:30] *= -1.0                    # negative head weights
    p.w[1, 30:35] = 0.0                      # all-zero weights: every score 0 (ties)
    say("case degenerate: empty prefixes, clamps, negative and zero weights, k > N")
    gi, gs = run_dense(p, 100)               # k larger than every prefix
    check_rows(p, 100, gi, gs, all_rows(p), "degenerate")
    assert (gi[0, :5] == -1).all()
    assert (gi[1, 30:35, :31] >= 0).all()


def test_empty_tiles_write_padding():
    # whole 8-query tiles with empty prefixes (q_pos < 0, and a sequence with an empty cache): the
    # self-selecting score kernel must still write -1 / -inf rows over a pre-filled sentinel
    p = W.make_prefill(96, 64, 128, seed=41, B=2)
    p.q_pos[0, :16] = -1
    p.k_len[1] = 0
    k = 64
    say("case empty tiles: q_pos[0,:16] = -1, k_len[1] = 0, bf16 self-selecting path")
    t = dev(p)
    oi = torch.full((2, 96, k), 12345, dtype=torch.int32, device="cuda")
    osc = torch.full((2, 96, k), 7.0, dtype=torch.float32, device="cuda")
    idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"], out_idx=oi,
                   out_score=osc)
    torch.cuda.synchronize()
    gi, gs = oi.cpu().numpy(), osc.cpu().numpy()
    assert (gi[0, :16] == -1).all() and np.isneginf(gs[0, :16]).all()
    assert (gi[1] == -1).all() and np.isneginf(gs[1]).all()
    check_rows(p, k, gi, gs, [(0, t_) for t_ in range(16, 96)], "empty-tiles")


def test_exact_ties_keep_lowest_slots():
    p = W.make_prefill(1500, 64, 128, seed=21)
    p.k[0, 300:] = np.tile(p.k[0, :100], (12, 1))    # key 300 + 100 j + i repeats key i: equal scores
    p.w[0, 1200:1210] = 0.0                          # rows whose every score is 0
    k = 300
    say("case exact ties: repeated keys and all-zero rows, L=1500 H=64 D=128 k=300")
    gi, gs = run_dense(p, k)
    check_rows(p, k, gi, gs, [(0, t) for t in list(range(280, 1500, 37)) + list(range(1200, 1210))], "ties")
    for t in range(1200, 1210):                      # all scores 0: the k lowest tokens
        assert set(gi[0, t].tolist()) == set(range(k)), f"ties t{t}"
    for t in range(400, 1500):                       # a kept copy implies every lower copy is kept
        sel = set(gi[0, t][gi[0, t] >= 0].tolist())
        for s in sel:
            if s >= 300:
                lower = (s - 300) % 100 if s < 400 else s - 100
                assert lower in sel, f"ties t{t}: token {s} kept but its lower copy {lower} not"


def test_long_rows_wide_boundary_bin():
    # D=64: the boundary bin of these rows holds more slots than the selector keeps in LDS, so
    # they are compacted into the score row; the all-zero rows also tie at the k-th key
    p = W.make_prefill(24000, 8, 64, seed=31)
    p.w[0, 22000:22003] = 0.0
    k = 2048
    say("case long rows: L=24000 H=8 D=64 k=2048, three all-zero rows")
    gi, gs = run_dense(p, k)
    check_rows(p, k, gi, gs, [(0, t) for t in (2047, 2048, 9000, 17001, 22000, 22002, 23999)], "long")
    for t in range(22000, 22003):
        assert set(gi[0, t].tolist()) == set(range(k)), f"long t{t}"


def test_stream_selector_long_boundary_bin_and_ties():
    # fp32 queries: the separate stream selector; rows of all-zero scores longer than its
    # candidate buffer re-read the row for each digit and keep the lowest slots of the tie
    p = W.make_prefill(5000, 8, 64, seed=33, q_dtype=W.F32)
    p.w[0, 4000:4003] = 0.0
    k = 300
    say("case stream selector: L=5000 fp32 queries, k=300, three all-zero rows")
    gi, gs = run_dense(p, k)
    check_rows(p, k, gi, gs, [(0, t) for t in (299, 300, 2500, 4000, 4002, 4999)], "stream-long")
    for t in range(4000, 4003):
        assert set(gi[0, t].tolist()) == set(range(k)), f"stream-long t{t}"


def test_deterministic():
    p = W.make_prefill(600, 64, 128, seed=12)
    say("case determinism")
    a = run_dense(p, 256)
    b = run_dense(p, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.timeout(900)
def test_dense16k_full_size_sampled_rows():
    spec = W.WORKLOADS["dense16k"]
    p = spec["gen"](0)
    say("case dense16k full size (L=16384, H=64, D=128, k=2048)")
    gi, gs = run_dense(p, spec["k"])
    # 128 rows spread over the causal triangle (one per 128-row stratum, at varying offsets in
    # the 8-query tile) plus the tile and k boundaries
    rng = np.random.default_rng(0)
    ts = sorted(set([0, 1, 7, 8, 2046, 2047, 2048, 2049, 8191, 8192, 16383] +
                    [128 * j + int(rng.integers(0, 128)) for j in range(128)]))
    flips = check_rows(p, spec["k"], gi, gs, [(0, t) for t in ts], "dense16k")
    say(f"dense16k: {len(ts)} rows checked, {flips} tie-band swaps")
    # structure of every row: count = min(k, t+1), ascending, causal
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(spec["k"], np.arange(16384) + 1))
    assert (gi[0].max(-1) <= np.arange(16384)).all()


@pytest.mark.timeout(1200)
def test_dense64k_full_size_sampled_rows():
    # rows of up to 65536 keys, selected by the score kernel's own waves (12-bit first digits,
    # boundary bins beyond the LDS copy compacted into the score row); the rows are scored in
    # chunks of 4096 queries, so both sides of every chunk boundary are checked
    spec = W.WORKLOADS["dense64k"]
    p = spec["gen"](0)
    say("case dense64k full size (L=65536, H=64, D=128, k=2048)")
    gi, gs = run_dense(p, spec["k"])
    rng = np.random.default_rng(1)
    ts = sorted(set([0, 2047, 2048, 32767, 65535] + [4096 * j + d for j in range(1, 16) for d in (-1, 0)] +
                    list(rng.integers(0, 65536, 7))))
    flips = check_rows(p, spec["k"], gi, gs, [(0, t) for t in ts], "dense64k")
    say(f"dense64k: {len(ts)} rows checked, {flips} tie-band swaps")
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(spec["k"], np.arange(65536) + 1))
    assert (gi[0].max(-1) <= np.arange(65536)).all()


@pytest.mark.timeout(600)
def test_rows_of_65536_slots_with_equal_scores():
    # the last tile's rows have all-zero head weights, so every score is 0: row 65535 puts all
    # 65536 slots into one bin of the 16-bit-half histogram (slot 65535 is counted outside it),
    # and the selection keeps the 2048 lowest slots of the tie; D=64 keeps fewer boundary slots in
    # LDS, so the other long rows take the compacted-row path
    p = W.make_prefill(65536, 8, 64, seed=61)
    p.w[0, 65528:] = 0.0
    k = 2048
    say("case rows of 65536 slots: L=65536 H=8 D=64 k=2048, last tile all-zero weights")
    gi, gs = run_dense(p, k)
    for t in range(65528, 65536):
        assert set(gi[0, t].tolist()) == set(range(k)), f"equal-65536 t{t}"
        assert (gs[0, t] == 0).all()
    check_rows(p, k, gi, gs, [(0, t) for t in (2047, 4095, 4096, 40000, 65000, 65527, 65535)], "rows-65536")


@pytest.mark.timeout(900)
def test_decode128k_full_size_sampled_rows():
    spec = W.WORKLOADS["decode128k"]
    p = spec["gen"](0)
    say("case decode128k full size (B=32, N=131072, T=2, fp8 keys, k=2048)")
    gi, gs = run_dense(p, spec["k"])
    rows = [(b, t) for b in (0, 7, 31) for t in (0, 1)]
    flips = check_rows(p, spec["k"], gi, gs, rows, "decode128k")
    say(f"decode128k: {len(rows)} rows checked, {flips} tie-band swaps")
    assert ((gi >= 0).sum(-1) == spec["k"]).all()
