"""GPU check of the allocation-free dense entry point (idx_score_topk_noalloc, whose scratch is
the library's static device array) against idx_score_topk with a caller workspace: identical
index sets and bit-identical scores, on consecutive calls of decreasing size (the static array
keeps the previous call's contents), for a prefill long enough to be chunked over the scratch and
for a decode-shaped call."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _both(prob, k):
    t = dev(prob)
    ref_i, ref_s = idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"],
                                  k_scale=t["k_scale"])
    B, T = prob.B, prob.T
    oi = torch.full((B, T, k), 777, dtype=torch.int32, device="cuda")
    osc = torch.full((B, T, k), 3.0, dtype=torch.float32, device="cuda")
    p = idx.make_problem(t["q"], t["k"], t["w"], t["q_pos"], t["k_len"], t["k_scale"])
    st = idx.lib().idx_score_topk_noalloc(ctypes.byref(p), k, oi.data_ptr(), osc.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 0, idx.lib().idx_strerror(st).decode()
    torch.cuda.synchronize()
    return ref_i.cpu().numpy(), ref_s.cpu().numpy(), oi.cpu().numpy(), osc.cpu().numpy()


def _same_rows(ri, rs, gi, gs, name):
    """Rows are sets: compare (index, score bits) sorted by index, padding included."""
    B, T, k = ri.shape
    for b in range(B):
        oa = np.argsort(ri[b], axis=-1, kind="stable")
        ob = np.argsort(gi[b], axis=-1, kind="stable")
        ia, ib = np.take_along_axis(ri[b], oa, -1), np.take_along_axis(gi[b], ob, -1)
        sa = np.take_along_axis(rs[b], oa, -1).view(np.uint32)
        sb = np.take_along_axis(gs[b], ob, -1).view(np.uint32)
        bad = np.nonzero((ia != ib).any(-1) | (sa != sb).any(-1))[0]
        assert len(bad) == 0, f"{name}: {len(bad)} rows differ, first b{b} t{bad[0]}"


def test_noalloc_matches_workspace_entry_point():
    # 1) a prefill whose score rows (20000 x 80 KB) exceed the 256 MiB scratch: chunked
    p1 = W.make_prefill(20000, 64, 128, seed=51)
    p1.q_pos[0, :9] = -1                              # a tile of empty prefixes
    say("case noalloc 1: prefill L=20000 H=64 D=128 k=2048 (chunked over the static scratch)")
    ri, rs, gi, gs = _both(p1, 2048)
    _same_rows(ri, rs, gi, gs, "noalloc-prefill-20000")
    # 2) a smaller prefill right after it: the scratch still holds the first call's rows
    p2 = W.make_prefill(700, 32, 64, seed=52, B=2)
    p2.k_len[1] = 500
    say("case noalloc 2: prefill B=2 L=700 H=32 D=64 k=300")
    ri, rs, gi, gs = _both(p2, 300)
    _same_rows(ri, rs, gi, gs, "noalloc-prefill-700")
    # 3) decode-shaped, then 4) a smaller decode
    p3 = W.make_decode(8, 40000, T=2, seed=53, k_len=[40000, 39000, 12345, 40000, 2048, 30000, 7, 40000])
    say("case noalloc 3: decode fp8 B=8 N=40000 T=2 k=2048")
    ri, rs, gi, gs = _both(p3, 2048)
    _same_rows(ri, rs, gi, gs, "noalloc-decode-40000")
    p4 = W.make_decode(3, 5000, T=2, seed=54)
    say("case noalloc 4: decode fp8 B=3 N=5000 T=2 k=1024")
    ri, rs, gi, gs = _both(p4, 1024)
    _same_rows(ri, rs, gi, gs, "noalloc-decode-5000")


def test_noalloc_rejects_problems_beyond_the_scratch():
    # a decode batch needing more than 256 MiB of candidate lists is refused before any launch
    p = idx.Problem(64, 4, 64, 128, 131072, idx.BF16, idx.FP8_E4M3, 0x10000, 0x20000, 0x30000,
                    0x40000, 0x50000, None)
    assert idx.lib().idx_score_topk_noalloc(ctypes.byref(p), 2048, 0x60000, None, None) == -4
