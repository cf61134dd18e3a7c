"""Host-side checks of the C ABI (no GPU): the library loads, exports every function that
include/idx.h declares, and rejects bad arguments before enqueueing anything. The pointers
used here are never dereferenced: every call below fails validation first."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_02_amd as idx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(idx.LIB_PATH):
        from sparse_attention_indexer_02_amd import build
        build.build()
    return idx.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_0-9]+\s*\*?\s*(idx_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    f = declared_functions()
    for name in ("idx_score_topk", "idx_group_proxy_refine", "idx_block_coarse_refine",
                 "idx_workspace_bytes", "idx_strerror"):
        assert name in f
    assert sorted(idx.EXPORTS) == f


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror(L):
    for code in range(0, -7, -1):
        assert L.idx_strerror(code)
    assert L.idx_strerror(-99) == b"unknown status"


def _problem(**kw):
    base = dict(B=1, T=64, H=64, D=128, N=64, q_dtype=idx.BF16, k_dtype=idx.BF16,
                q=0x10000, k=0x20000, k_scale=None, w=0x30000, q_pos=0x40000, k_len=None,
                q_scale=None)
    base.update(kw)
    return idx.Problem(**base)


def _call(L, p, k=8, out=0x50000, ws=0x60000, ws_bytes=1 << 40):
    return L.idx_score_topk(ctypes.byref(p) if p is not None else None, k, out, None, ws,
                            ws_bytes, None)


def test_workspace_bytes(L):
    p = _problem()
    n = L.idx_workspace_bytes(idx.OP_SCORE_TOPK, ctypes.byref(p), 8, 0, 0)
    assert n >= 64 * 64 * 4
    assert L.idx_workspace_bytes(idx.OP_GROUP, ctypes.byref(p), 8, 4, 16) > 0
    assert L.idx_workspace_bytes(idx.OP_BLOCK, ctypes.byref(p), 8, 16, 2) > 0
    assert L.idx_workspace_bytes(idx.OP_GROUP, ctypes.byref(p), 8, 0, 16) == 0
    assert L.idx_workspace_bytes(99, ctypes.byref(p), 8, 0, 0) == 0
    assert L.idx_workspace_bytes(idx.OP_SCORE_TOPK, None, 8, 0, 0) == 0
    bad = _problem(T=0)
    assert L.idx_workspace_bytes(idx.OP_SCORE_TOPK, ctypes.byref(bad), 8, 0, 0) == 0


def test_invalid_arguments(L):
    assert _call(L, None) == -1
    assert _call(L, _problem(), k=0) == -1
    assert _call(L, _problem(B=0)) == -1
    assert _call(L, _problem(q=None)) == -1
    assert _call(L, _problem(), out=None) == -1
    assert _call(L, _problem(k_dtype=idx.FP8_E4M3)) == -1          # fp8 needs k_scale


def test_unsupported_shapes(L):
    assert _call(L, _problem(D=48)) == -2
    assert _call(L, _problem(H=129)) == -2
    # FP8 queries: need q_scale, FP8 keys and D >= 64, and only the dense entry points take them
    assert _call(L, _problem(q_dtype=idx.FP8_E4M3)) == -1
    assert _call(L, _problem(q_dtype=idx.FP8_E4M3, q_scale=0x70000)) == -2
    assert _call(L, _problem(q_dtype=idx.FP8_E4M3, q_scale=0x70000, k_dtype=idx.FP8_E4M3,
                             k_scale=0x78000, D=32)) == -2
    assert _call(L, _problem(q_dtype=idx.FP8_E4M3, q_scale=0x70002, k_dtype=idx.FP8_E4M3,
                             k_scale=0x78000)) == -3
    p8 = _problem(q_dtype=idx.FP8_E4M3, q_scale=0x70000, k_dtype=idx.FP8_E4M3, k_scale=0x78000)
    assert L.idx_group_proxy_refine(ctypes.byref(p8), 8, 4, 16, 0x50000, None, None, 0x60000,
                                    1 << 40, None) == -2
    assert L.idx_group_proxy_reuse(ctypes.byref(p8), 8, 4, 0x50000, None, 0x60000, 1 << 40, None) == -2
    assert _call(L, _problem(k_dtype=7)) == -2


def test_misaligned(L):
    assert _call(L, _problem(q=0x10002)) == -3
    assert _call(L, _problem(k=0x20008)) == -3
    assert _call(L, _problem(q_pos=0x40002)) == -3


def test_workspace_too_small(L):
    assert _call(L, _problem(), ws_bytes=100) == -4
    assert _call(L, _problem(), ws=None) == -4


def test_variant_arguments(L):
    p = _problem()
    g = lambda G, C: L.idx_group_proxy_refine(ctypes.byref(p), 8, G, C, 0x50000, None, None,
                                              0x60000, 1 << 40, None)
    assert g(0, 16) == -1 and g(4, 0) == -1
    # more candidates than the cache holds is valid: a proxy keeps at most its prefix, so the
    # workspace is that of n_cand = N (the GPU test shows the result equals the dense indexer's)
    gs = lambda G, C, ws_bytes: L.idx_group_proxy_refine(ctypes.byref(p), 8, G, C, 0x50000, None,
                                                         None, 0x60000, ws_bytes, None)
    assert gs(4, 2 * p.N, 100) == -4
    assert L.idx_workspace_bytes(idx.OP_GROUP, ctypes.byref(p), 8, 4, 2 * p.N) == \
        L.idx_workspace_bytes(idx.OP_GROUP, ctypes.byref(p), 8, 4, p.N) > 0
    b = lambda Bs, keep, pp=p: L.idx_block_coarse_refine(ctypes.byref(pp), 8, Bs, keep, 0x50000,
                                                         None, None, 0x60000, 1 << 40, None)
    assert b(0, 4) == -1 and b(16, 0) == -1
    assert b(16, 40000) == -2
    assert b(16, 4, _problem(k_dtype=idx.FP8_E4M3)) == -1           # fp8 keys need k_scale


def test_pooled_arguments(L):
    p = _problem()
    bp = lambda Bs, pooled, pp=p: L.idx_block_pool(ctypes.byref(pp), Bs, pooled, None)
    assert bp(16, None) == -1 and bp(0, 0x70000) == -1
    assert bp(16, 0x70008) == -3                                     # pooled not 16-byte aligned
    assert bp(16, 0x70000, pp=_problem(D=48)) == -2
    assert bp(16, 0x70000, pp=_problem(k_dtype=idx.FP8_E4M3)) == -1  # fp8 keys need k_scale
    bc = lambda pooled, ws_bytes=1 << 40: L.idx_block_coarse_refine_pooled(
        ctypes.byref(p), 8, 16, 4, pooled, 0x50000, None, None, 0x60000, ws_bytes, None)
    assert bc(None) == -1 and bc(0x70008) == -3 and bc(0x70000, ws_bytes=100) == -4
    gc = lambda pooled, ws_bytes=1 << 40: L.idx_group_block_refine_pooled(
        ctypes.byref(p), 8, 4, 16, 4, pooled, 0x50000, None, None, 0x60000, ws_bytes, None)
    assert gc(None) == -1 and gc(0x70008) == -3 and gc(0x70000, ws_bytes=100) == -4


def test_refine_given_arguments(L):
    p = _problem()
    r = lambda G, cand, C, pp=p, ws_bytes=1 << 40: L.idx_refine_given(
        ctypes.byref(pp), 8, G, cand, None, C, 0x50000, None, 0x60000, ws_bytes, None)
    assert r(0, 0x70000, 16) == -1 and r(4, None, 16) == -1 and r(4, 0x70000, 0) == -1
    assert r(4, 0x70002, 16) == -3                                   # candidates not 4-aligned
    assert r(4, 0x70000, 16, pp=_problem(N=1048577)) == -2           # set bitmap beyond LDS
    assert r(4, 0x70000, 16, ws_bytes=100) == -4
    assert L.idx_workspace_bytes(idx.OP_REFINE, ctypes.byref(p), 8, 4, 16) > 0
    assert L.idx_workspace_bytes(idx.OP_REFINE, ctypes.byref(p), 8, 4, 0) == 0


def test_reuse_arguments(L):
    p = _problem()
    u = lambda G, ws_bytes=1 << 40: L.idx_group_proxy_reuse(ctypes.byref(p), 8, G, 0x50000, None,
                                                            0x60000, ws_bytes, None)
    assert u(0) == -1 and u(4, ws_bytes=100) == -4
    assert L.idx_workspace_bytes(idx.OP_REUSE, ctypes.byref(p), 8, 4, 0) > 0
    assert L.idx_workspace_bytes(idx.OP_REUSE, ctypes.byref(p), 8, 0, 0) == 0


def test_group_block_arguments(L):
    p = _problem()
    gb = lambda G, Bs, keep, pp=p, ws_bytes=1 << 40: L.idx_group_block_refine(
        ctypes.byref(pp), 8, G, Bs, keep, 0x50000, None, None, 0x60000, ws_bytes, None)
    assert gb(0, 16, 4) == -1 and gb(4, 0, 4) == -1 and gb(4, 16, 0) == -1
    assert gb(4, 16, 40000) == -2
    assert gb(4, 16, 4, pp=_problem(k_dtype=idx.FP8_E4M3)) == -1     # fp8 keys need k_scale
    assert gb(4, 16, 4, ws_bytes=100) == -4
    assert L.idx_group_block_workspace_bytes(ctypes.byref(p), 8, 4, 16, 4) > 0
    assert L.idx_group_block_workspace_bytes(ctypes.byref(p), 8, 0, 16, 4) == 0


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 2, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 32, dtype=torch.bfloat16)
    w = torch.zeros(1, 4, 2)
    pos = torch.zeros(1, 4, dtype=torch.int32)
    with pytest.raises(idx.IdxError):
        idx.make_problem(q, k, w, pos)
    with pytest.raises(idx.IdxError):
        idx.make_problem(q, k[:, :, :16], w, pos)


def test_absorb_arguments(L):
    a = lambda q=0x10000, rows=4, H=2, D=128, wk=0x20000, Dc=64, out=0x30000: L.idx_absorb_queries(
        q, rows, H, D, wk, Dc, out, None)
    assert a(q=None) == -1 and a(wk=None) == -1 and a(out=None) == -1
    assert a(rows=0) == -1 and a(H=0) == -1
    assert a(D=96) == -2 and a(Dc=16) == -2
    assert a(q=0x10008) == -3 and a(wk=0x20002) == -3 and a(out=0x30004) == -3
