"""Python binding of libidx.so, the MI355X DeepSeek-Sparse-Attention lightning indexer.

Argument marshalling only: every step of the indexer runs in the library's HIP kernels. Tensors
must be on the GPU; the library is loaded from this package directory and its absence is an
error (there is no other implementation to fall back to).

    idx, score = score_topk(q, k, w, q_pos, topk=2048)
    idx, score, cand = group_proxy_refine(q, k, w, q_pos, topk=2048, group_size=16, n_cand=8192)
    idx, score, blocks = block_coarse_refine(q, k, w, q_pos, topk=2048, block_size=128,
                                             n_blocks_keep=128)
    idx, score = refine_given(q, k, w, q_pos, cand, cand_cnt=None, topk=2048, group_size=1)
    idx, score = group_proxy_reuse(q, k, w, q_pos, topk=2048, group_size=16)
    idx, score, blocks = group_block_refine(q, k, w, q_pos, topk=2048, group_size=16,
                                            block_size=128, n_blocks_keep=128)

Shapes: q [B,T,H,D] (bf16 or fp32; float8_e4m3fn / uint8 E4M3FN bytes with q_scale [B,T,H] fp32
for score_topk), k [B,N,D] (bf16, fp32, or float8_e4m3fn / uint8 E4M3FN
bytes with k_scale [B,N] fp32), w [B,T,H] fp32, q_pos [B,T] int32, k_len [B] int32 or None.
Outputs: int32 [B,T,topk] token-index sets (order within a row unspecified, -1 padded) and the
matching fp32 scores (-inf padded).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["F32", "BF16", "FP8_E4M3", "IdxError", "lib", "score_topk", "score_topk_noalloc",
           "group_proxy_refine",
           "block_coarse_refine", "refine_given", "group_proxy_reuse", "group_block_refine", "block_pool", "absorb_queries",
           "workspace_bytes", "timer_enable", "timer_read", "EXPORTS"]

F32, BF16, FP8_E4M3 = 0, 1, 2
OP_SCORE_TOPK, OP_GROUP, OP_BLOCK, OP_REFINE, OP_REUSE = 0, 1, 2, 3, 4
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidx.so")
EXPORTS = ["idx_score_topk", "idx_score_topk_noalloc", "idx_group_proxy_refine", "idx_block_coarse_refine",
           "idx_refine_given", "idx_group_proxy_reuse", "idx_group_block_refine",
           "idx_group_block_workspace_bytes", "idx_workspace_bytes", "idx_strerror", "idx_timer_enable",
           "idx_timer_read", "idx_block_pool", "idx_block_coarse_refine_pooled", "idx_group_block_refine_pooled",
           "idx_absorb_queries"]


class IdxError(RuntimeError):
    pass


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("N", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("k_dtype", ctypes.c_int32), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("w", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
                ("k_len", ctypes.c_void_p), ("q_scale", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises IdxError if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise IdxError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_attention_indexer_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.idx_score_topk.argtypes = [P, i32, vp, vp, vp, sz, vp]
        L.idx_score_topk_noalloc.argtypes = [P, i32, vp, vp, vp]
        L.idx_group_proxy_refine.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.idx_block_coarse_refine.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.idx_refine_given.argtypes = [P, i32, i32, vp, vp, i32, vp, vp, vp, sz, vp]
        L.idx_group_proxy_reuse.argtypes = [P, i32, i32, vp, vp, vp, sz, vp]
        L.idx_group_block_refine.argtypes = [P, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.idx_block_pool.argtypes = [P, i32, vp, vp]
        L.idx_absorb_queries.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp]
        L.idx_block_coarse_refine_pooled.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.idx_group_block_refine_pooled.argtypes = [P, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.idx_group_block_workspace_bytes.argtypes = [P, i32, i32, i32, i32]
        L.idx_group_block_workspace_bytes.restype = sz
        L.idx_workspace_bytes.argtypes = [ctypes.c_int, P, i32, i32, i32]
        L.idx_workspace_bytes.restype = sz
        L.idx_strerror.argtypes = [ctypes.c_int]
        L.idx_strerror.restype = ctypes.c_char_p
        L.idx_timer_enable.argtypes = [ctypes.c_int]
        L.idx_timer_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int32)]
        for f in ("idx_score_topk", "idx_score_topk_noalloc", "idx_group_proxy_refine", "idx_block_coarse_refine",
                  "idx_refine_given", "idx_group_proxy_reuse", "idx_group_block_refine",
                  "idx_timer_enable", "idx_timer_read", "idx_block_pool",
                  "idx_block_coarse_refine_pooled", "idx_group_block_refine_pooled",
                  "idx_absorb_queries"):
            getattr(L, f).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        raise IdxError(f"{what}: {lib().idx_strerror(status).decode()} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise IdxError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise IdxError("tensors must be contiguous")
    return t.data_ptr()


def _qcode(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    raise IdxError(f"unsupported query dtype {t.dtype}")


def _kcode(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    raise IdxError(f"unsupported key dtype {t.dtype}")


def make_problem(q, k, w, q_pos, k_len=None, k_scale=None, q_scale=None) -> Problem:
    """Fill the ABI's problem struct from tensors (shape checks only). FP8 queries (float8_e4m3fn
    or uint8 E4M3FN bytes) need q_scale float32 [B,T,H]."""
    if q.dim() != 4 or k.dim() != 3 or w.dim() != 3 or q_pos.dim() != 2:
        raise IdxError("expected q [B,T,H,D], k [B,N,D], w [B,T,H], q_pos [B,T]")
    B, T, H, D = q.shape
    N = k.shape[1]
    if k.shape[0] != B or k.shape[2] != D or tuple(w.shape) != (B, T, H) or \
            tuple(q_pos.shape) != (B, T):
        raise IdxError("inconsistent shapes")
    if w.dtype != torch.float32 or q_pos.dtype != torch.int32:
        raise IdxError("w must be float32 and q_pos int32")
    if k_len is not None and (k_len.dtype != torch.int32 or tuple(k_len.shape) != (B,)):
        raise IdxError("k_len must be int32 [B]")
    kc = _kcode(k)
    if kc == FP8_E4M3 and (k_scale is None or k_scale.dtype != torch.float32 or
                           tuple(k_scale.shape) != (B, N)):
        raise IdxError("fp8 keys need k_scale float32 [B,N]")
    qc = _qcode(q)
    if qc == FP8_E4M3 and (q_scale is None or q_scale.dtype != torch.float32 or
                           tuple(q_scale.shape) != (B, T, H)):
        raise IdxError("fp8 queries need q_scale float32 [B,T,H]")
    return Problem(B, T, H, D, N, qc, kc, _ptr(q), _ptr(k),
                   _ptr(k_scale) if kc == FP8_E4M3 else None, _ptr(w), _ptr(q_pos), _ptr(k_len),
                   _ptr(q_scale) if qc == FP8_E4M3 else None)


def workspace_bytes(op: int, p: Problem, topk: int, p1: int = 0, p2: int = 0) -> int:
    return int(lib().idx_workspace_bytes(op, ctypes.byref(p), topk, p1, p2))


def _stream(t, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _outputs(q, topk, out_idx, out_score, want_score):
    B, T = q.shape[:2]
    if out_idx is None:
        out_idx = torch.empty((B, T, topk), dtype=torch.int32, device=q.device)
    if out_score is None and want_score:
        out_score = torch.empty((B, T, topk), dtype=torch.float32, device=q.device)
    return out_idx, out_score


def _workspace(q, need, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < need:
            raise IdxError("workspace too small")
        return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)


def score_topk(q, k, w, q_pos, topk: int = 2048, k_len=None, k_scale=None, out_idx=None,
               out_score=None, want_score: bool = True, workspace=None, stream=None, q_scale=None):
    """Dense lightning indexer (idx_score_topk)."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale, q_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    need = workspace_bytes(OP_SCORE_TOPK, p, topk)
    ws = _workspace(q, need, workspace)
    _check(lib().idx_score_topk(ctypes.byref(p), topk, _ptr(out_idx), _ptr(out_score),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(q, stream)),
           "idx_score_topk")
    return out_idx, out_score


def score_topk_noalloc(q, k, w, q_pos, topk: int = 2048, k_len=None, k_scale=None, out_idx=None,
                       out_score=None, stream=None, q_scale=None):
    """Dense lightning indexer on the library's static scratch (idx_score_topk_noalloc): the
    outputs must be passed in for an allocation-free call."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale, q_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, True)
    _check(lib().idx_score_topk_noalloc(ctypes.byref(p), topk, _ptr(out_idx), _ptr(out_score),
                                        _stream(q, stream)),
           "idx_score_topk_noalloc")
    return out_idx, out_score


def group_proxy_refine(q, k, w, q_pos, topk: int = 2048, group_size: int = 16,
                       n_cand: int = 8192, k_len=None, k_scale=None, out_idx=None,
                       out_score=None, want_score: bool = True, return_cand: bool = False,
                       workspace=None, stream=None):
    """Group-shared proxy scan + per-query refine (idx_group_proxy_refine)."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    cand = None
    if return_cand:
        NG = (q.shape[1] + group_size - 1) // group_size
        cand = torch.empty((q.shape[0], NG, n_cand), dtype=torch.int32, device=q.device)
    need = workspace_bytes(OP_GROUP, p, topk, group_size, n_cand)
    ws = _workspace(q, need, workspace)
    _check(lib().idx_group_proxy_refine(ctypes.byref(p), topk, group_size, n_cand, _ptr(out_idx),
                                        _ptr(out_score), _ptr(cand), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(q, stream)),
           "idx_group_proxy_refine")
    return out_idx, out_score, cand


def group_proxy_reuse(q, k, w, q_pos, topk: int = 2048, group_size: int = 16, k_len=None,
                      k_scale=None, out_idx=None, out_score=None, want_score: bool = True,
                      workspace=None, stream=None):
    """Group-shared scan without refine, PIVOT-Reuse (idx_group_proxy_reuse)."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    need = workspace_bytes(OP_REUSE, p, topk, group_size, 0)
    ws = _workspace(q, need, workspace)
    _check(lib().idx_group_proxy_reuse(ctypes.byref(p), topk, group_size, _ptr(out_idx),
                                       _ptr(out_score), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(q, stream)),
           "idx_group_proxy_reuse")
    return out_idx, out_score


def pooled_shape(k, block_size):
    """Shape and dtype of the pooled block keys of a key cache k [B,N,D]."""
    B, N, D = k.shape
    return (B, (N + block_size - 1) // block_size, D), (torch.float32 if k.dtype == torch.float32 else torch.bfloat16)


def block_pool(k, block_size: int = 128, k_len=None, k_scale=None, out=None, stream=None):
    """Pooled block keys of the whole cache (idx_block_pool): bf16 [B, ceil(N/Bs), D] for bf16 and
    FP8 keys, fp32 for fp32 keys."""
    B, N, D = k.shape
    kc = _kcode(k)
    if kc == FP8_E4M3 and (k_scale is None or k_scale.dtype != torch.float32):
        raise IdxError("fp8 keys need k_scale float32 [B,N]")
    shape, dt = pooled_shape(k, block_size)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=k.device)
    p = Problem(B, 1, 1, D, N, BF16, kc, None, _ptr(k), _ptr(k_scale) if kc == FP8_E4M3 else None, None,
                None, _ptr(k_len), None)
    _check(lib().idx_block_pool(ctypes.byref(p), block_size, _ptr(out), _stream(k, stream)), "idx_block_pool")
    return out


def absorb_queries(q, wk, out=None, stream=None):
    """Absorbed queries of a layer scoring a shared latent cache (idx_absorb_queries): bf16
    q [B,T,H,D] and key decoder wk [Dc,D] -> bf16 [B,T,H,Dc]."""
    if q.dim() != 4 or wk.dim() != 2 or wk.shape[1] != q.shape[3]:
        raise IdxError("expected q [B,T,H,D] and wk [Dc,D]")
    if q.dtype != torch.bfloat16 or wk.dtype != torch.bfloat16:
        raise IdxError("absorb_queries takes bf16 queries and decoder")
    B, T, H, D = q.shape
    Dc = wk.shape[0]
    if out is None:
        out = torch.empty((B, T, H, Dc), dtype=torch.bfloat16, device=q.device)
    _check(lib().idx_absorb_queries(_ptr(q), B * T, H, D, _ptr(wk), Dc, _ptr(out), _stream(q, stream)),
           "idx_absorb_queries")
    return out


def group_block_refine(q, k, w, q_pos, topk: int = 2048, group_size: int = 16,
                       block_size: int = 128, n_blocks_keep: int = 128, k_len=None, k_scale=None,
                       out_idx=None, out_score=None, want_score: bool = True,
                       return_blocks: bool = False, workspace=None, stream=None, pooled=None):
    """Block-filtered group proxy with per-query refine (idx_group_block_refine, or
    idx_group_block_refine_pooled when the pooled keys are given)."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = None
    if return_blocks:
        NG = (q.shape[1] + group_size - 1) // group_size
        blocks = torch.empty((q.shape[0], NG, n_blocks_keep), dtype=torch.int32, device=q.device)
    need = int(lib().idx_group_block_workspace_bytes(ctypes.byref(p), topk, group_size, block_size,
                                                     n_blocks_keep))
    ws = _workspace(q, need, workspace)
    if pooled is None:
        _check(lib().idx_group_block_refine(ctypes.byref(p), topk, group_size, block_size, n_blocks_keep,
                                            _ptr(out_idx), _ptr(out_score), _ptr(blocks), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(q, stream)),
               "idx_group_block_refine")
    else:
        _check(lib().idx_group_block_refine_pooled(ctypes.byref(p), topk, group_size, block_size,
                                                   n_blocks_keep, _ptr(pooled), _ptr(out_idx),
                                                   _ptr(out_score), _ptr(blocks), _ptr(ws),
                                                   ws.numel() * ws.element_size(), _stream(q, stream)),
               "idx_group_block_refine_pooled")
    return out_idx, out_score, blocks


def refine_given(q, k, w, q_pos, cand, cand_cnt=None, topk: int = 2048, group_size: int = 1,
                 k_len=None, k_scale=None, out_idx=None, out_score=None, want_score: bool = True,
                 workspace=None, stream=None):
    """Per-query refine over caller-supplied candidate sets (idx_refine_given).
    cand: int32 [B, ceil(T/group_size), n_cand] token ids; cand_cnt: int32 [B, ceil(T/group_size)]
    or None (all n_cand entries read). Values outside [0, k_len[b]) are dropped, repeats count
    once."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale)
    NG = (q.shape[1] + group_size - 1) // group_size
    if cand.dtype != torch.int32 or cand.dim() != 3 or tuple(cand.shape[:2]) != (q.shape[0], NG):
        raise IdxError(f"cand must be int32 [B, {NG}, n_cand]")
    if cand_cnt is not None and (cand_cnt.dtype != torch.int32 or tuple(cand_cnt.shape) != (q.shape[0], NG)):
        raise IdxError(f"cand_cnt must be int32 [B, {NG}]")
    cand = cand.contiguous()
    cand_cnt = cand_cnt.contiguous() if cand_cnt is not None else None
    C = cand.shape[2]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    need = workspace_bytes(OP_REFINE, p, topk, group_size, C)
    ws = _workspace(q, need, workspace)
    _check(lib().idx_refine_given(ctypes.byref(p), topk, group_size, _ptr(cand), _ptr(cand_cnt), C,
                                  _ptr(out_idx), _ptr(out_score), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(q, stream)),
           "idx_refine_given")
    return out_idx, out_score


def block_coarse_refine(q, k, w, q_pos, topk: int = 2048, block_size: int = 128,
                        n_blocks_keep: int = 128, k_len=None, out_idx=None, out_score=None,
                        want_score: bool = True, return_blocks: bool = False, workspace=None,
                        stream=None, k_scale=None, pooled=None):
    """Block-pooled coarse filter + token refine (idx_block_coarse_refine, or
    idx_block_coarse_refine_pooled when the pooled keys are given)."""
    p = make_problem(q, k, w, q_pos, k_len, k_scale)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = None
    if return_blocks:
        blocks = torch.empty((q.shape[0], q.shape[1], n_blocks_keep), dtype=torch.int32,
                             device=q.device)
    need = workspace_bytes(OP_BLOCK, p, topk, block_size, n_blocks_keep)
    ws = _workspace(q, need, workspace)
    if pooled is None:
        _check(lib().idx_block_coarse_refine(ctypes.byref(p), topk, block_size, n_blocks_keep,
                                             _ptr(out_idx), _ptr(out_score), _ptr(blocks), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(q, stream)),
               "idx_block_coarse_refine")
    else:
        _check(lib().idx_block_coarse_refine_pooled(ctypes.byref(p), topk, block_size, n_blocks_keep,
                                                    _ptr(pooled), _ptr(out_idx), _ptr(out_score),
                                                    _ptr(blocks), _ptr(ws), ws.numel() * ws.element_size(),
                                                    _stream(q, stream)),
               "idx_block_coarse_refine_pooled")
    return out_idx, out_score, blocks


def timer_enable(on: bool = True):
    _check(lib().idx_timer_enable(1 if on else 0), "idx_timer_enable")


def timer_read(kernel_substr: str = ""):
    """(total milliseconds, launches) of the recorded kernels whose name contains the text."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int32(0)
    _check(lib().idx_timer_read(kernel_substr.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "idx_timer_read")
    return ms.value, n.value
