"""CPU oracle for the DSA lightning indexer and its two accelerated variants.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import this module. It shares no code with the HIP library (sparse_attention_indexer_02_amd)
and imports nothing from it; the only module both sides use is `workloads` (seeded inputs).

Plain numpy, float64 for every real-valued quantity the method defines as a real number, so
that its results are the mathematical definitions up to fp64 rounding. Two steps are defined by
this implementation as rounding steps in fp32 (the proxy query and the pooled block key, both of
which are themselves indexer inputs stored in the query/key format); they are written as plain
fp32 operations in a stated order.

Sources (web pages, cited by title and section):
  [DSA]   the DeepSeek Sparse Attention lightning indexer that all five pages build on. Its score
          for query t and key s is I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]). The pages name
          its multiple indexer heads ("PIVOT: Efficient Query-Group Indexing ...", related-papers
          list, MISA entry) and say it keeps the k = 2048 best-scoring tokens per query
          ("Multi-layer Indexer ...", authors' abstract); none of them prints the formula.
  [PIVOT] "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention", abstract:
          consecutive queries form fixed-size groups; each group is reduced to one proxy query;
          the proxy's single scan of the prefix yields a candidate set; in the Refine variant
          every query then scores those candidates with its own indexer and picks its top-k.
  [HISA]  "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse Attention", abstract:
          blocks of keys are pooled and scored to drop unpromising regions, then the unchanged
          token-level indexer runs only over the tokens of the blocks that were kept.
  [LatentIndex] "LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for Sparse
          Attention", abstract: a group of layers shares one latent cache, and each layer scores
          it directly by absorbing its key decoder into its queries instead of rebuilding its
          own keys.

Parity status: every function below is pinned by tests/test_oracle_*.py (hand-computed cases,
library special cases, invariants, reductions and, for the absorbed queries, the identity with
scoring rebuilt keys). Recall of the group and block variants
against the dense indexer has no published value and is reported, not pinned.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

F32, BF16, FP8_E4M3 = 0, 1, 2


# ----------------------------------------------------------------------------------------------
# number formats (written from the format definitions, not from any library)

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 = the upper 16 bits of an IEEE binary32; decoding is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is subnormal
    (m * 2^-9); S.1111.111 is NaN; there is no infinity (max finite 448)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round binary32 to bfloat16, nearest-even, NaN kept quiet."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint64)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def f64_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round binary64 straight to bfloat16 (8 significant bits), nearest-even, in one step (no
    intermediate fp32 rounding). Finite inputs within bf16's range; subnormals keep the fixed
    2^-133 spacing."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)                                 # |x| = m * 2^e, 0.5 <= m < 1
    ue = np.maximum(e - 8, -133).astype(np.float64)    # exponent of the bf16 unit in the last place
    r = np.rint(np.ldexp(x, (-ue).astype(np.int32))) * np.exp2(ue)   # rint: ties to even
    return f32_to_bf16_bits_rne(r.astype(np.float32))  # r is exact in bf16, so this is a re-encoding


def queries_f64(q: np.ndarray, q_dtype: int, q_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Real query values. FP8 queries carry one fp32 scale per (query, head), the same
    per-vector quantisation as the FP8 key cache: query = decode(byte) * scale (exact in fp64)."""
    if q_dtype == F32:
        return np.asarray(q, np.float32).astype(np.float64)
    if q_dtype == BF16:
        return bf16_bits_to_f64(q)
    if q_dtype == FP8_E4M3:
        return e4m3fn_bits_to_f64(q) * np.asarray(q_scale, np.float32).astype(np.float64)[..., None]
    raise ValueError("query dtype must be F32, BF16 or FP8_E4M3")


def keys_f64(k: np.ndarray, k_dtype: int, k_scale: Optional[np.ndarray]) -> np.ndarray:
    """Real key values. FP8 keys carry one fp32 scale per token: key = decode(byte) * scale
    (exact in fp64)."""
    if k_dtype == F32:
        return np.asarray(k, np.float32).astype(np.float64)
    if k_dtype == BF16:
        return bf16_bits_to_f64(k)
    if k_dtype == FP8_E4M3:
        return e4m3fn_bits_to_f64(k) * np.asarray(k_scale, np.float32).astype(np.float64)[..., None]
    raise ValueError("unknown key dtype")


# ----------------------------------------------------------------------------------------------
# the indexer score and the top-k selection  [DSA]

def index_scores(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """I[s] = sum_h w[h] * max(q[h] . k[s], 0) for every row s of `keys` ([DSA]).

    q_t [H,D], w_t [H], keys [S,D], all float64. Returns [S] float64."""
    x = keys @ q_t.T                      # [S,H] dot products
    return np.maximum(x, 0.0) @ w_t       # ReLU, then the head-weighted sum


def score_magnitude(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """A[s] = sum_h |w[h]| * sum_d |q[h,d] * k[s,d]|: the scale of the rounding error that any
    fp32 evaluation of index_scores can make (a standard a-priori dot-product bound uses it)."""
    return (np.abs(keys) @ np.abs(q_t).T) @ np.abs(w_t)


def select_topk(scores: np.ndarray, ids: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """The min(k, len) highest scores; equal scores prefer the lower token index (a full stable
    sort on (-score, id)). Returns (ids, scores) in that order. The indexer keeps the k best
    tokens of each query ("Multi-layer Indexer ...", authors' abstract)."""
    order = np.lexsort((ids, -scores))[: max(0, min(k, len(ids)))]
    return ids[order], scores[order]


def visible_len(q_pos: int, k_len: int) -> int:
    """Causal prefix length: keys s <= q_pos that exist in the cache (s < k_len). Only the
    query's causal prefix is scored ("ADIndex ...", abstract; "PIVOT ...", abstract). Reading:
    the prefix includes the query's own token, whose key is already cached when it is scored."""
    return max(0, min(int(q_pos) + 1, int(k_len)))


class Inputs:
    """Float64 views of one Problem (see workloads.Problem for the storage layout)."""

    def __init__(self, prob):
        self.prob = prob
        self.q = queries_f64(prob.q, prob.q_dtype, getattr(prob, "q_scale", None))   # [B,T,H,D]
        self.w = np.asarray(prob.w, np.float32).astype(np.float64)
        self._keys: Dict[int, np.ndarray] = {}

    def keys(self, b: int) -> np.ndarray:
        if b not in self._keys:
            p = self.prob
            sc = None if p.k_scale is None else p.k_scale[b]
            self._keys[b] = keys_f64(p.k[b], p.k_dtype, sc)
        return self._keys[b]

    def P(self, b: int, t: int) -> int:
        return visible_len(self.prob.q_pos[b, t], self.prob.k_len[b])


# ----------------------------------------------------------------------------------------------
# dense indexer  [DSA]

def dense_row(inp: Inputs, b: int, t: int, k: int):
    """One query row of the dense indexer: scores over the whole causal prefix, then the top-k.

    Returns dict(ids, scores) for the selection plus the full prefix scores and magnitudes."""
    P = inp.P(b, t)
    keys = inp.keys(b)[:P]
    s = index_scores(inp.q[b, t], inp.w[b, t], keys)
    ids = np.arange(P, dtype=np.int64)
    sel, sc = select_topk(s, ids, k)
    return dict(ids=sel, scores=sc, universe=ids, all_scores=s,
                magnitude=score_magnitude(inp.q[b, t], inp.w[b, t], keys))


def dense(prob, k: int):
    """Full dense indexer output: out_idx [B,T,k] int32 padded with -1, out_score float64
    padded with -inf, each row in selection order."""
    inp = Inputs(prob)
    B, T = prob.q_pos.shape
    out_idx = np.full((B, T, k), -1, np.int32)
    out_sc = np.full((B, T, k), -np.inf)
    for b in range(B):
        for t in range(T):
            r = dense_row(inp, b, t, k)
            n = len(r["ids"])
            out_idx[b, t, :n] = r["ids"]
            out_sc[b, t, :n] = r["scores"]
    return out_idx, out_sc


# ----------------------------------------------------------------------------------------------
# group-shared scan with per-query refine  [PIVOT]

def group_members(T: int, G: int, g: int) -> range:
    """Fixed-size groups of consecutive queries; the last group may be shorter ([PIVOT])."""
    return range(g * G, min(g * G + G, T))


def proxy_query(prob, b: int, g: int, G: int):
    """One proxy query per group ([PIVOT]; the page says only that the group is aggregated).
    Reading: the element-wise mean of the members' queries and of their head weights.
    The proxy is an indexer query, so it is stored in the query format: the mean is taken in
    fp32 (sum in ascending t starting from +0, then one fp32 division by the member count) and
    rounded to bf16 (nearest-even) for bf16 queries. Its position is the last member's, i.e.
    the largest member position, so its scan covers every member's prefix.

    Returns (q_bits_or_f32 [H,D], w [H] float32, pos int)."""
    mem = group_members(prob.T, G, g)
    if prob.q_dtype == FP8_E4M3:
        raise ValueError("proxy queries are defined for bf16 and fp32 queries")
    if prob.q_dtype == BF16:
        qf = (np.asarray(prob.q[b, mem.start:mem.stop], np.uint16).astype(np.uint32)
              << np.uint32(16)).view(np.float32)
    else:
        qf = np.asarray(prob.q[b, mem.start:mem.stop], np.float32)
    wf = np.asarray(prob.w[b, mem.start:mem.stop], np.float32)
    qs = np.zeros(qf.shape[1:], np.float32)
    ws = np.zeros(wf.shape[1:], np.float32)
    for i in range(len(mem)):              # ascending member order, fp32 adds
        qs = (qs + qf[i]).astype(np.float32)
        ws = (ws + wf[i]).astype(np.float32)
    n = np.float32(len(mem))
    qm = (qs / n).astype(np.float32)
    wm = (ws / n).astype(np.float32)
    qout = f32_to_bf16_bits_rne(qm) if prob.q_dtype == BF16 else qm
    pos = int(np.max(prob.q_pos[b, mem.start:mem.stop]))
    return qout, wm, pos


def group_proxy_scan(inp: Inputs, b: int, g: int, G: int, n_cand: int):
    """The proxy's one scan over its whole prefix and the candidate set it yields ([PIVOT]):
    the min(n_cand, P) best-scoring keys of the proxy's prefix. Returns dict(cand sorted
    ascending, proxy scores over the prefix, ...)."""
    prob = inp.prob
    qb, wb, pos = proxy_query(prob, b, g, G)
    q64 = queries_f64(qb, prob.q_dtype)
    w64 = wb.astype(np.float64)
    P = visible_len(pos, prob.k_len[b])
    keys = inp.keys(b)[:P]
    s = index_scores(q64, w64, keys)
    ids = np.arange(P, dtype=np.int64)
    cand, csc = select_topk(s, ids, n_cand)
    return dict(cand=np.sort(cand), cand_by_rank=cand, proxy_scores=s,
                proxy_magnitude=score_magnitude(q64, w64, keys), P=P, n_cand=len(cand),
                proxy_q=qb, proxy_w=wb, proxy_pos=pos)


def refine_row(inp: Inputs, b: int, t: int, k: int, candidates: np.ndarray):
    """Score a candidate token set with query t's own indexer and keep its top-k (the Refine
    step of [PIVOT]; the token-level stage of [HISA], which runs the unchanged indexer only over
    the kept blocks' tokens). Candidates outside t's causal prefix are dropped first."""
    P = inp.P(b, t)
    v = np.asarray(candidates, np.int64)
    v = np.sort(v[(v >= 0) & (v < P)])
    keys = inp.keys(b)[v]
    s = index_scores(inp.q[b, t], inp.w[b, t], keys)
    sel, sc = select_topk(s, v, k)
    return dict(ids=sel, scores=sc, universe=v, all_scores=s,
                magnitude=score_magnitude(inp.q[b, t], inp.w[b, t], keys))


def group(prob, k: int, G: int, n_cand: int):
    """Full PIVOT-Refine output: (out_idx [B,T,k], out_score, cand dict {(b,g): sorted ids})."""
    inp = Inputs(prob)
    B, T = prob.q_pos.shape
    NG = (T + G - 1) // G
    out_idx = np.full((B, T, k), -1, np.int32)
    out_sc = np.full((B, T, k), -np.inf)
    cands = {}
    for b in range(B):
        for g in range(NG):
            ps = group_proxy_scan(inp, b, g, G, n_cand)
            cands[(b, g)] = ps["cand"]
            for t in group_members(T, G, g):
                r = refine_row(inp, b, t, k, ps["cand"])
                n = len(r["ids"])
                out_idx[b, t, :n] = r["ids"]
                out_sc[b, t, :n] = r["scores"]
    return out_idx, out_sc, cands


def reuse_row(inp: Inputs, b: int, t: int, ps):
    """PIVOT-Reuse ([PIVOT]: the proxy's top-k is shared across the group, nothing is re-scored).
    `ps` is group_proxy_scan with n_cand = k, so its candidates are the proxy's top-k. Reading:
    a member keeps the proxy's top-k tokens that lie in its own causal prefix (an earlier member
    sees a shorter prefix than the proxy), each with the proxy's score. Returns dict(ids, scores)
    in the proxy's rank order."""
    P = inp.P(b, t)
    ids = np.asarray(ps["cand_by_rank"], np.int64)
    keep = ids < P
    return dict(ids=ids[keep], scores=ps["proxy_scores"][ids[keep]])


def group_reuse(prob, k: int, G: int):
    """Full PIVOT-Reuse output: (out_idx [B,T,k] int32 -1 padded, out_score -inf padded, proxy
    scans {(b,g): group_proxy_scan(..., n_cand=k)})."""
    inp = Inputs(prob)
    B, T = prob.q_pos.shape
    NG = (T + G - 1) // G
    out_idx = np.full((B, T, k), -1, np.int32)
    out_sc = np.full((B, T, k), -np.inf)
    scans = {}
    for b in range(B):
        for g in range(NG):
            ps = group_proxy_scan(inp, b, g, G, k)
            scans[(b, g)] = ps
            for t in group_members(T, G, g):
                r = reuse_row(inp, b, t, ps)
                n = len(r["ids"])
                out_idx[b, t, :n] = r["ids"]
                out_sc[b, t, :n] = r["scores"]
    return out_idx, out_sc, scans


# ----------------------------------------------------------------------------------------------
# block-pooled coarse filter with token refine  [HISA]

def pool_keys(prob, b: int, block_size: int) -> np.ndarray:
    """Pooled block keys ([HISA] scores pooled representations of key blocks; it does not say
    which pooling). Reading: the mean of the keys of each block of `block_size` consecutive tokens, over the tokens that
    exist in the cache (the last block may be partial). Like the proxy query it is an indexer
    input stored in a key format: fp32 sum in ascending token order from +0, one fp32
    division by the token count, nearest-even to bf16 for bf16 and FP8 keys (fp32 keys stay
    fp32). An FP8 key enters the sum as its fp32 value decode(byte) * scale (one fp32 multiply).
    Returns the pooled keys in storage form [NB,D]."""
    L = int(prob.k_len[b])
    if prob.k_dtype == BF16:
        kf = (np.asarray(prob.k[b, :L], np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif prob.k_dtype == FP8_E4M3:
        kf = (e4m3fn_bits_to_f64(prob.k[b, :L]).astype(np.float32) *
              np.asarray(prob.k_scale[b, :L], np.float32)[:, None]).astype(np.float32)
    else:
        kf = np.asarray(prob.k[b, :L], np.float32)
    NB = (L + block_size - 1) // block_size
    nfull = L // block_size
    out = np.zeros((NB, prob.D), np.float32)
    full = kf[: nfull * block_size].reshape(nfull, block_size, prob.D)
    acc = np.zeros((nfull, prob.D), np.float32)
    for i in range(block_size):           # ascending token order inside every full block
        acc = (acc + full[:, i]).astype(np.float32)
    out[:nfull] = (acc / np.float32(block_size)).astype(np.float32)
    if NB > nfull:                        # the partial last block
        acc1 = np.zeros(prob.D, np.float32)
        for s in range(nfull * block_size, L):
            acc1 = (acc1 + kf[s]).astype(np.float32)
        out[nfull] = (acc1 / np.float32(L - nfull * block_size)).astype(np.float32)
    return out if prob.k_dtype == F32 else f32_to_bf16_bits_rne(out)


def block_row(inp: Inputs, b: int, t: int, k: int, block_size: int, n_keep: int,
              pooled: np.ndarray):
    """One query of the hierarchical indexer ([HISA]): (1) score every pooled block whose first
    token is in the query's causal prefix, keep the min(n_keep, eligible) best blocks; (2) run
    the original indexer over the tokens of the kept blocks (causal prefix only) and take the
    top-k. Returns the kept blocks (ascending), their scores, and the refine result."""
    prob = inp.prob
    pk = pooled.astype(np.float64) if prob.k_dtype == F32 else bf16_bits_to_f64(pooled)
    NB = pk.shape[0]
    qp = int(prob.q_pos[b, t])
    n_elig = 0 if qp < 0 else min(NB, qp // block_size + 1)
    bs = index_scores(inp.q[b, t], inp.w[b, t], pk[:n_elig])
    bids = np.arange(n_elig, dtype=np.int64)
    kept, _ = select_topk(bs, bids, n_keep)
    kept = np.sort(kept)
    toks = (kept[:, None] * block_size + np.arange(block_size)[None]).reshape(-1)
    r = refine_row(inp, b, t, k, toks)
    r.update(blocks=kept, block_scores=bs,
             block_magnitude=score_magnitude(inp.q[b, t], inp.w[b, t], pk[:n_elig]))
    return r


def group_block_scan(inp: Inputs, b: int, g: int, G: int, block_size: int, n_keep: int,
                     pooled: np.ndarray):
    """The block-filtered proxy (PIVOT's group proxy ([PIVOT]) scoring HISA's pooled blocks
    ([HISA]) instead of every token of its prefix). Reading: the proxy of proxy_query scores the
    pooled blocks whose first token is in its prefix and keeps the min(n_keep, eligible) best
    (ties to the lower block); the group's candidates are the tokens of the kept blocks.
    Returns dict(blocks ascending, block_scores, block_magnitude, tokens ascending)."""
    prob = inp.prob
    qb, wb, pos = proxy_query(prob, b, g, G)
    q64 = queries_f64(qb, prob.q_dtype)
    w64 = wb.astype(np.float64)
    pk = pooled.astype(np.float64) if prob.k_dtype == F32 else bf16_bits_to_f64(pooled)
    NB = pk.shape[0]
    n_elig = 0 if pos < 0 else min(NB, pos // block_size + 1)
    bs = index_scores(q64, w64, pk[:n_elig])
    kept, _ = select_topk(bs, np.arange(n_elig, dtype=np.int64), n_keep)
    kept = np.sort(kept)
    toks = (kept[:, None] * block_size + np.arange(block_size)[None]).reshape(-1)
    toks = toks[toks < int(prob.k_len[b])]
    return dict(blocks=kept, block_scores=bs, block_magnitude=score_magnitude(q64, w64, pk[:n_elig]),
                tokens=toks)


def group_block(prob, k: int, G: int, block_size: int, n_keep: int):
    """Block-filtered proxy with per-query refine: (out_idx [B,T,k], out_score, scans {(b,g)})."""
    inp = Inputs(prob)
    B, T = prob.q_pos.shape
    NG = (T + G - 1) // G
    out_idx = np.full((B, T, k), -1, np.int32)
    out_sc = np.full((B, T, k), -np.inf)
    scans = {}
    for b in range(B):
        pooled = pool_keys(prob, b, block_size)
        for g in range(NG):
            gs = group_block_scan(inp, b, g, G, block_size, n_keep, pooled)
            scans[(b, g)] = gs
            for t in group_members(T, G, g):
                r = refine_row(inp, b, t, k, gs["tokens"])
                n = len(r["ids"])
                out_idx[b, t, :n] = r["ids"]
                out_sc[b, t, :n] = r["scores"]
    return out_idx, out_sc, scans


def block(prob, k: int, block_size: int, n_keep: int):
    """Full hierarchical output: (out_idx, out_score, blocks [B,T,n_keep] padded with -1)."""
    inp = Inputs(prob)
    B, T = prob.q_pos.shape
    out_idx = np.full((B, T, k), -1, np.int32)
    out_sc = np.full((B, T, k), -np.inf)
    out_blk = np.full((B, T, n_keep), -1, np.int32)
    for b in range(B):
        pooled = pool_keys(prob, b, block_size)
        for t in range(T):
            r = block_row(inp, b, t, k, block_size, n_keep, pooled)
            n = len(r["ids"])
            out_idx[b, t, :n] = r["ids"]
            out_sc[b, t, :n] = r["scores"]
            out_blk[b, t, :len(r["blocks"])] = r["blocks"]
    return out_idx, out_sc, out_blk


# ----------------------------------------------------------------------------------------------
# absorbed-query scoring of a shared latent cache  [LatentIndex]

def absorb_queries(q: np.ndarray, q_dtype: int, wk: np.ndarray) -> Dict[str, np.ndarray]:
    """[LatentIndex] Reading: a layer's indexer key is a linear decoding of the shared latent
    row, k[s] = c[s] @ Wk (latent c[s] of Dc elements, decoder Wk [Dc, D] in bf16), so
    q[h] . k[s] = (Wk @ q[h]) . c[s]: the decoder moves into the query, which then scores the
    latent cache with the unchanged indexer. The absorbed query is itself an indexer query and is
    stored in the query format, bf16 rounded to nearest-even from its exact value (the reading
    the proxy query follows).

    q [..., H, D] in q_dtype storage, wk [Dc, D] bf16 bits. Returns dict(
      bits  [..., H, Dc] uint16: the absorbed queries,
      exact [..., H, Dc] float64: Wk @ q before rounding,
      bound [..., H, Dc] float64: D * 2^-24 * sum_d |Wk[j,d] q[h,d]|, the a-priori error of an
            fp32 evaluation of the same sums, within which another rounding decision is valid)."""
    q64 = queries_f64(q, q_dtype)
    w64 = bf16_bits_to_f64(wk)
    exact = q64 @ w64.T
    bound = (np.abs(q64) @ np.abs(w64).T) * (q64.shape[-1] * 2.0 ** -24)
    return dict(bits=f64_to_bf16_bits_rne(exact), exact=exact, bound=bound)


def latent_problem(prob, q_lat_bits: np.ndarray):
    """The indexer problem the absorbed queries pose: the same head weights, positions and cache
    lengths, queries q_lat (bf16 [B,T,H,Dc]) against the latent cache prob.k [B,N,Dc]."""
    return dataclasses.replace(prob, q=q_lat_bits, q_dtype=BF16, q_scale=None, wk=None)


def latent_definition_row(prob, b: int, t: int, k: int):
    """One query scored as the layer's own indexer would score it: its original queries against
    keys rebuilt from the latent cache (k[s] = c[s] @ Wk, exact in float64) over its causal
    prefix; the top-k as in dense_row. Returns dict(ids, scores, all_scores)."""
    qp = visible_len(int(prob.q_pos[b, t]), int(prob.k_len[b]))
    q64 = queries_f64(prob.q[b, t], prob.q_dtype)
    c64 = keys_f64(prob.k[b, :qp], prob.k_dtype, None if prob.k_scale is None else prob.k_scale[b, :qp])
    keys = c64 @ bf16_bits_to_f64(prob.wk)
    sc = index_scores(q64, np.asarray(prob.w[b, t], np.float32).astype(np.float64), keys)
    ids, top = select_topk(sc, np.arange(qp, dtype=np.int64), k)
    return dict(ids=ids, scores=top, all_scores=sc)
