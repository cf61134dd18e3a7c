"""Seeded synthetic inputs for the DSA lightning indexer, shared by the oracle's tests,
the HIP path's parity tests and bench.py.

This module only draws random numbers and stores them in the indexer's input formats
(fp32, bf16 bit patterns, OCP FP8 E4M3 bit patterns with one fp32 scale per token). It holds
none of the indexer's arithmetic: no scoring, no selection, no pooling, no proxy queries.

The shapes and value distributions follow the workloads the indexer pages describe: long
prefills and decode steps with multi-token prediction (PIVOT, abstract), k = 2048 selected tokens
(Multi-layer Indexer, abstract), nearby queries with overlapping selections (AR(1) queries) and
long-tailed scores along the key axis (a few heavy key rows or regions) (PIVOT, abstract).

Draw order inside one generator: queries (or their AR noise), keys, heavy rows or regions,
head weights. numpy's PCG64 (`default_rng(seed)`) is the only random source.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8_E4M3: "fp8_e4m3"}
E4M3_MAX = 448.0


@dataclasses.dataclass
class Problem:
    """Indexer inputs in storage form (host numpy arrays).

    q      [B,T,H,D]  float32 (q_dtype F32), uint16 bf16 bit patterns (BF16) or uint8 E4M3FN bits
                      (FP8_E4M3)
    k      [B,N,D]    float32 (F32), uint16 bf16 bits (BF16) or uint8 E4M3FN bits (FP8_E4M3)
    k_scale[B,N]      float32, only for FP8_E4M3 keys (real key = decoded byte * scale)
    w      [B,T,H]    float32 head weights
    q_pos  [B,T]      int32: key s is visible to query (b,t) iff s <= q_pos[b,t] and s < k_len[b]
    k_len  [B]        int32 valid keys per sequence
    q_scale[B,T,H]    float32, only for FP8_E4M3 queries (real query = decoded byte * scale)
    wk     [Dc,D]     uint16 bf16 bits, only for a shared latent cache: k then holds latent rows
                      [B,N,Dc] and a layer's key is latent @ wk (its key decoder)
    """
    q: np.ndarray
    q_dtype: int
    k: np.ndarray
    k_dtype: int
    k_scale: Optional[np.ndarray]
    w: np.ndarray
    q_pos: np.ndarray
    k_len: np.ndarray
    q_scale: Optional[np.ndarray] = None
    wk: Optional[np.ndarray] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def T(self): return self.q.shape[1]
    @property
    def H(self): return self.q.shape[2]
    @property
    def D(self): return self.q.shape[3]
    @property
    def N(self): return self.k.shape[1]

    def pairs(self) -> int:
        """Causally visible (query, key) pairs = dense-equivalent work."""
        P = np.minimum(self.q_pos.astype(np.int64) + 1, self.k_len[:, None].astype(np.int64))
        return int(np.clip(P, 0, None).sum())


# ----------------------------------------------------------------------------------------------
# storage conversions (library routines: torch's RNE casts)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_per_token(x: np.ndarray):
    """Per-token (last axis) scaled E4M3FN: scale = amax/448, byte = RNE(x/scale), saturated."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / safe[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    b = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return b, scale


# ----------------------------------------------------------------------------------------------
# random pieces

def _ar1(rng, B, T, shape, rho):
    """AR(1) along t with unit stationary variance, independent per sequence and element."""
    out = np.empty((B, T) + tuple(shape), np.float32)
    c = np.float32(np.sqrt(1.0 - rho * rho))
    r = np.float32(rho)
    chunk = 256
    for b in range(B):
        prev = None
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            eps = rng.standard_normal((t1 - t0,) + tuple(shape), dtype=np.float32)
            for i in range(t1 - t0):
                if prev is None:
                    prev = eps[i]
                else:
                    prev = r * prev + c * eps[i]
                out[b, t0 + i] = prev
    return out


def _heavy_rows(rng, keys, frac, factor):
    B, N, _ = keys.shape
    n_heavy = int(round(frac * N))
    for b in range(B):
        rows = rng.choice(N, size=n_heavy, replace=False)
        keys[b, rows] *= np.float32(factor)


def _heavy_regions(rng, keys, n_regions, length, factor):
    B, N, _ = keys.shape
    for b in range(B):
        starts = rng.integers(0, N - length + 1, size=n_regions)
        mask = np.zeros(N, bool)
        for s in starts:
            mask[s:s + length] = True
        keys[b, mask] *= np.float32(factor)


def _store(x, dtype):
    if dtype == F32:
        return np.ascontiguousarray(x, np.float32), None
    if dtype == BF16:
        return f32_to_bf16_bits(x), None
    if dtype == FP8_E4M3:
        return f32_to_e4m3_per_token(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# generators

def make_prefill(L, H, D, *, seed=0, rho=0.9, q_dtype=BF16, k_dtype=BF16, heavy_frac=0.01,
                 heavy_factor=3.0, w_scale=0.125, B=1, iid_queries=False) -> Problem:
    """One (or B) causal prefill sequence(s): query t sits at position t, k_len = L. FP8
    queries are quantised per (query, head) vector like the FP8 key cache is per token."""
    rng = np.random.default_rng(seed)
    if iid_queries:
        q = rng.standard_normal((B, L, H, D), dtype=np.float32)
    else:
        q = _ar1(rng, B, L, (H, D), rho)
    keys = rng.standard_normal((B, L, D), dtype=np.float32)
    _heavy_rows(rng, keys, heavy_frac, heavy_factor)
    w = (rng.random((B, L, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    qs, qsc = _store(q, q_dtype)
    ks, sc = _store(keys, k_dtype)
    q_pos = np.broadcast_to(np.arange(L, dtype=np.int32), (B, L)).copy()
    k_len = np.full(B, L, np.int32)
    return Problem(qs, q_dtype, ks, k_dtype, sc, w, q_pos, k_len, q_scale=qsc)


def make_tiny(seed=0, L=1024, H=4, D=32, n_heavy=16) -> Problem:
    """fp32 queries/keys ~ N(0,1), 16 key rows x4, w ~ U(0,1), causal, one sequence."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, L, H, D), dtype=np.float32)
    keys = rng.standard_normal((1, L, D), dtype=np.float32)
    rows = rng.choice(L, size=n_heavy, replace=False)
    keys[0, rows] *= np.float32(4.0)
    w = rng.random((1, L, H), dtype=np.float32)
    q_pos = np.arange(L, dtype=np.int32)[None]
    return Problem(q, F32, keys, F32, None, w, q_pos, np.array([L], np.int32))


def make_decode(B, N, T=2, H=64, D=128, *, seed=0, k_dtype=FP8_E4M3, heavy_frac=0.01,
                heavy_factor=3.0, w_scale=0.125, k_len=None, n_regions=0, region=128) -> Problem:
    """B sequences with N cached keys; the T multi-token-prediction queries of one decode step
    sit at positions k_len-T .. k_len-1 (each sees the earlier ones' keys). Heavy keys are single
    rows (a fraction heavy_frac of the cache), or with n_regions > 0 that many runs of `region`
    consecutive tokens per sequence (the locality a block-level filter relies on)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D), dtype=np.float32)
    keys = np.empty((B, N, D), np.float32)
    for b in range(B):
        keys[b] = rng.standard_normal((N, D), dtype=np.float32)
    if n_regions > 0:
        _heavy_regions(rng, keys, n_regions, region, heavy_factor)
    else:
        _heavy_rows(rng, keys, heavy_frac, heavy_factor)
    w = (rng.random((B, T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    qs, _ = _store(q, BF16)
    ks, sc = _store(keys, k_dtype)
    kl = np.full(B, N, np.int32) if k_len is None else np.asarray(k_len, np.int32)
    q_pos = (kl[:, None] - T + np.arange(T, dtype=np.int32)[None]).astype(np.int32)
    return Problem(qs, BF16, ks, k_dtype, sc, w, q_pos, kl)


def make_hier(N, T, H=64, D=128, *, seed=0, rho=0.9, n_regions=64, region=128,
              heavy_factor=3.0, w_scale=0.125) -> Problem:
    """A T-query prefill chunk at the end of an N-token context (positions N-T .. N-1); keys
    N(0,1) with heavy 128-token regions, AR(1) queries."""
    rng = np.random.default_rng(seed)
    q = _ar1(rng, 1, T, (H, D), rho)
    keys = rng.standard_normal((1, N, D), dtype=np.float32)
    _heavy_regions(rng, keys, n_regions, region, heavy_factor)
    w = (rng.random((1, T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    qs, _ = _store(q, BF16)
    ks, _ = _store(keys, BF16)
    q_pos = (N - T + np.arange(T, dtype=np.int32))[None].astype(np.int32)
    return Problem(qs, BF16, ks, BF16, None, w, q_pos, np.array([N], np.int32))


def make_latent(B, T, N, H=64, D=128, Dc=64, *, seed=0, rho=0.9, k_dtype=BF16, heavy_frac=0.01,
                heavy_factor=3.0, w_scale=0.125, decode=False) -> Problem:
    """A layer that scores a shared latent cache: queries of head dimension D, latent rows of Dc
    elements (N(0,1) with heavy rows, like the key caches), head weights, and the layer's key
    decoder wk [Dc, D] ~ N(0, 1/Dc) (a random projection: the rebuilt keys latent @ wk have unit
    variance, no trained weights). Prefill (decode=False): T = N queries at positions 0..N-1 with
    AR(1) queries; decode: T multi-token-prediction queries at N-T .. N-1 with N(0,1) queries."""
    rng = np.random.default_rng(seed)
    if decode:
        q = rng.standard_normal((B, T, H, D), dtype=np.float32)
    else:
        q = _ar1(rng, B, T, (H, D), rho)
    lat = np.empty((B, N, Dc), np.float32)
    for b in range(B):
        lat[b] = rng.standard_normal((N, Dc), dtype=np.float32)
    _heavy_rows(rng, lat, heavy_frac, heavy_factor)
    w = (rng.random((B, T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    wk = (rng.standard_normal((Dc, D), dtype=np.float32) / np.float32(np.sqrt(Dc))).astype(np.float32)
    qs, _ = _store(q, BF16)
    ks, sc = _store(lat, k_dtype)
    k_len = np.full(B, N, np.int32)
    if decode:
        q_pos = np.broadcast_to((N - T + np.arange(T, dtype=np.int32))[None], (B, T)).astype(np.int32).copy()
    else:
        q_pos = np.broadcast_to(np.arange(T, dtype=np.int32), (B, T)).copy()
    return Problem(qs, BF16, ks, k_dtype, sc, w, q_pos, k_len, wk=f32_to_bf16_bits(wk))


def make_banks(prob: Problem, G: int, C: int, seed: int = 0) -> np.ndarray:
    """Candidate token banks for a per-query refine over caller-supplied sets: for each group of
    G consecutive queries, C distinct tokens drawn uniformly from the group's prefix (the tokens
    up to the largest member position that are in the cache), in random order, -1 padded when the
    prefix is shorter than C. int32 [B, ceil(T/G), C]."""
    rng = np.random.default_rng(seed + 1000)
    B, T = prob.q_pos.shape
    NG = (T + G - 1) // G
    out = np.full((B, NG, C), -1, np.int32)
    for b in range(B):
        for g in range(NG):
            pos = int(prob.q_pos[b, g * G:min(T, g * G + G)].max())
            P = max(0, min(pos + 1, int(prob.k_len[b])))
            m = min(C, P)
            out[b, g, :m] = rng.choice(P, m, replace=False)
    return out


# ----------------------------------------------------------------------------------------------
# named workloads (shapes of the long-context prefill and decode settings the indexer pages study)

WORKLOADS = {
    "tiny": dict(op="dense", k=64, gen=lambda seed=0: make_tiny(seed)),
    "dense16k": dict(op="dense", k=2048,
                     gen=lambda seed=0: make_prefill(16384, 64, 128, seed=seed, rho=0.9)),
    "dense64k": dict(op="dense", k=2048,
                     gen=lambda seed=0: make_prefill(65536, 64, 128, seed=seed, rho=0.95)),
    "dense16k_fp8": dict(op="dense", k=2048,
                         gen=lambda seed=0: make_prefill(16384, 64, 128, seed=seed, rho=0.9,
                                                         q_dtype=FP8_E4M3, k_dtype=FP8_E4M3)),
    "dense64k_fp8": dict(op="dense", k=2048,
                         gen=lambda seed=0: make_prefill(65536, 64, 128, seed=seed, rho=0.95,
                                                         q_dtype=FP8_E4M3, k_dtype=FP8_E4M3)),
    "decode128k": dict(op="dense", k=2048,
                       gen=lambda seed=0: make_decode(32, 131072, 2, seed=seed)),
    "group64k": dict(op="group", k=2048, group_size=16, n_cand=8192,
                     gen=lambda seed=0: make_prefill(65536, 64, 128, seed=seed, rho=0.95)),
    "reuse64k": dict(op="reuse", k=2048, group_size=16,
                     gen=lambda seed=0: make_prefill(65536, 64, 128, seed=seed, rho=0.95)),
    "given16k": dict(op="given", k=2048, group_size=16, n_cand=4096,
                     gen=lambda seed=0: make_prefill(16384, 64, 128, seed=seed, rho=0.9)),
    "gblock128k": dict(op="gblock", k=2048, group_size=16, block_size=128, n_blocks_keep=128,
                       gen=lambda seed=0: make_hier(131072, 4096, seed=seed)),
    "hier128k": dict(op="block", k=2048, block_size=128, n_blocks_keep=128,
                     gen=lambda seed=0: make_hier(131072, 4096, seed=seed)),
    # decode with a block filter on the FP8 cache: 32 sequences of 131072 tokens, 2 queries each,
    # pooled block keys kept beside the cache; per query (block) or shared by a step's 2 queries
    "decodeblk128k": dict(op="block", k=2048, block_size=128, n_blocks_keep=128, pooled=True,
                          gen=lambda seed=0: make_decode(32, 131072, 2, seed=seed, n_regions=64)),
    "decodegblk128k": dict(op="gblock", k=2048, group_size=2, block_size=128, n_blocks_keep=128,
                           pooled=True,
                           gen=lambda seed=0: make_decode(32, 131072, 2, seed=seed, n_regions=64)),
    # decode-phase grouping (a step's 2 MTP queries form one group, PIVOT) on decode128k's inputs
    "decodegroup128k": dict(op="group", k=2048, group_size=2, n_cand=8192,
                            gen=lambda seed=0: make_decode(32, 131072, 2, seed=seed)),
    "decodereuse128k": dict(op="reuse", k=2048, group_size=2,
                            gen=lambda seed=0: make_decode(32, 131072, 2, seed=seed)),
    # a layer scoring a shared 64-dimensional latent cache through absorbed queries (D = 128):
    # a 64K prefill (bf16 latent) and a 128K decode step (FP8 latent with per-token scales)
    "latent64k": dict(op="latent", k=2048,
                      gen=lambda seed=0: make_latent(1, 65536, 65536, seed=seed, rho=0.95)),
    "latentdec128k": dict(op="latent", k=2048,
                          gen=lambda seed=0: make_latent(32, 2, 131072, seed=seed, k_dtype=FP8_E4M3,
                                                         decode=True)),
}
