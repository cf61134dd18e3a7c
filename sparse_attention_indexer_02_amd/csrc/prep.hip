// Small producer kernels of the two accelerated indexer variants.
//
// proxy_kernel: one proxy query per group of consecutive queries ("PIVOT: Efficient Query-Group
//   Indexing for Token-Level Sparse Attention", abstract). Reading of the aggregation: the
//   element-wise mean of the members' queries and head weights, summed in fp32 in ascending
//   member order from +0, divided once (IEEE fp32), and rounded to bf16 (nearest-even) when the
//   queries are bf16, because the proxy is itself an indexer query. Its position is the largest
//   member position, so its scan covers the prefix of every member.
//
// pool_kernel: pooled block keys ("HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
//   Attention", abstract, scores pooled block representations). Reading: the mean of the keys
//   of each block of consecutive tokens that are in the cache, with the same fp32 order and
//   rounding rule as the proxy, stored in the key format.
//
// given_lists_kernel: candidate sets supplied by the caller for a per-query refine ("ADIndex:
//   Layer-Adaptive Sparse Attention Indexing via Group-Level Distillation", abstract: a token bank
//   shared within a query group, refined per query; "LatentIndex: Cross-Layer Sharing with
//   Layer-Specific Selection for Sparse Attention", abstract: followers refine the candidate set
//   the anchor proposes). Each list becomes a set of token ids in ascending order.
//
// reuse_rows_kernel: PIVOT-Reuse ("PIVOT ...", abstract: the proxy's top-k is shared across the
//   group). Reading: each member keeps the proxy's top-k tokens inside its own causal prefix,
//   with the proxy's scores.
//
// expand_blocks_kernel: the block-filtered proxy (a PIVOT group proxy scoring HISA's pooled
//   blocks): the kept blocks of a group become its candidate token list.
#include "common.h"
#include "kernels.h"

namespace idx {

// 8 consecutive elements of a row as fp32 (one 16-byte load for bf16, two for fp32)
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t e, float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(base) + e);
    const f32x4_t y = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(base) + e + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = x[i];
      v[4 + i] = y[i];
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t e, const float (&m)[8]) {
  if constexpr (DT == DT_BF16) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16_rne(m[2 * i]) | ((uint32_t)f32_to_bf16_rne(m[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(base) + e) = w;
  } else {
    f32x4_t x, y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = m[i];
      y[i] = m[4 + i];
    }
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + e) = x;
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + e + 4) = y;
  }
}

// Sum over rows r0 .. r1-1 (stride `step` elements) of 8 elements, in ascending row order from
// +0; loads run four rows ahead of the adds.
template <int DT>
__device__ __forceinline__ void sum_rows8(const void* base, int64_t e0, int64_t step, int r0, int r1,
                                          float (&s)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.f;
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<DT>(base, e0 + (int64_t)(r + u) * step, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += v[u][i];
  }
  for (; r < r1; ++r) {
    float v[8];
    load8<DT>(base, e0 + (int64_t)r * step, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += v[i];
  }
}

template <int DT>
__global__ void __launch_bounds__(256) proxy_kernel(ProxyArgs a) {
  const int bg = blockIdx.x;                   // b * n_groups + g
  const int b = bg / a.n_groups, g = bg % a.n_groups;
  const int t0 = g * a.G, t1 = min(t0 + a.G, a.T);
  const float cnt = (float)(t1 - t0);
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t e = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (e < HD) {
    float s[8];
    sum_rows8<DT>(a.q, (int64_t)b * a.T * HD + e, HD, t0, t1, s);
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = __fdiv_rn(s[i], cnt);
    store8<DT>(a.pq, (int64_t)bg * HD + e, m);
  }
  if (blockIdx.y == 0) {
    for (int h = threadIdx.x; h < a.H; h += blockDim.x) {
      float s = 0.f;
      for (int t = t0; t < t1; ++t) s += a.w[((int64_t)b * a.T + t) * a.H + h];
      a.pw[(int64_t)bg * a.H + h] = __fdiv_rn(s, cnt);
    }
    if (threadIdx.x == 0) {
      int p = a.q_pos[(int64_t)b * a.T + t0];
      for (int t = t0 + 1; t < t1; ++t) p = max(p, a.q_pos[(int64_t)b * a.T + t]);
      a.ppos[bg] = p;
    }
  }
}

hipError_t launch_proxy(const ProxyArgs& a, hipStream_t s) {
  const int64_t HD = (int64_t)a.H * a.D;    // D in {32, 64, 128}: a multiple of 8
  dim3 grid(a.B * a.n_groups, (unsigned)((HD / 8 + 255) / 256));
  if (a.q_dtype == DT_BF16) hipLaunchKernelGGL(proxy_kernel<DT_BF16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(proxy_kernel<DT_F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// FP8 keys: the same ascending sum over the fp32 key values decode(byte) * scale (one rounding
// each; multiply and add kept apart: the compiler would otherwise contract them into an FMA,
// which rounds once).
__device__ __forceinline__ void sum_rows8_fp8(const uint8_t* base, const float* scale, int64_t e0, int64_t step,
                                              int r0, int r1, float (&s)[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.f;
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    u32x2_t v[4];
    float sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = *reinterpret_cast<const u32x2_t*>(base + e0 + (int64_t)(r + u) * step);
      sc[u] = scale[r + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        s[i] = s[i] + e4m3_to_f32((v[u][i >> 2] >> (8 * (i & 3))) & 0xFFu) * sc[u];
  }
  for (; r < r1; ++r) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(base + e0 + (int64_t)r * step);
    const float sc = scale[r];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s[i] = s[i] + e4m3_to_f32((v[i >> 2] >> (8 * (i & 3))) & 0xFFu) * sc;
  }
}

// Thread = 8 dimensions of one pooled block; D / 8 threads per block, 256 / (D / 8) blocks per
// work-group. DT is the key format; pooled keys are fp32 for fp32 keys, bf16 otherwise.
template <int DT>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  const int tpb = a.D / 8;
  const int64_t jb = (int64_t)blockIdx.x * (256 / tpb) + threadIdx.x / tpb;   // b * n_blocks + j
  if (jb >= (int64_t)a.B * a.n_blocks) return;
  const int b = (int)(jb / a.n_blocks), j = (int)(jb % a.n_blocks);
  const int d = (threadIdx.x % tpb) * 8;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int s0 = j * a.block_size, s1 = min(s0 + a.block_size, kl);
  const int64_t o = jb * a.D + d;
  float m[8];
  if (s0 >= s1) {                              // block beyond the cache: never scored
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0.f;
  } else {
    float s[8];
    if constexpr (DT == DT_FP8)
      sum_rows8_fp8(reinterpret_cast<const uint8_t*>(a.keys), a.k_scale + (int64_t)b * a.N,
                    (int64_t)b * a.N * a.D + d, a.D, s0, s1, s);
    else
      sum_rows8<DT>(a.keys, (int64_t)b * a.N * a.D + d, a.D, s0, s1, s);
    const float n = (float)(s1 - s0);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = __fdiv_rn(s[i], n);
  }
  store8<DT == DT_F32 ? DT_F32 : DT_BF16>(a.pooled, o, m);
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  const int per_wg = 256 / (a.D / 8);
  const int64_t nb = (int64_t)a.B * a.n_blocks;
  dim3 grid((unsigned)((nb + per_wg - 1) / per_wg));
  if (a.k_dtype == DT_FP8) hipLaunchKernelGGL(pool_kernel<DT_FP8>, grid, dim3(256), 0, s, a);
  else if (a.k_dtype == DT_BF16) hipLaunchKernelGGL(pool_kernel<DT_BF16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(pool_kernel<DT_F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Row r = b * n_groups + g of `src` (C entries, the first cnt[r] of them used, all when cnt is
// NULL; counts are clamped into [0, C]) becomes the ascending set of its values inside
// [0, k_len[b]) (k_len NULL: [0, N)) in row r of `dst` (C entries), with the set's size in
// dst_cnt[r]. Other values, such as -1 padding or tokens not in the cache, are dropped and
// repeated values are kept once. One work-group per row: the values set bits of an
// LDS bitmap of N bits, then each thread writes the set bits of its contiguous range of words at
// the exclusive prefix of the popcounts.
// STAGE: the ascending set is assembled in LDS after the bitmap ([C] words) and written out
// coalesced (each thread emits a contiguous run, so direct stores scatter a wave's writes)
template <bool STAGE>
__global__ void __launch_bounds__(256) given_lists_kernel(const int32_t* src, const int32_t* cnt, int C,
                                                          int N, const int32_t* k_len, int n_groups,
                                                          int32_t* dst, int32_t* dst_cnt, int nwords) {
  extern __shared__ uint32_t bm[];
  int32_t* stg = reinterpret_cast<int32_t*>(bm + nwords);
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int32_t* row = src + (int64_t)r * C;
  int32_t* out = dst + (int64_t)r * C;
  const int c = cnt ? min(max(cnt[r], 0), C) : C;
  const int kl = k_len ? max(0, min(k_len[r / n_groups], N)) : N;
  for (int i = tid; i < nwords; i += 256) bm[i] = 0u;
  __syncthreads();
  for (int i = tid; i < c; i += 256) {
    const int v = row[i];
    if (v >= 0 && v < kl) atomicOr(&bm[v >> 5], 1u << (v & 31));
  }
  __syncthreads();
  const int per = (nwords + 255) / 256;
  const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
  uint32_t n = 0;
  for (int w = w0; w < w1; ++w) n += __popc(bm[w]);
  const uint32_t inc = wave_scan_dpp(n);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pos = inc - n;
  for (int w = 0; w < wave; ++w) pos += wsum[w];
  int32_t* o = STAGE ? stg : out;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bm[w];
    while (m) {
      o[pos++] = w * 32 + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
  const int total = (int)(wsum[0] + wsum[1] + wsum[2] + wsum[3]);   // <= c distinct values
  if constexpr (STAGE) {
    __syncthreads();
    for (int i = tid; i < total; i += 256) out[i] = stg[i];
  }
  if (tid == 0) dst_cnt[r] = total;
}

// One wave per member row (b, t) of group g = t / G: the first gcnt[b * NG + g] entries of the
// group's top-k row (gidx, gsc: [B, NG, k]) that lie in the member's prefix
// [0, min(q_pos + 1, k_len)) go to out_idx / out_score row (b, t) in the group's order; the rest
// of the row is -1 / -inf.
__global__ void __launch_bounds__(256) reuse_rows_kernel(ReuseArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.T) return;                 // whole wave
  const int b = (int)(row / a.T), t = (int)(row % a.T), g = t / a.G;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int P = max(0, min(a.q_pos[row] + 1, kl));
  const int64_t src = ((int64_t)b * a.NG + g) * a.k;
  const int n = min(max(a.gcnt[(int64_t)b * a.NG + g], 0), a.k);
  int32_t* oi = a.out_idx + row * a.k;
  float* os = a.out_score ? a.out_score + row * a.k : nullptr;
  // eight 64-entry steps are loaded before their stores (the compiler keeps a load behind a
  // store it cannot prove distinct, so per-step loads would pay their latencies one by one)
  constexpr int U = 8;
  int pos = 0;
  for (int i0 = 0; i0 < n; i0 += 64 * U) {
    int v[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 64 * u + lane;
      v[u] = i < n ? a.gidx[src + i] : -1;
      sc[u] = i < n ? a.gsc[src + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool keep = v[u] >= 0 && v[u] < P;
      const uint64_t m = __ballot(keep);
      if (keep) {
        const int p = pos + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        oi[p] = v[u];
        if (os) os[p] = sc[u];
      }
      pos += __popcll(m);
    }
  }
  for (int p = pos + lane; p < a.k; p += 64) {
    oi[p] = -1;
    if (os) os[p] = -INFINITY;
  }
}

hipError_t launch_reuse_rows(const ReuseArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.T;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(reuse_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Row r = b * n_groups + g: the first n_kept[r] block ids of blocks row r (ascending, `keep` per
// row) become the ascending list of their tokens inside the cache, [0, k_len[b]), in row r of
// `list` (keep * block_size entries), with the count in cnt[r]. Only the highest block can be
// partial, so the tokens of block j start at entry j * block_size.
__global__ void __launch_bounds__(256) expand_blocks_kernel(const int32_t* blocks, const int32_t* n_kept,
                                                            int keep, int block_size, int N,
                                                            const int32_t* k_len, int n_groups,
                                                            int32_t* list, int32_t* cnt) {
  const int r = blockIdx.x;
  const int kl = k_len ? max(0, min(k_len[r / n_groups], N)) : N;
  const int nk = min(max(n_kept[r], 0), keep);
  const int32_t* brow = blocks + (int64_t)r * keep;
  int32_t* out = list + (int64_t)r * keep * block_size;
  const int total = nk * block_size;
  for (int i = threadIdx.x; i < total; i += 256) {
    const int tok = brow[i / block_size] * block_size + i % block_size;
    out[i] = tok < kl ? tok : -1;
  }
  if (threadIdx.x == 0)
    cnt[r] = nk > 0 ? (nk - 1) * block_size + min(block_size, kl - brow[nk - 1] * block_size) : 0;
}

hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* n_kept, int keep, int block_size,
                                int N, const int32_t* k_len, int n_groups, int32_t* list, int32_t* cnt,
                                int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(expand_blocks_kernel, dim3(n_rows), dim3(256), 0, s, blocks, n_kept, keep, block_size,
                     N, k_len, n_groups, list, cnt);
  return hipGetLastError();
}

hipError_t launch_given_lists(const int32_t* src, const int32_t* cnt, int C, int N, const int32_t* k_len,
                              int n_groups, int32_t* dst, int32_t* dst_cnt, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int nwords = (N + 31) / 32;
  if (nwords > 32768) return hipErrorInvalidValue;   // the bitmap must fit in LDS (128 KB)
  const size_t staged = ((size_t)nwords + (size_t)C) * sizeof(uint32_t);
  if (staged <= 65536) {
    hipLaunchKernelGGL(given_lists_kernel<true>, dim3(n_rows), dim3(256), staged, s, src, cnt, C, N, k_len,
                       n_groups, dst, dst_cnt, nwords);
    return hipGetLastError();
  }
  const size_t lds = (size_t)nwords * sizeof(uint32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(given_lists_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(given_lists_kernel<false>, dim3(n_rows), dim3(256), lds, s, src, cnt, C, N, k_len, n_groups,
                     dst, dst_cnt, nwords);
  return hipGetLastError();
}

}  // namespace idx
