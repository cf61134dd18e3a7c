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

// Thread = 8 dimensions of one pooled block; D / 8 threads per block, 256 / (D / 8) blocks per
// work-group.
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
    sum_rows8<DT>(a.keys, (int64_t)b * a.N * a.D + d, a.D, s0, s1, s);
    const float n = (float)(s1 - s0);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = __fdiv_rn(s[i], n);
  }
  store8<DT>(a.pooled, o, m);
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  const int per_wg = 256 / (a.D / 8);
  const int64_t nb = (int64_t)a.B * a.n_blocks;
  dim3 grid((unsigned)((nb + per_wg - 1) / per_wg));
  if (a.k_dtype == DT_BF16) hipLaunchKernelGGL(pool_kernel<DT_BF16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(pool_kernel<DT_F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
