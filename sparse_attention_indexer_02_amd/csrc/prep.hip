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

__global__ void __launch_bounds__(256) proxy_kernel(ProxyArgs a) {
  const int bg = blockIdx.x;                   // b * n_groups + g
  const int b = bg / a.n_groups, g = bg % a.n_groups;
  const int t0 = g * a.G, t1 = min(t0 + a.G, a.T);
  const float cnt = (float)(t1 - t0);
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t e = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  if (e < HD) {
    float s = 0.f;
    for (int t = t0; t < t1; ++t) {
      const int64_t off = ((int64_t)b * a.T + t) * HD + e;
      const float v = a.q_dtype == DT_BF16
                          ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[off])
                          : reinterpret_cast<const float*>(a.q)[off];
      s += v;
    }
    const float m = __fdiv_rn(s, cnt);
    const int64_t o = (int64_t)bg * HD + e;
    if (a.q_dtype == DT_BF16) reinterpret_cast<uint16_t*>(a.pq)[o] = f32_to_bf16_rne(m);
    else reinterpret_cast<float*>(a.pq)[o] = m;
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
  const int64_t HD = (int64_t)a.H * a.D;
  dim3 grid(a.B * a.n_groups, (unsigned)((HD + 255) / 256));
  hipLaunchKernelGGL(proxy_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  const int b = blockIdx.x / a.n_blocks, j = blockIdx.x % a.n_blocks;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int s0 = j * a.block_size, s1 = min(s0 + a.block_size, kl);
  const int d = blockIdx.y * blockDim.x + threadIdx.x;
  if (d >= a.D) return;
  const int64_t o = ((int64_t)b * a.n_blocks + j) * a.D + d;
  if (s0 >= s1) {                              // block beyond the cache: never scored
    if (a.k_dtype == DT_BF16) reinterpret_cast<uint16_t*>(a.pooled)[o] = 0;
    else reinterpret_cast<float*>(a.pooled)[o] = 0.f;
    return;
  }
  float s = 0.f;
  for (int t = s0; t < s1; ++t) {
    const int64_t off = ((int64_t)b * a.N + t) * a.D + d;
    s += a.k_dtype == DT_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.keys)[off])
                              : reinterpret_cast<const float*>(a.keys)[off];
  }
  const float m = __fdiv_rn(s, (float)(s1 - s0));
  if (a.k_dtype == DT_BF16) reinterpret_cast<uint16_t*>(a.pooled)[o] = f32_to_bf16_rne(m);
  else reinterpret_cast<float*>(a.pooled)[o] = m;
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.n_blocks, (a.D + 255) / 256);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(min(a.D, 256)), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
