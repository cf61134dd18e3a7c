// Per-row top-k selection over fp32 score rows: exact radix select on the order-preserving
// 32-bit image of the scores (digits of 12, 12 and 8 bits, most significant first, counted in
// LDS histograms), then one ordered pass that writes the selected slots in ascending slot order.
// Among slots whose score equals the k-th largest, the lowest slots are taken, so the selected
// set is unique. Slots holding -inf count as "no candidate" and are never selected, so the
// number of selections is min(k, number of finite slots).
//
// The indexer keeps the k = 2048 best tokens of each query ("Multi-layer Indexer ...",
// authors' abstract); the same selector yields the candidate sets of the group and block
// variants ("PIVOT ...", abstract; "HISA ...", abstract).
#include "common.h"
#include "kernels.h"

namespace idx {

constexpr int TK_THREADS = 1024;
constexpr int TK_LDS_CAP = 32768;        // row slots that are staged in LDS
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;

// Exclusive scan over the work-group (1024 threads = 16 waves). sh needs 80 words.
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t s = lane < nw ? sh[lane] : 0u;
    const uint32_t si = wave_incl_scan(s);
    if (lane < nw) sh[32 + lane] = si - s;
    if (lane == 63) sh[64] = si;
  }
  __syncthreads();
  const uint32_t res = sh[32 + wave] + inc - v;
  *total = sh[64];
  __syncthreads();
  return res;
}

// Finds the bin holding the need-th largest element (1 <= need <= sum of hist): returns the bin
// and, in *above, the number of elements in higher bins.
__device__ __forceinline__ int find_bin(const uint32_t* hist, int nbins, uint32_t need,
                                        uint32_t* sh, uint32_t* above) {
  const int per = (nbins + TK_THREADS - 1) / TK_THREADS;
  const int hi = nbins - 1 - (int)threadIdx.x * per;
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int bin = hi - i;
    if (bin >= 0) s += hist[bin];
  }
  uint32_t tot;
  const uint32_t ab = block_scan_excl(s, sh, &tot);
  if (ab < need && need <= ab + s) {
    uint32_t run = ab;
    for (int i = 0; i < per; ++i) {
      const int bin = hi - i;
      const uint32_t h = hist[bin];
      if (run + h >= need) {
        sh[70] = (uint32_t)bin;
        sh[71] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  const int bin = (int)sh[70];
  *above = sh[71];
  __syncthreads();
  return bin;
}

template <bool IN_LDS>
__global__ void __launch_bounds__(TK_THREADS) topk_kernel(TopkArgs a) {
  extern __shared__ __align__(16) uint32_t sm[];
  uint32_t* hist = sm;                 // 4096 bins
  uint32_t* sh = sm + 4096;            // 128 words scratch
  uint32_t* rowk = sm + 4096 + 128;    // staged row (IN_LDS)
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* srow = a.scores + (int64_t)r * a.score_stride;
  const int n = a.row_len[r];
  const int bb = r / a.rows_per_seq, tt = a.t_off + r % a.rows_per_seq;
  const int64_t orow = (int64_t)bb * a.T_out + tt;
  int32_t* oidx = a.out_idx + orow * a.out_stride;
  float* osc = a.out_score ? a.out_score + orow * a.out_stride : nullptr;

  auto KEY = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return rowk[i];
    else return f2key(srow[i]);
  };

  for (int i = tid; i < 4096; i += TK_THREADS) hist[i] = 0u;
  __syncthreads();
  uint32_t nv = 0;
  for (int i = tid; i < n; i += TK_THREADS) {
    const uint32_t u = f2key(srow[i]);
    if constexpr (IN_LDS) rowk[i] = u;
    if (u > KEY_NEG_INF) {
      atomicAdd(&hist[u >> 20], 1u);
      ++nv;
    }
  }
  uint32_t nvalid;
  block_scan_excl(nv, sh, &nvalid);
  const uint32_t kk = min((uint32_t)a.k, nvalid);

  uint32_t T = 0xFFFFFFFFu, need = 0;
  if (kk > 0) {
    uint32_t ab;
    const int b1 = find_bin(hist, 4096, kk, sh, &ab);
    need = kk - ab;
    for (int i = tid; i < 4096; i += TK_THREADS) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += TK_THREADS) {
      const uint32_t u = KEY(i);
      if ((int)(u >> 20) == b1) atomicAdd(&hist[(u >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    const int b2 = find_bin(hist, 4096, need, sh, &ab);
    need -= ab;
    const uint32_t pre = ((uint32_t)b1 << 12) | (uint32_t)b2;
    for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += TK_THREADS) {
      const uint32_t u = KEY(i);
      if ((u >> 8) == pre) atomicAdd(&hist[u & 0xFFu], 1u);
    }
    __syncthreads();
    const int b3 = find_bin(hist, 256, need, sh, &ab);
    need -= ab;
    T = (pre << 8) | (uint32_t)b3;
  }

  // ordered output: slot i is selected iff key > T, or key == T and fewer than `need` equal
  // keys precede it
  uint32_t base_gt = 0, base_eq = 0;
  if (kk > 0) {
    for (int i0 = 0; i0 < n; i0 += TK_THREADS) {
      const int i = i0 + tid;
      const uint32_t u = i < n ? KEY(i) : 0u;
      const uint32_t gt = u > T ? 1u : 0u;
      const uint32_t eq = u == T ? 1u : 0u;
      uint32_t tot;
      const uint32_t ex = block_scan_excl(gt | (eq << 16), sh, &tot);
      const uint32_t gpre = base_gt + (ex & 0xFFFFu), epre = base_eq + (ex >> 16);
      if (gt || (eq && epre < need)) {
        const uint32_t pos = gpre + min(epre, need);
        int key;
        if (a.map_mode == MAP_IDENT) {
          key = i;
        } else if (a.map_mode == MAP_LIST) {
          key = a.list[((int64_t)bb * a.n_groups + tt / a.group_size) * a.list_stride + i];
        } else {
          key = a.blocks[orow * a.blocks_stride + i / a.block_size] * a.block_size + i % a.block_size;
        }
        oidx[pos] = key;
        if (osc) osc[pos] = key2f(u);
      }
      base_gt += tot & 0xFFFFu;
      base_eq += tot >> 16;
    }
  }
  for (int p = (int)kk + tid; p < a.k; p += TK_THREADS) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
  if (a.out_count && tid == 0) a.out_count[orow] = (int32_t)kk;
}

hipError_t launch_topk(const TopkArgs& a, int max_row_len, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const size_t base = (4096 + 128) * sizeof(uint32_t);
  if (max_row_len <= TK_LDS_CAP) {
    const size_t lds = base + (size_t)max(max_row_len, 1) * sizeof(uint32_t);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_kernel<true>, dim3(a.n_rows), dim3(TK_THREADS), lds, s, a);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, dim3(a.n_rows), dim3(TK_THREADS), base, s, a);
  }
  return hipGetLastError();
}

}  // namespace idx
