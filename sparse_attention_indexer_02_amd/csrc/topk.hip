// Per-row top-k selection over fp32 score rows.
//
// Exact radix select on the order-preserving 32-bit image of the scores:
//   1. one sweep over the row builds an LDS histogram of the top 12 bits and counts the finite
//      slots; a suffix scan finds the bin b1 that holds the k-th largest key;
//   2. a second sweep compacts the slots of bin b1 (the candidates) into LDS; the remaining 20
//      bits are resolved on the candidates only (12-bit, then 8-bit histograms), giving the
//      exact k-th key T and the number `need` of slots equal to T that are kept;
//   3. two ordered sweeps (count, then write) give every selected slot its output position:
//      (slots > T before it) + min(slots == T before it, need). Positions come from wave ballots
//      and per-wave prefix counts, so the output is in ascending slot order and, among slots
//      equal to T, the lowest ones are kept.
// If more slots than fit in LDS share bin b1, step 2 falls back to sweeping the whole row for
// the remaining digits. Slots holding -inf are "no candidate" and never selected, so a row
// yields min(k, number of finite slots) selections.
//
// The indexer keeps the k = 2048 best tokens of each query ("Multi-layer Indexer ...",
// authors' abstract); the same selector yields the candidate sets of the group and block
// variants ("PIVOT ...", abstract; "HISA ...", abstract).
#include "common.h"
#include "kernels.h"

namespace idx {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAND = 4096;                 // candidate slots kept in LDS

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive scan over the work-group (TK_THREADS threads). sh needs 2 * TK_WAVES + 1 words.
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t s = lane < TK_WAVES ? sh[lane] : 0u;
    const uint32_t si = wave_incl_scan(s);
    if (lane < TK_WAVES) sh[TK_WAVES + lane] = si - s;
    if (lane == 63) sh[2 * TK_WAVES] = si;
  }
  __syncthreads();
  const uint32_t res = sh[TK_WAVES + wave] + inc - v;
  *total = sh[2 * TK_WAVES];
  __syncthreads();
  return res;
}

// Bin holding the need-th largest element (1 <= need <= sum of hist); *above = elements in
// higher bins.
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
        sh[32] = (uint32_t)bin;
        sh[33] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  const int bin = (int)sh[32];
  *above = sh[33];
  __syncthreads();
  return bin;
}

__global__ void __launch_bounds__(TK_THREADS) topk_long_kernel(TopkArgs a) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t ckey[TK_CAND];
  __shared__ uint32_t cidx[TK_CAND];
  __shared__ uint32_t sh[64];
  __shared__ uint32_t wcnt[2 * TK_WAVES];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = a.scores + (int64_t)r * a.score_stride;
  const int n = a.row_len[r];
  const int bb = r / a.rows_per_seq, tt = a.t_off + r % a.rows_per_seq;
  const int64_t orow = (int64_t)bb * a.T_out + tt;
  int32_t* oidx = a.out_idx + orow * a.out_stride;
  float* osc = a.out_score ? a.out_score + orow * a.out_stride : nullptr;

  for (int i = tid; i < 4096; i += TK_THREADS) hist[i] = 0u;
  if (tid == 0) sh[40] = 0u;
  __syncthreads();

  // sweep 1: histogram of the top 12 bits, count of finite slots (16-byte loads)
  uint32_t nv = 0;
  const int n4 = n & ~3;
  for (int i = tid * 4; i < n4; i += TK_THREADS * 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(srow + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = f2key(v[e]);
      if (u > KEY_NEG_INF) {
        atomicAdd(&hist[u >> 20], 1u);
        ++nv;
      }
    }
  }
  for (int i = n4 + tid; i < n; i += TK_THREADS) {
    const uint32_t u = f2key(srow[i]);
    if (u > KEY_NEG_INF) {
      atomicAdd(&hist[u >> 20], 1u);
      ++nv;
    }
  }
  uint32_t nvalid;
  block_scan_excl(nv, sh, &nvalid);
  const uint32_t kk = min((uint32_t)a.k, nvalid);

  uint32_t T = KEY_NEG_INF, need = 0;          // kk == nvalid: every finite slot is selected
  if (kk > 0 && kk < nvalid) {
    uint32_t ab;
    const int b1 = find_bin(hist, 4096, kk, sh, &ab);
    need = kk - ab;
    const uint32_t c1 = hist[b1];
    __syncthreads();
    for (int i = tid; i < 4096; i += TK_THREADS) hist[i] = 0u;
    __syncthreads();
    if (c1 <= (uint32_t)TK_CAND) {
      // sweep 2: compact bin b1 into LDS
      for (int i0 = wave * 64; i0 < n; i0 += TK_THREADS) {
        const int i = i0 + lane;
        const uint32_t u = i < n ? f2key(srow[i]) : 0u;
        const bool c = (int)(u >> 20) == b1 && i < n;
        const uint64_t m = __ballot(c);
        if (m) {
          uint32_t basec = 0;
          if (lane == 0) basec = atomicAdd(&sh[40], (uint32_t)__popcll(m));
          basec = __shfl(basec, 0, 64);
          if (c) {
            const uint32_t p = basec + lanes_below(m);
            ckey[p] = u;
            cidx[p] = (uint32_t)i;
          }
        }
      }
      __syncthreads();
      for (uint32_t j = tid; j < c1; j += TK_THREADS) atomicAdd(&hist[(ckey[j] >> 8) & 0xFFFu], 1u);
      __syncthreads();
      const int b2 = find_bin(hist, 4096, need, sh, &ab);
      need -= ab;
      const uint32_t pre = ((uint32_t)b1 << 12) | (uint32_t)b2;
      for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < c1; j += TK_THREADS)
        if ((ckey[j] >> 8) == pre) atomicAdd(&hist[ckey[j] & 0xFFu], 1u);
      __syncthreads();
      const int b3 = find_bin(hist, 256, need, sh, &ab);
      need -= ab;
      T = (pre << 8) | (uint32_t)b3;
    } else {
      // many slots share the top 12 bits: resolve the other digits over the whole row
      for (int i = tid; i < n; i += TK_THREADS) {
        const uint32_t u = f2key(srow[i]);
        if ((int)(u >> 20) == b1) atomicAdd(&hist[(u >> 8) & 0xFFFu], 1u);
      }
      __syncthreads();
      const int b2 = find_bin(hist, 4096, need, sh, &ab);
      need -= ab;
      const uint32_t pre = ((uint32_t)b1 << 12) | (uint32_t)b2;
      for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += TK_THREADS) {
        const uint32_t u = f2key(srow[i]);
        if ((u >> 8) == pre) atomicAdd(&hist[u & 0xFFu], 1u);
      }
      __syncthreads();
      const int b3 = find_bin(hist, 256, need, sh, &ab);
      need -= ab;
      T = (pre << 8) | (uint32_t)b3;
    }
  }

  // sweeps 3-4: ordered output. Wave w owns the contiguous slot range [w*chunk, (w+1)*chunk).
  if (kk > 0) {
    const int chunk = ((n + TK_WAVES - 1) / TK_WAVES + 63) & ~63;
    const int s0 = min(n, wave * chunk), s1 = min(n, s0 + chunk);
    uint32_t cg = 0, ce = 0;
    for (int i0 = s0; i0 < s1; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t u = i < s1 ? f2key(srow[i]) : 0u;
      cg += (uint32_t)__popcll(__ballot(u > T));
      ce += (uint32_t)__popcll(__ballot(u == T && i < s1));
    }
    if (lane == 0) {
      wcnt[wave] = cg;
      wcnt[TK_WAVES + wave] = ce;
    }
    __syncthreads();
    uint32_t bg = 0, be = 0;
    for (int w = 0; w < wave; ++w) {
      bg += wcnt[w];
      be += wcnt[TK_WAVES + w];
    }
    const int gmode = a.map_mode;
    const int32_t* lrow = gmode == MAP_LIST
        ? a.list + ((int64_t)bb * a.n_groups + tt / a.group_size) * a.list_stride : nullptr;
    const int32_t* brow = gmode == MAP_BLOCKS ? a.blocks + orow * a.blocks_stride : nullptr;
    for (int i0 = s0; i0 < s1; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t u = i < s1 ? f2key(srow[i]) : 0u;
      const bool gt = u > T;
      const bool eq = u == T && i < s1;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const uint32_t gpre = bg + lanes_below(mg), epre = be + lanes_below(me);
      if (gt || (eq && epre < need)) {
        const uint32_t pos = gpre + min(epre, need);
        int key;
        if (gmode == MAP_IDENT) key = i;
        else if (gmode == MAP_LIST) key = lrow[i];
        else key = brow[i / a.block_size] * a.block_size + i % a.block_size;
        oidx[pos] = key;
        if (osc) osc[pos] = key2f(u);
      }
      bg += (uint32_t)__popcll(mg);
      be += (uint32_t)__popcll(me);
    }
  }
  for (int p = (int)kk + tid; p < a.k; p += TK_THREADS) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
  if (a.out_count && tid == 0) a.out_count[orow] = (int32_t)kk;
}

// Register-resident selector for rows of up to NWV * 256 * J slots. Wave w owns the contiguous
// slot range [w*CH, (w+1)*CH), CH = 256 * J; lane l holds slots w*CH + 256*j + 4*l + e
// (16-byte loads, all issued before use). Digit histograms (11/11/10 bits) are built with LDS
// atomics from the registers; each threshold search runs in a single wave with DPP scans; the
// ordered output takes per-lane counts, one DPP scan per 256-slot block and one table of wave
// totals. A row's scores span a narrow range (one query's scores: a few binary exponents), so
// the keys are first re-based on the row: v = (x - min) << s + 2^23 (s aligns the row's range
// to bit 30) maps the finite keys one to one and in order onto the upper part of the key space,
// which spreads them over ~1024 first-digit bins instead of a handful, where the histogram's
// LDS atomics would collide; selected keys are mapped back for their scores.
template <int NWV, int J>
__global__ void __launch_bounds__(64 * NWV) topk_reg_kernel(TopkArgs a) {
  constexpr int NT = 64 * NWV;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t bc[8];                     // broadcast: bin, above, ...
  __shared__ uint32_t wtot[2 * NWV];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = a.scores + (int64_t)r * a.score_stride;
  const int n = a.row_len[r];
  const int bb = r / a.rows_per_seq, tt = a.t_off + r % a.rows_per_seq;
  const int64_t orow = (int64_t)bb * a.T_out + tt;
  int32_t* oidx = a.out_idx + orow * a.out_stride;
  float* osc = a.out_score ? a.out_score + orow * a.out_stride : nullptr;
  const int CH = 256 * J;
  const int w0 = wave * CH;

  uint32_t u[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = w0 + 256 * j + 4 * lane;
    if (i + 4 <= n) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(srow + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[j][e] = f2key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[j][e] = i + e < n ? f2key(srow[i + e]) : 0u;
    }
  }
  // the row's finite key range
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (u[j][e] > KEY_NEG_INF) {
        kmin = min(kmin, u[j][e]);
        kmax = max(kmax, u[j][e]);
      }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    wtot[wave] = kmin;
    wtot[NWV + wave] = kmax;
  }
  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    kmin = min(kmin, wtot[w]);
    kmax = max(kmax, wtot[NWV + w]);
  }
  // no finite key: kmin > kmax, nothing is re-based
  const uint32_t rng = kmax >= kmin ? kmax - kmin : 0u;
  const int rs = rng ? max(__builtin_clz(rng) - 1, 0) : 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (u[j][e] > KEY_NEG_INF) u[j][e] = KEY_NEG_INF + 1u + ((u[j][e] - kmin) << rs);
  auto orig_key = [&](uint32_t v) -> uint32_t { return ((v - KEY_NEG_INF - 1u) >> rs) + kmin; };
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (u[j][e] > KEY_NEG_INF) atomicAdd(&hist[u[j][e] >> 21], 1u);
  __syncthreads();

  // wave 0: total finite count and the bin of the need-th largest key, with the bank-spread
  // histogram walk (a need above the total finds no bin: every finite key is then selected)
  auto wave_find = [&](int nbins, uint32_t need, bool) {
    int bin;
    uint32_t above;
    const uint32_t tot = wave_hist_find(nbins, need, [&](int i) { return hist[i]; }, &bin, &above);
    if (lane == 0) {
      bc[2] = tot;
      if (bin >= 0) {
        bc[0] = (uint32_t)bin;
        bc[1] = above;
      }
    }
  };
  if (wave == 0) wave_find(2048, (uint32_t)a.k, true);
  __syncthreads();
  const uint32_t nvalid = bc[2];
  const uint32_t kk = min((uint32_t)a.k, nvalid);
  uint32_t T = KEY_NEG_INF, need = 0;            // kk == nvalid: every finite slot is selected
  if (kk > 0 && kk < nvalid) {
    const uint32_t b1 = bc[0];
    need = kk - bc[1];
    __syncthreads();
    for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((u[j][e] >> 21) == b1) atomicAdd(&hist[(u[j][e] >> 10) & 0x7FFu], 1u);
    __syncthreads();
    if (wave == 0) wave_find(2048, need, false);
    __syncthreads();
    const uint32_t pre = (b1 << 11) | bc[0];
    need -= bc[1];
    __syncthreads();
    for (int i = tid; i < 1024; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((u[j][e] >> 10) == pre) atomicAdd(&hist[u[j][e] & 0x3FFu], 1u);
    __syncthreads();
    if (wave == 0) wave_find(1024, need, false);
    __syncthreads();
    T = (pre << 10) | bc[0];
    need -= bc[1];
  }

  if (kk > 0) {
    uint32_t ex[J];
    uint32_t wg = 0, we = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (u[j][e] > T ? 1u : 0u) | (u[j][e] == T ? 0x10000u : 0u);
      const uint32_t inc = wave_scan_dpp(c);
      ex[j] = (inc - c) + ((we << 16) | wg);
      const uint32_t tot = wave_bcast(inc, 63);
      wg += tot & 0xFFFFu;
      we += tot >> 16;
    }
    if (lane == 0) {
      wtot[wave] = wg;
      wtot[NWV + wave] = we;
    }
    __syncthreads();
    uint32_t bg = 0, be = 0;
    for (int w = 0; w < wave; ++w) {
      bg += wtot[w];
      be += wtot[NWV + w];
    }
    const int gmode = a.map_mode;
    const int32_t* lrow = gmode == MAP_LIST
        ? a.list + ((int64_t)bb * a.n_groups + tt / a.group_size) * a.list_stride : nullptr;
    const int32_t* brow = gmode == MAP_BLOCKS ? a.blocks + orow * a.blocks_stride : nullptr;
    // with blocks of a multiple of 4 slots, a lane's 4 slots of step j share one block: its id is
    // loaded for every step before the first output store (the compiler keeps a load after a
    // store it cannot prove distinct, so loads between the stores would pay their latencies one
    // after another)
    const bool bk4 = gmode == MAP_BLOCKS && (a.block_size & 3) == 0;
    int bk[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = w0 + 256 * j + 4 * lane;
      bk[j] = bk4 && i < n ? brow[i / a.block_size] * a.block_size - i / a.block_size * a.block_size : 0;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t gb = bg + (ex[j] & 0xFFFFu), eb = be + (ex[j] >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = u[j][e];
        const bool gt = x > T, eq = x == T;
        if (gt || (eq && eb < need)) {
          const uint32_t pos = gb + min(eb, need);
          const int i = w0 + 256 * j + 4 * lane + e;
          int key;
          if (gmode == MAP_IDENT) key = i;
          else if (gmode == MAP_LIST) key = lrow[i];
          else if (bk4) key = bk[j] + i;
          else key = brow[i / a.block_size] * a.block_size + i % a.block_size;
          oidx[pos] = key;
          if (osc) osc[pos] = key2f(orig_key(x));
        }
        gb += gt ? 1u : 0u;
        eb += eq ? 1u : 0u;
      }
    }
  }
  for (int p = (int)kk + tid; p < a.k; p += NT) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
  if (a.out_count && tid == 0) a.out_count[orow] = (int32_t)kk;
}

// ---------------------------------------------------------------------------------------------
// Selector for rows that come with a summary from the score kernel (finite count, bin b1 of the
// k-th key in the first radix digit, slots above b1, slots in b1). One streaming pass: slots above
// b1 are written straight away, slots in b1 are compacted into LDS; the remaining key bits are
// resolved on those candidates; among candidates equal to the exact k-th key the lowest slots
// are kept. Output order within a row is unspecified (positions from LDS counters); the selected
// set is deterministic. Rows whose b1 holds more slots than fit in LDS re-read the row for the
// remaining digits.
constexpr int TS_THREADS = 256;
constexpr int TS_WAVES = TS_THREADS / 64;
constexpr int TS_CAND = 3072;
constexpr int TS_OUT = 2048;                     // selections staged in LDS, stored at the end
constexpr int TS_UNROLL = 2;

template <int MAPM, bool BIGK>
__global__ void __launch_bounds__(TS_THREADS) topk_stream_kernel(TopkArgs a) {
  __shared__ uint32_t ckey[TS_CAND];
  __shared__ uint32_t cidx[TS_CAND];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cnt[2];                    // selections written, candidates collected
  __shared__ uint32_t bcv[4];
  __shared__ uint32_t weq[TS_WAVES];
  __shared__ int32_t obi[TS_OUT];
  __shared__ float obs[TS_OUT];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = a.scores + (int64_t)r * a.score_stride;
  const int n = a.row_len[r];
  const int bb = r / a.rows_per_seq, tt = a.t_off + r % a.rows_per_seq;
  const int64_t orow = (int64_t)bb * a.T_out + tt;
  int32_t* oidx = a.out_idx + orow * a.out_stride;
  float* osc = a.out_score ? a.out_score + orow * a.out_stride : nullptr;
  const int32_t* lrow = MAPM == MAP_LIST
      ? a.list + ((int64_t)bb * a.n_groups + tt / a.group_size) * a.list_stride : nullptr;
  const int32_t* brow = MAPM == MAP_BLOCKS ? a.blocks + orow * a.blocks_stride : nullptr;
  auto map_key = [&](int i) -> int {
    if constexpr (MAPM == MAP_IDENT) return i;
    else if constexpr (MAPM == MAP_LIST) return lrow[i];
    else return brow[i / a.block_size] * a.block_size + i % a.block_size;
  };
  // selections (slot, score) go to LDS and are mapped and stored at the end: global traffic
  // inside the streaming loop would make every wait for the next block's loads wait for it too.
  // Positions past TS_OUT (only when k > TS_OUT) go straight out.
  auto emit = [&](uint32_t pos, int i, uint32_t key) {
    if (!BIGK || pos < (uint32_t)TS_OUT) {
      obi[pos] = i;
      obs[pos] = key2f(key);
    } else {
      oidx[pos] = map_key(i);
      if (osc) osc[pos] = key2f(key);
    }
  };
  const int d1 = a.digit_bits;                   // first digit: key >> (32 - d1)
  const int s1 = 32 - d1;
  const int d2 = s1 - 10;                        // second digit: bits [s1-1 : 10]
  const uint32_t m2 = (1u << d2) - 1u;

  const int32_t* meta = a.row_meta + (int64_t)r * 4;
  const uint32_t nvalid = n > 0 ? (uint32_t)meta[META_NVALID] : 0u;
  const uint32_t kk = min((uint32_t)a.k, nvalid);
  const bool all = kk == nvalid;                 // every finite slot is selected
  const uint32_t b1 = all ? 0u : (uint32_t)meta[META_BIN];
  const uint32_t above = all ? 0u : (uint32_t)meta[META_ABOVE];
  const uint32_t c1 = all ? 0u : (uint32_t)meta[META_INBIN];
  const bool fits = c1 <= (uint32_t)TS_CAND;
  if (tid == 0) {
    cnt[0] = 0u;
    cnt[1] = 0u;
  }
  __syncthreads();

  // streaming pass (next block's loads issued before the current block is processed)
  if (kk > 0) {
    constexpr int STEP = TS_THREADS * 4 * TS_UNROLL;
    // branch-free 16-byte loads: the address is clamped into the row's allocation (stride >=
    // n rounded up to 64) and slots at or past n are masked out
    const int last = (int)a.score_stride - 4;
    auto load = [&](int base, f32x4_t (&v)[TS_UNROLL]) {
#pragma unroll
      for (int q = 0; q < TS_UNROLL; ++q)
        v[q] = *reinterpret_cast<const f32x4_t*>(srow + min(base + (q * TS_THREADS + tid) * 4, last));
    };
    f32x4_t vcur[TS_UNROLL], vnxt[TS_UNROLL];
    load(0, vcur);
    for (int base = 0; base < n; base += STEP) {
      load(base + STEP, vnxt);   // unconditional (clamped) so the load count is static; raw data
      uint32_t cur[TS_UNROLL][4];
#pragma unroll
      for (int q = 0; q < TS_UNROLL; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cur[q][e] = base + (q * TS_THREADS + tid) * 4 + e < n ? f2key(vcur[q][e]) : 0u;
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < TS_UNROLL; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = cur[q][e];
          const bool sel = all ? x > KEY_NEG_INF : (x >> s1) > b1;
          const bool cand = !all && fits && (x >> s1) == b1;
          c += (sel ? 1u : 0u) | (cand ? 0x10000u : 0u);
        }
      const uint32_t inc = wave_scan_dpp(c);
      const uint32_t tot = wave_bcast(inc, 63);
      uint32_t sb = 0, cb = 0;
      if (lane == 0 && tot) {
        if (tot & 0xFFFFu) sb = atomicAdd(&cnt[0], tot & 0xFFFFu);
        if (tot >> 16) cb = atomicAdd(&cnt[1], tot >> 16);
      }
      sb = wave_bcast(sb, 0) + ((inc - c) & 0xFFFFu);
      cb = wave_bcast(cb, 0) + ((inc - c) >> 16);
#pragma unroll
      for (int q = 0; q < TS_UNROLL; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = cur[q][e];
          const int i = base + (q * TS_THREADS + tid) * 4 + e;
          if (all ? x > KEY_NEG_INF : (x >> s1) > b1) emit(sb++, i, x);
          else if (!all && fits && (x >> s1) == b1) {
            ckey[cb] = x;
            cidx[cb] = (uint32_t)i;
            ++cb;
          }
        }
#pragma unroll
      for (int q = 0; q < TS_UNROLL; ++q) vcur[q] = vnxt[q];
    }
  }
  __syncthreads();

  if (kk > 0 && !all) {
    // re-reads of the row when bin b1 does not fit: 16-byte loads clamped into the row's
    // allocation, four per thread in flight, f(key) for every slot below n
    const int lastf = (int)a.score_stride - 4;
    auto sweep = [&](auto f) {
      constexpr int FU = 4;
      for (int base = 0; base < n; base += TS_THREADS * 4 * FU) {
        f32x4_t v[FU];
#pragma unroll
        for (int q = 0; q < FU; ++q)
          v[q] = *reinterpret_cast<const f32x4_t*>(srow + min(base + (q * TS_THREADS + tid) * 4, lastf));
#pragma unroll
        for (int q = 0; q < FU; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (base + (q * TS_THREADS + tid) * 4 + e < n) f(f2key(v[q][e]));
      }
    };
    // exact k-th key T among the slots of bin b1, and how many slots equal to T are kept
    uint32_t need = kk - above;
    const uint32_t nc = min(cnt[1], (uint32_t)TS_CAND);     // == c1 when it fits
    for (int i = tid; i < 2048; i += TS_THREADS) hist[i] = 0u;
    __syncthreads();
    if (fits) {
      for (uint32_t j = tid; j < nc; j += TS_THREADS) atomicAdd(&hist[(ckey[j] >> 10) & m2], 1u);
    } else {
      sweep([&](uint32_t x) {
        if ((x >> s1) == b1) atomicAdd(&hist[(x >> 10) & m2], 1u);
      });
    }
    __syncthreads();
    if (wave == 0) {
      int b2;
      uint32_t ab;
      wave_hist_find(hist, 1 << d2, need, &b2, &ab);
      if (lane == 0) {
        bcv[0] = (uint32_t)b2;
        bcv[1] = ab;
      }
    }
    __syncthreads();
    const uint32_t pre = (b1 << d2) | bcv[0];    // key >> 10 of the k-th key
    need -= bcv[1];
    __syncthreads();
    for (int i = tid; i < 1024; i += TS_THREADS) hist[i] = 0u;
    __syncthreads();
    if (fits) {
      for (uint32_t j = tid; j < nc; j += TS_THREADS)
        if ((ckey[j] >> 10) == pre) atomicAdd(&hist[ckey[j] & 0x3FFu], 1u);
    } else {
      sweep([&](uint32_t x) {
        if ((x >> 10) == pre) atomicAdd(&hist[x & 0x3FFu], 1u);
      });
    }
    __syncthreads();
    if (wave == 0) {
      int b3;
      uint32_t ab;
      wave_hist_find(hist, 1024, need, &b3, &ab);
      if (lane == 0) {
        bcv[0] = (pre << 10) | (uint32_t)b3;
        bcv[1] = need - ab;
        bcv[2] = hist[b3];
      }
    }
    __syncthreads();
    const uint32_t T = bcv[0], need_eq = bcv[1], n_eq = bcv[2];
    if (fits) {
      // candidates: keys above T are kept; of those equal to T, the need_eq lowest slots
      for (uint32_t j0 = 0; j0 < nc; j0 += TS_THREADS) {
        const uint32_t j = j0 + tid;
        bool sel = false;
        uint32_t x = 0;
        int i = 0;
        if (j < nc) {
          x = ckey[j];
          i = (int)cidx[j];
          if (x > T) {
            sel = true;
          } else if (x == T) {
            if (n_eq == need_eq) {
              sel = true;
            } else {
              uint32_t rank = 0;
              for (uint32_t q = 0; q < nc; ++q) rank += (ckey[q] == T && cidx[q] < (uint32_t)i) ? 1u : 0u;
              sel = rank < need_eq;
            }
          }
        }
        const uint64_t m = __ballot(sel);
        uint32_t pb = 0;
        if (lane == 0 && m) pb = atomicAdd(&cnt[0], (uint32_t)__popcll(m));
        pb = wave_bcast(pb, 0);
        if (sel) emit(pb + lanes_below(m), i, x);
      }
    } else {
      // keys of bin b1 above T are kept; equal ones by ascending slot: wave w takes a
      // contiguous slot range (a multiple of 256 slots, 4 consecutive slots per lane and step),
      // counts its equal keys, then takes its share of need_eq
      const int chunk = ((n + TS_WAVES - 1) / TS_WAVES + 255) & ~255;
      const int s0 = min(n, wave * chunk), e0 = min(n, s0 + chunk);
      auto keys4 = [&](int i0, uint32_t (&x)[4]) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(srow + min(i0 + 4 * lane, lastf));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = i0 + 4 * lane + e < e0 ? f2key(v[e]) : 0u;
      };
      uint32_t ce = 0;
      for (int i0 = s0; i0 < e0; i0 += 256) {
        uint32_t x[4];
        keys4(i0, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) ce += x[e] == T ? 1u : 0u;
      }
      ce = wave_bcast(wave_scan_dpp(ce), 63);
      if (lane == 0) weq[wave] = ce;
      __syncthreads();
      uint32_t eb = 0;
      for (int w = 0; w < wave; ++w) eb += weq[w];
      for (int i0 = s0; i0 < e0; i0 += 256) {
        uint32_t x[4];
        keys4(i0, x);
        uint32_t eqc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) eqc += x[e] == T ? 1u : 0u;
        const uint32_t einc = wave_scan_dpp(eqc);
        uint32_t rk = eb + einc - eqc;                   // rank of this lane's first equal slot
        bool sel[4];
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool eq = x[e] == T;
          sel[e] = ((x[e] >> s1) == b1 && x[e] > T) || (eq && rk < need_eq);
          rk += eq ? 1u : 0u;
          c += sel[e] ? 1u : 0u;
        }
        const uint32_t inc = wave_scan_dpp(c);
        const uint32_t tot = wave_bcast(inc, 63);
        uint32_t pb = 0;
        if (lane == 0 && tot) pb = atomicAdd(&cnt[0], tot);
        pb = wave_bcast(pb, 0) + inc - c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (sel[e]) emit(pb, i0 + 4 * lane + e, x[e]);
          pb += sel[e] ? 1u : 0u;
        }
        eb += wave_bcast(einc, 63);
      }
    }
  }
  __syncthreads();
  const int staged = min((int)kk, TS_OUT);
  if constexpr (MAPM == MAP_IDENT) {
    for (int p = tid; p < staged; p += TS_THREADS) {
      oidx[p] = obi[p];
      if (osc) osc[p] = obs[p];
    }
  } else {
    // every mapped token of a thread is loaded before its first store (the compiler keeps a load
    // after a store it cannot prove distinct, so interleaved loads would pay their latencies one
    // after another)
    constexpr int FL = (TS_OUT + TS_THREADS - 1) / TS_THREADS;
    int fk[FL];
#pragma unroll
    for (int u = 0; u < FL; ++u) {
      const int p = tid + u * TS_THREADS;
      fk[u] = p < staged ? map_key(obi[p]) : 0;
    }
#pragma unroll
    for (int u = 0; u < FL; ++u) {
      const int p = tid + u * TS_THREADS;
      if (p < staged) {
        oidx[p] = fk[u];
        if (osc) osc[p] = obs[p];
      }
    }
  }
  for (int p = (int)kk + tid; p < a.k; p += TS_THREADS) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
  if (a.out_count && tid == 0) a.out_count[orow] = (int32_t)kk;
}

// Ascending sort of the first count[row] entries of each row (bitonic, in LDS), for candidate
// lists that later stages index by slot.
__global__ void __launch_bounds__(256) sort_rows_kernel(int32_t* rows, int stride, const int32_t* count,
                                                        int pow2) {
  extern __shared__ int32_t sv[];
  const int r = blockIdx.x;
  int32_t* row = rows + (int64_t)r * stride;
  const int c = count[r];
  for (int i = threadIdx.x; i < pow2; i += blockDim.x) sv[i] = i < c ? row[i] : INT32_MAX;
  __syncthreads();
  for (int size = 2; size <= pow2; size <<= 1)
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < pow2; i += blockDim.x) {
        const int l = i ^ j;
        if (l > i) {
          const bool up = (i & size) == 0;
          const int32_t x = sv[i], y = sv[l];
          if ((x > y) == up) {
            sv[i] = y;
            sv[l] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < c; i += blockDim.x) row[i] = sv[i];
}

// Ascending order of rows of DISTINCT values in [0, max_value): the values become bits of an LDS
// bitmap, and each thread writes the set bits of its contiguous range of words at its exclusive
// prefix of the popcounts. One pass over the row and one over the bitmap.
// STAGE: the sorted row is assembled in LDS after the bitmap and written out coalesced (each
// thread's values are contiguous in the output, so direct stores scatter a wave's writes over 64
// cache lines)
template <bool STAGE>
__global__ void __launch_bounds__(256) sort_rows_bitmap_kernel(int32_t* rows, int stride, const int32_t* count,
                                                               int nwords, int cap) {
  extern __shared__ uint32_t bm[];
  int32_t* stg = reinterpret_cast<int32_t*>(bm + nwords);   // [cap] when STAGE
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  int32_t* row = rows + (int64_t)r * stride;
  const int c = min(count[r], cap);          // a row holds at most cap values
  for (int i = tid; i < nwords; i += 256) bm[i] = 0u;
  __syncthreads();
  for (int i = tid; i < c; i += 256) {
    const uint32_t v = (uint32_t)row[i];
    atomicOr(&bm[v >> 5], 1u << (v & 31u));
  }
  __syncthreads();
  const int per = (nwords + 255) / 256;
  const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  const uint32_t inc = wave_scan_dpp(cnt);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pos = inc - cnt;
  for (int w = 0; w < wave; ++w) pos += wsum[w];
  int32_t* dst = STAGE ? stg : row;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bm[w];
    while (m) {
      dst[pos++] = w * 32 + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
  if constexpr (STAGE) {
    __syncthreads();
    for (int i = tid; i < c; i += 256) row[i] = stg[i];
  }
}

hipError_t launch_sort_rows(int32_t* rows, int stride, const int32_t* count, int n_rows, int max_count,
                            int max_value, hipStream_t s) {
  if (n_rows <= 0 || max_count <= 1) return hipSuccess;
  const int nwords = (max_value + 31) / 32;
  if (max_value > 0 && nwords <= 32768) {
    const size_t staged = ((size_t)nwords + (size_t)max_count) * sizeof(uint32_t);
    if (staged <= 65536) {
      hipLaunchKernelGGL(sort_rows_bitmap_kernel<true>, dim3(n_rows), dim3(256), staged, s, rows, stride, count,
                         nwords, max_count);
      return hipGetLastError();
    }
    const size_t lds = (size_t)nwords * sizeof(uint32_t);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sort_rows_bitmap_kernel<false>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sort_rows_bitmap_kernel<false>, dim3(n_rows), dim3(256), lds, s, rows, stride, count, nwords,
                       max_count);
    return hipGetLastError();
  }
  int pow2 = 1;
  while (pow2 < max_count) pow2 <<= 1;
  const size_t lds = (size_t)pow2 * sizeof(int32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sort_rows_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sort_rows_kernel, dim3(n_rows), dim3(256), lds, s, rows, stride, count, pow2);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int max_row_len, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if ((a.score_stride & 3) != 0 || (reinterpret_cast<uintptr_t>(a.scores) & 15) != 0)
    return hipErrorInvalidValue;                 // rows must allow 16-byte loads
  dim3 g(a.n_rows);
  // rows of up to 4096 slots: the register selector, even with a summary (paired runs on the
  // given-set refine's 4096-slot rows: 0.19 against 0.25 ms; at 8192 slots the summary's single
  // streaming pass is faster, 1.29 against 1.49 ms on the group refine)
  if (a.row_meta && max_row_len > 4096) {
    const dim3 b(TS_THREADS);
    if (a.k <= TS_OUT) {
      if (a.map_mode == MAP_IDENT) hipLaunchKernelGGL((topk_stream_kernel<MAP_IDENT, false>), g, b, 0, s, a);
      else if (a.map_mode == MAP_LIST) hipLaunchKernelGGL((topk_stream_kernel<MAP_LIST, false>), g, b, 0, s, a);
      else hipLaunchKernelGGL((topk_stream_kernel<MAP_BLOCKS, false>), g, b, 0, s, a);
    } else {
      if (a.map_mode == MAP_IDENT) hipLaunchKernelGGL((topk_stream_kernel<MAP_IDENT, true>), g, b, 0, s, a);
      else if (a.map_mode == MAP_LIST) hipLaunchKernelGGL((topk_stream_kernel<MAP_LIST, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((topk_stream_kernel<MAP_BLOCKS, true>), g, b, 0, s, a);
    }
    return hipGetLastError();
  }
  const int m = max_row_len;
  if (m <= 1024) hipLaunchKernelGGL((topk_reg_kernel<4, 1>), g, dim3(256), 0, s, a);
  else if (m <= 2048) hipLaunchKernelGGL((topk_reg_kernel<4, 2>), g, dim3(256), 0, s, a);
  else if (m <= 4096) hipLaunchKernelGGL((topk_reg_kernel<4, 4>), g, dim3(256), 0, s, a);
  // rows of 4K-16K slots: 8 waves of 4 or 8 steps (16 resident waves per CU; 4 waves of 8 or 16
  // steps need twice the registers per lane and leave 8)
  else if (m <= 8192) hipLaunchKernelGGL((topk_reg_kernel<8, 4>), g, dim3(512), 0, s, a);
  else if (m <= 16384) hipLaunchKernelGGL((topk_reg_kernel<8, 8>), g, dim3(512), 0, s, a);
  else if (m <= 32768) hipLaunchKernelGGL((topk_reg_kernel<8, 16>), g, dim3(512), 0, s, a);
  else hipLaunchKernelGGL(topk_long_kernel, g, dim3(TK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
