// Token-level refine of the hierarchical (block-pooled) indexer: each query scores only the
// tokens of the blocks it kept in the coarse stage, with the unchanged indexer score ("HISA:
// Efficient Hierarchical Indexing for Fine-Grained Sparse Attention", abstract: the token-level
// stage runs the original indexer inside the retained candidate blocks).
//
// A work-group takes a tile of consecutive queries (8, or 4 in the direct bf16 kernel, whose
// work-groups run two per CU). Adjacent queries keep mostly the same blocks, so the group forms
// the union of their kept blocks (LDS bitmap + prefix popcounts),
// streams each union block's keys through LDS once, and every wave runs the MFMA tile only for
// 32-key steps that hold at least one of its own blocks. Score slot of query t for token
// o of its p-th kept block = p * block_size + o; tokens past the cache end or past the query's
// position get -inf.
#include "score_tile.h"

namespace idx {

// Waits until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ITERS loads of 16 bytes per lane: load i reads base + i STEP into the 1 KB LDS block
// (i NW + wave) of dst (lane l writing bytes 16 l .. 16 l + 15 of it)
template <int ITERS, int STEP, int NW>
__device__ __forceinline__ void load_rows_lds(const uint8_t* base, uint8_t* dst, int wave) {
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
    __builtin_amdgcn_global_load_lds(base + i * STEP,
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(dst + (i * NW + wave) * 1024)),
                                     16, 0, 0);
}

constexpr int BR_UMAX = 2048;        // union blocks handled per round
constexpr int BR_NBW = 2048;         // bitmap words: blocks per sequence <= 65536
constexpr int BRD_UMAX = 1024;       // union blocks per round of the direct kernel

template <class Mma, int D, int HB, int KST>
__global__ void __launch_bounds__(WavesFor<HB>::value * 64)
block_refine_kernel(BlockRefineArgs a) {
  constexpr int NW = WavesFor<HB>::value;
  constexpr int NTHR = NW * 64;
  typedef Geo<Mma, D, KEY_TILE> G;
  typedef TileLoader<Mma, D, KST, NTHR, KEY_TILE> Loader;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tiles = smem;
  int16_t* pos_tab = reinterpret_cast<int16_t*>(smem + 2 * G::TILE_BYTES);   // [NW][UMAX]
  int32_t* ublk = reinterpret_cast<int32_t*>(pos_tab + NW * BR_UMAX);        // [UMAX]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ublk + BR_UMAX);            // [NBW]
  uint32_t* wpre = bitmap + BR_NBW;                                          // [NBW]
  uint32_t* sh = wpre + BR_NBW;                                              // [80]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lin = gridDim.x - 1 - blockIdx.x;
  const int b = lin % a.B;
  const int ti = lin / a.B;
  const int tb = a.t0 + ti * NW, te = min(tb + NW, a.t1);
  const int t = tb + wave;
  const bool active = t < te;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int Bs = a.block_size;
  const int NB = (kl + Bs - 1) / Bs;
  const int NBW = (NB + 31) / 32;
  const int64_t qrow_i = (int64_t)b * a.T + (active ? t : tb);
  const int my_pos = active ? a.q_pos[qrow_i] : -1;
  const int nk = active ? a.n_kept[qrow_i] : 0;
  const int32_t* mylist = a.blocks + qrow_i * a.keep_stride;
  if (active && lane == 0) a.row_len[(int64_t)b * a.rows_per_seq + (t - a.t0)] = nk * Bs;

  // union of the tile's kept blocks
  for (int i = tid; i < NBW; i += NTHR) bitmap[i] = 0u;
  __syncthreads();
  for (int p = lane; p < nk; p += 64) {
    const int blk = mylist[p];
    atomicOr(&bitmap[blk >> 5], 1u << (blk & 31));
  }
  __syncthreads();
  uint32_t n_union;
  {
    const int per = (NBW + NTHR - 1) / NTHR;
    const int w0 = tid * per;
    uint32_t c = 0;
    for (int i = 0; i < per; ++i)
      if (w0 + i < NBW) c += __popc(bitmap[w0 + i]);
    // exclusive scan over the work-group
    const uint32_t inc = wave_incl_scan(c);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (wave == 0) {
      const uint32_t s = lane < NW ? sh[lane] : 0u;
      const uint32_t si = wave_incl_scan(s);
      if (lane < NW) sh[32 + lane] = si - s;
      if (lane == 63) sh[64] = si;
    }
    __syncthreads();
    uint32_t run = sh[32 + wave] + inc - c;
    for (int i = 0; i < per; ++i)
      if (w0 + i < NBW) {
        wpre[w0 + i] = run;
        run += __popc(bitmap[w0 + i]);
      }
    n_union = sh[64];
    __syncthreads();
  }

  typename Mma::frag_t qf[HB][G::NKK];
  float wv[HB][16];
  {
    const int hh = lane >> 5, ln = lane & 31;
    const int qeb = dtype_bytes(a.q_dtype);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 32 * hb + ln;
      const bool ok = active && head < a.H;
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                            (qrow_i * a.H + (ok ? head : 0)) * D * qeb;
#pragma unroll
      for (int kk = 0; kk < G::NKK; ++kk) {
        if (ok) qf[hb][kk] = load_frag<Mma>(qrow, a.q_dtype, hh * (D / 2) + kk * Mma::E);
        else qf[hb][kk] = typename Mma::frag_t{};
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = acc_head(hb, r, lane);
        wv[hb][r] = (active && h < a.H) ? a.w[qrow_i * a.H + h] : 0.f;
      }
    }
  }

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)b * a.N * (D * Loader::SRC_EB);
  float* srow = a.scores + ((int64_t)b * a.rows_per_seq + (active ? t - a.t0 : 0)) * a.score_stride;

  for (uint32_t rb = 0; rb < n_union; rb += BR_UMAX) {
    const int rcount = (int)min((uint32_t)BR_UMAX, n_union - rb);
    // union list of this round and this wave's slot table
    {
      const int per = (NBW + NTHR - 1) / NTHR;
      const int w0 = tid * per;
      for (int i = 0; i < per; ++i) {
        const int wi = w0 + i;
        if (wi >= NBW) break;
        uint32_t m = bitmap[wi];
        uint32_t u = wpre[wi];
        while (m) {
          const int bit = __builtin_ctz(m);
          m &= m - 1;
          if (u >= rb && u < rb + (uint32_t)rcount) ublk[u - rb] = wi * 32 + bit;
          ++u;
        }
      }
      for (int i = tid; i < NW * rcount; i += NTHR) pos_tab[(i / rcount) * BR_UMAX + i % rcount] = -1;
    }
    __syncthreads();
    for (int p = lane; p < nk; p += 64) {
      const int blk = mylist[p];
      const uint32_t u = wpre[blk >> 5] + __popc(bitmap[blk >> 5] & ((1u << (blk & 31)) - 1u));
      if (u >= rb && u < rb + (uint32_t)rcount) pos_tab[wave * BR_UMAX + (u - rb)] = (int16_t)p;
    }
    __syncthreads();

    const int nslots = rcount * Bs;
    auto key_at = [&](int base, int n) -> int {
      const int v = base + n;
      if (v >= nslots) return -1;
      const int key = ublk[v / Bs] * Bs + v % Bs;
      return key < kl ? key : -1;
    };
    Loader ld;
    const int ntile = (nslots + KEY_TILE - 1) / KEY_TILE;
    ld.load(kseq, tid, [&](int n) { return key_at(0, n); });
    ld.store(tiles, tid);
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
      const int cur = it & 1;
      const int base = it * KEY_TILE;
      const bool more = it + 1 < ntile;
      if (more) ld.load(kseq, tid, [&](int n) { return key_at(base + KEY_TILE, n); });
#pragma unroll
      for (int sub = 0; sub < KEY_TILE / 32; ++sub) {
        const int sb = base + sub * 32;
        if (sb >= nslots) break;
        const int v = sb + (lane & 31);
        const int u = v / Bs, o = v % Bs;
        const int mem = (lane < 32 && v < nslots) ? pos_tab[wave * BR_UMAX + u] : -1;
        if (active && __ballot(mem >= 0) != 0ull) {
          f32x16_t acc[HB];
          tile_mma<Mma, D, HB, KEY_TILE>(qf, tiles + cur * G::TILE_BYTES, sub * 32, lane, acc);
          const float tot = tile_epilogue<HB>(acc, wv);
          if (mem >= 0) {
            const int key = ublk[u] * Bs + o;
            srow[mem * Bs + o] = (key < kl && key <= my_pos) ? tot : -INFINITY;
          }
        }
      }
      if (more) ld.store(tiles + (cur ^ 1) * G::TILE_BYTES, tid);
      __syncthreads();
    }
  }
}

// bf16 keys and queries: the union's key rows stream straight into LDS (global_load_lds, 128-key
// tiles in a ring of NBUF buffers, loads issued NBUF - 1 tiles ahead: the union's blocks are
// scattered over the cache, so a tile's rows come from L2, the MALL or HBM with a latency longer
// than one tile's MFMA work) and a wave that owns all four 32-key steps of a tile runs them
// pipelined (the epilogue of one step under the MFMAs of the next, the next step's fragments read
// during the current step), as the dense score kernel does; partly owned tiles run step by step.
template <int D, int HB, int NBUF, bool BIG, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(8 / NW)))
block_refine_direct_kernel(BlockRefineArgs a) {
  constexpr int NTHR = NW * 64;
  constexpr int KT = 128;
  constexpr int NSUB = KT / 32;
  constexpr int DIST = NBUF - 1;                    // tiles in flight ahead of the one in use
  static_assert(NBUF == 2 || NBUF == 3, "ring of two or three tiles");
  typedef Geo<MmaBf16, D, KT> G;
  typedef DirectLoader<MmaBf16, D, NTHR, KT> DLoader;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tiles = smem;
  // the bitmap holds the sequence's blocks: (ceil(N / Bs) + 31) / 32 words, sized at launch
  const int nbw_cap = ((a.N + a.block_size - 1) / a.block_size + 31) / 32;
  int16_t* pos_tab = reinterpret_cast<int16_t*>(smem + NBUF * G::TILE_BYTES);   // [NW][BRD_UMAX]
  int32_t* ublk = reinterpret_cast<int32_t*>(pos_tab + NW * BRD_UMAX);       // [BRD_UMAX]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ublk + BRD_UMAX);           // [nbw_cap]
  uint32_t* wpre = bitmap + nbw_cap;                                         // [nbw_cap]
  uint32_t* sh = wpre + nbw_cap;                                             // [80]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lin = gridDim.x - 1 - blockIdx.x;
  const int b = lin % a.B;
  const int ti = lin / a.B;
  const int tb = a.t0 + ti * NW, te = min(tb + NW, a.t1);
  const int t = tb + wave;
  const bool active = t < te;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int Bs = a.block_size;                      // a power of two here
  const int lb = __builtin_ctz((unsigned)Bs);
  const int NB = (kl + Bs - 1) >> lb;
  const int NBW = (NB + 31) / 32;
  const int64_t qrow_i = (int64_t)b * a.T + (active ? t : tb);
  const int my_pos = active ? a.q_pos[qrow_i] : -1;
  const int nk = active ? a.n_kept[qrow_i] : 0;
  const int32_t* mylist = a.blocks + qrow_i * a.keep_stride;
  if (active && lane == 0) a.row_len[(int64_t)b * a.rows_per_seq + (t - a.t0)] = nk * Bs;

  // union of the tile's kept blocks
  for (int i = tid; i < NBW; i += NTHR) bitmap[i] = 0u;
  __syncthreads();
  for (int p = lane; p < nk; p += 64) {
    const int blk = mylist[p];
    atomicOr(&bitmap[blk >> 5], 1u << (blk & 31));
  }
  __syncthreads();
  uint32_t n_union;
  {
    const int per = (NBW + NTHR - 1) / NTHR;
    const int w0 = tid * per;
    uint32_t c = 0;
    for (int i = 0; i < per; ++i)
      if (w0 + i < NBW) c += __popc(bitmap[w0 + i]);
    const uint32_t inc = wave_incl_scan(c);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (wave == 0) {
      const uint32_t s = lane < NW ? sh[lane] : 0u;
      const uint32_t si = wave_incl_scan(s);
      if (lane < NW) sh[32 + lane] = si - s;
      if (lane == 63) sh[64] = si;
    }
    __syncthreads();
    uint32_t run = sh[32 + wave] + inc - c;
    for (int i = 0; i < per; ++i)
      if (w0 + i < NBW) {
        wpre[w0 + i] = run;
        run += __popc(bitmap[w0 + i]);
      }
    n_union = sh[64];
    __syncthreads();
  }

  bf16x8_t qf[HB][G::NKK];
  float wv[HB][16];
  {
    const int hh = lane >> 5, ln = lane & 31;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 32 * hb + ln;
      const bool ok = active && head < a.H;
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + (qrow_i * a.H + (ok ? head : 0)) * D * 2;
#pragma unroll
      for (int kk = 0; kk < G::NKK; ++kk)
        qf[hb][kk] = ok ? load_frag<MmaBf16>(qrow, DT_BF16, hh * (D / 2) + kk * 8) : bf16x8_t{};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = acc_head(hb, r, lane);
        wv[hb][r] = (active && h < a.H) ? a.w[qrow_i * a.H + h] : 0.f;
      }
    }
  }

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.keys) + (int64_t)b * a.N * (D * 2);
  float* srow = a.scores + ((int64_t)b * a.rows_per_seq + (active ? t - a.t0 : 0)) * a.score_stride;

  for (uint32_t rb = 0; rb < n_union; rb += BRD_UMAX) {
    const int rcount = (int)min((uint32_t)BRD_UMAX, n_union - rb);
    {
      const int per = (NBW + NTHR - 1) / NTHR;
      const int w0 = tid * per;
      for (int i = 0; i < per; ++i) {
        const int wi = w0 + i;
        if (wi >= NBW) break;
        uint32_t m = bitmap[wi];
        uint32_t u = wpre[wi];
        while (m) {
          const int bit = __builtin_ctz(m);
          m &= m - 1;
          if (u >= rb && u < rb + (uint32_t)rcount) ublk[u - rb] = wi * 32 + bit;
          ++u;
        }
      }
      for (int i = tid; i < NW * rcount; i += NTHR) pos_tab[(i / rcount) * BRD_UMAX + i % rcount] = -1;
    }
    __syncthreads();
    for (int p = lane; p < nk; p += 64) {
      const int blk = mylist[p];
      const uint32_t u = wpre[blk >> 5] + __popc(bitmap[blk >> 5] & ((1u << (blk & 31)) - 1u));
      if (u >= rb && u < rb + (uint32_t)rcount) pos_tab[wave * BRD_UMAX + (u - rb)] = (int16_t)p;
    }
    __syncthreads();

    const int nslots = rcount * Bs;
    const int ntile = (nslots + KT - 1) / KT;
    bf16x8_t bfr[G::NKK];
    // the four steps of a tile the wave's query owns entirely, pipelined; scores two steps per
    // value: lanes 0-31 hold the even step, lanes 32-63 the odd one
    auto full_tile = [&](const uint8_t* tile, float (&ov)[NSUB / 2]) {
      auto put = [&](int st, float tot) {
        if ((st & 1) == (lane >> 5)) ov[st >> 1] = tot;
      };
      f32x16_t A[HB], Bq[HB];
      load_bfrag<MmaBf16, D, KT>(tile, 0, lane, bfr);
      tile_mma_rot<D, HB, KT>(qf, bfr, tile, 32, true, lane, A);
#pragma unroll
      for (int s = 1; s < NSUB; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        if (s & 1) {
          tile_mma_rot<D, HB, KT>(qf, bfr, tile, (s + 1) * 32, s + 1 < NSUB, lane, Bq);
          put(s - 1, tile_epilogue<HB>(A, wv));
        } else {
          tile_mma_rot<D, HB, KT>(qf, bfr, tile, (s + 1) * 32, s + 1 < NSUB, lane, A);
          put(s - 1, tile_epilogue<HB>(Bq, wv));
        }
#pragma unroll
        for (int kk = 0; kk < G::NKK; ++kk) {
          __builtin_amdgcn_sched_group_barrier(0x008, HB, 0);
          if (s + 1 < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (16 * HB * 2 + 8) / G::NKK + 1, 0);
        }
      }
      put(NSUB - 1, tile_epilogue<HB>(Bq, wv));
    };
    // Ring discipline: tile j lives in buffer j % NBUF; the loads of tile it + DIST are issued at
    // the start of iteration it, into the buffer that every wave finished reading in iteration
    // it - 1 (the barrier ending that iteration). Loads return in issue order, so "at most
    // ITERS outstanding" once the next tile's loads are issued means tile it + 1 has landed.
    if constexpr (BIG) {
      // Blocks of KT keys or more: a tile is KT consecutive keys of one union block, so all it
      // takes is the tile's first key and the block's kept position for this wave's query (-1:
      // not kept). Lane j holds both for tile w0 + j of a 64-tile window, read from LDS once per
      // window; a tile's values are then taken with readlane, with no LDS round trip in the tile
      // loop. Every tile is full (the union's slot count is a multiple of Bs).
      int k0_win = 0, m_win = -1, w0 = 0;
      auto refresh = [&](int first) {
        const int j = first + lane;
        const int v = j * KT;
        k0_win = j < ntile ? (ublk[v >> lb] << lb) + (v & (Bs - 1)) : 0;
        m_win = (active && j < ntile) ? (int)pos_tab[wave * BRD_UMAX + (v >> lb)] : -1;
      };
      // A lane's i-th load fills physical chunk p = (i NW + wave) 64 + lane of the tile: row
      // n_i = i RPI + n_0 and the same logical chunk for every i (the swizzle key repeats every
      // RPI rows), so its source is the tile's first key row + loff0 + i RPI rows.
      constexpr int RPI = NW * 64 / G::CPR;               // tile rows per load round
      static_assert((NW * 64) % G::CPR == 0 && RPI % (1 << G::SWZ_SH) == 0 &&
                        ((RPI >> G::SWZ_SH) % (G::SWZ + 1)) == 0,
                    "the swizzle key repeats every load round");
      const uint32_t loff0 = [&] {
        const int p0 = wave * 64 + lane;
        const int n0 = p0 / G::CPR, cp = p0 % G::CPR;
        return (uint32_t)(n0 * G::ROW_BYTES + ((cp ^ swz<G>(n0)) << 4));
      }();
      auto load_tile = [&](int j, int k0) {
        uint8_t* dst = tiles + (j % NBUF) * G::TILE_BYTES;
        if (k0 + KT <= kl) {
          // every row of the tile is in the cache: one uniform base, no per-row checks
          const uint8_t* base = kseq + (int64_t)k0 * G::ROW_BYTES + loff0;
          load_rows_lds<DLoader::ITERS, RPI * G::ROW_BYTES, NW>(base, dst, wave);
        } else {
          int kx[DLoader::ITERS];
#pragma unroll
          for (int i = 0; i < DLoader::ITERS; ++i) {
            const int key = k0 + DLoader::row_of(i, wave, lane);
            kx[i] = key < kl ? key : -1;
          }
          DLoader::load_idx(kseq, dst, wave, lane, kx);
        }
      };
      refresh(0);
#pragma unroll
      for (int j = 0; j < DIST; ++j)
        if (j < ntile) load_tile(j, __builtin_amdgcn_readlane(k0_win, j));
      if (DIST == 2 && ntile > 1) wait_vmem_n<DLoader::ITERS>();
      else wait_vmem();
      lds_barrier();
      for (int it = 0; it < ntile; ++it) {
        const bool more = it + 1 < ntile;
        if (it + DIST >= w0 + 64) {                     // the window covers tiles it .. it + DIST
          w0 = it;
          refresh(w0);
        }
        if (it + DIST < ntile) load_tile(it + DIST, __builtin_amdgcn_readlane(k0_win, it + DIST - w0));
        const int k0_cur = __builtin_amdgcn_readlane(k0_win, it - w0);
        const int m_cur = __builtin_amdgcn_readlane(m_win, it - w0);
        float ov[NSUB / 2];
        if (m_cur >= 0) full_tile(tiles + (it % NBUF) * G::TILE_BYTES, ov);
        if (DIST == 2 && it + 2 < ntile) wait_vmem_n<DLoader::ITERS>();
        else if (more) wait_vmem();
        if (m_cur >= 0) {
          const int sbase = (m_cur << lb) + ((it * KT) & (Bs - 1));
#pragma unroll
          for (int p = 0; p < NSUB / 2; ++p) {
            const int o = (2 * p + (lane >> 5)) * 32 + (lane & 31);
            const int key = k0_cur + o;
            srow[sbase + o] = (key < kl && key <= my_pos) ? ov[p] : -INFINITY;
          }
        }
        lds_barrier();
      }
      continue;
    }
    auto key_at = [&](int v) -> int {                // key of union slot v, or -1
      if (v >= nslots) return -1;
      const int key = (ublk[v >> lb] << lb) + (v & (Bs - 1));
      return key < kl ? key : -1;
    };
    int kidx[DLoader::ITERS];
    auto fetch_idx = [&](int base) {
#pragma unroll
      for (int i = 0; i < DLoader::ITERS; ++i) kidx[i] = key_at(base + DLoader::row_of(i, wave, lane));
    };
    {
      // every index is read from LDS before the first load goes out (an LDS read after the
      // loads would wait for them)
      int kj[DIST][DLoader::ITERS];
#pragma unroll
      for (int j = 0; j < DIST; ++j) {
        fetch_idx(j * KT);
#pragma unroll
        for (int i = 0; i < DLoader::ITERS; ++i) kj[j][i] = kidx[i];
      }
      fetch_idx(DIST * KT);
#pragma unroll
      for (int j = 0; j < DIST; ++j)
        if (j < ntile) DLoader::load_idx(kseq, tiles + j * G::TILE_BYTES, wave, lane, kj[j]);
    }
    if (DIST == 2 && ntile > 1) wait_vmem_n<DLoader::ITERS>();
    else wait_vmem();
    lds_barrier();
    for (int it = 0; it < ntile; ++it) {
      const int cur = it % NBUF;
      const int base = it * KT;
      const bool more = it + 1 < ntile;
      if (it + DIST < ntile) {
        DLoader::load_idx(kseq, tiles + ((it + DIST) % NBUF) * G::TILE_BYTES, wave, lane, kidx);
        if (it + DIST + 1 < ntile) fetch_idx(base + (DIST + 1) * KT);
      }
      const uint8_t* tile = tiles + cur * G::TILE_BYTES;
      // kept position of a union slot's block for this wave's query, or -1
      auto kept_pos = [&](int v) -> int { return v < nslots ? pos_tab[wave * BRD_UMAX + (v >> lb)] : -1; };
      // steps holding at least one of the query's blocks (lanes l and l + 32 share key l % 32)
      uint32_t own = 0;
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        if (__ballot(kept_pos(base + s * 32 + (lane & 31)) >= 0) != 0ull) own |= 1u << s;
      if (!active) own = 0;
      float ov[NSUB / 2];
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) ov[p] = 0.f;
      if (own == (1u << NSUB) - 1u) {
        full_tile(tile, ov);
      } else {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (own & (1u << s)) {
            f32x16_t acc[HB];
            load_bfrag<MmaBf16, D, KT>(tile, s * 32, lane, bfr);
            tile_mma_rot<D, HB, KT>(qf, bfr, tile, 0, false, lane, acc);
            const float tot = tile_epilogue<HB>(acc, wv);
            if ((s & 1) == (lane >> 5)) ov[s >> 1] = tot;
          }
        }
      }
      // tile it + 1 landed (this wave's share; the barrier below covers the others')
      if (DIST == 2 && it + 2 < ntile) wait_vmem_n<DLoader::ITERS>();
      else if (more) wait_vmem();
      // lanes 0-31 store the even steps, lanes 32-63 the odd ones
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) {
        const int s = 2 * p + (lane >> 5);
        const int slot = base + s * 32 + (lane & 31);
        const int m = kept_pos(slot);
        const float v = ov[p];
        if (m >= 0) {
          const int o = slot & (Bs - 1);
          const int key = (ublk[slot >> lb] << lb) + o;
          srow[(m << lb) + o] = (key < kl && key <= my_pos) ? v : -INFINITY;
        }
      }
      lds_barrier();
    }
  }
}

template <class Mma, int D, int HB, int KST>
static hipError_t launch_br(const BlockRefineArgs& a, hipStream_t s) {
  constexpr int NW = WavesFor<HB>::value;
  typedef Geo<Mma, D, KEY_TILE> G;
  const size_t lds = 2 * G::TILE_BYTES + NW * BR_UMAX * sizeof(int16_t) +
                     BR_UMAX * sizeof(int32_t) + 2 * BR_NBW * sizeof(uint32_t) + 80 * sizeof(uint32_t);
  auto kfn = block_refine_kernel<Mma, D, HB, KST>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kfn, dim3(a.B * a.tiles_per_seq), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <class Mma, int KST>
static hipError_t launch_br_dh(const BlockRefineArgs& a, hipStream_t s) {
  const int HB = (a.H + 31) / 32;
#define IDX_CASE(DD, HH) \
  if (a.D == DD && HB <= HH) return launch_br<Mma, DD, HH, KST>(a, s);
#define IDX_DCASES(DD) IDX_CASE(DD, 1) IDX_CASE(DD, 2) IDX_CASE(DD, 4)
  IDX_DCASES(32) IDX_DCASES(64) IDX_DCASES(128)
#undef IDX_DCASES
#undef IDX_CASE
  return hipErrorInvalidValue;
}

template <int D, int HB, int NBUF, bool BIG, int NW>
static hipError_t launch_brd(const BlockRefineArgs& a0, hipStream_t s) {
  typedef Geo<MmaBf16, D, 128> G;
  BlockRefineArgs a = a0;
  a.tiles_per_seq = (a.t1 - a.t0 + NW - 1) / NW;             // NW queries per work-group
  const size_t nbw_cap = ((size_t)(a.N + a.block_size - 1) / a.block_size + 31) / 32;
  const size_t lds = NBUF * G::TILE_BYTES + NW * BRD_UMAX * sizeof(int16_t) +
                     BRD_UMAX * sizeof(int32_t) + 2 * nbw_cap * sizeof(uint32_t) + 80 * sizeof(uint32_t);
  static_assert(NBUF * G::TILE_BYTES + NW * BRD_UMAX * 2 + BRD_UMAX * 4 + 2 * BR_NBW * 4 + 320 <= 160 * 1024,
                "LDS of one work-group at the largest bitmap");
  auto kfn = block_refine_direct_kernel<D, HB, NBUF, BIG, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(a.B * a.tiles_per_seq), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_block_refine(const BlockRefineArgs& a, hipStream_t s) {
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_BF16) {
    const int HB = (a.H + 31) / 32;
    const bool pow2 = (a.block_size & (a.block_size - 1)) == 0;
    const bool big = a.block_size >= 128;       // blocks of at least one 128-key tile
    if (pow2 && a.D == 128 && HB <= 2)
      return big ? launch_brd<128, 2, 2, true, 4>(a, s) : launch_brd<128, 2, 2, false, 4>(a, s);
    if (pow2 && a.D == 64 && HB <= 2)
      return big ? launch_brd<64, 2, 2, true, 4>(a, s) : launch_brd<64, 2, 2, false, 4>(a, s);
    return launch_br_dh<MmaBf16, DT_BF16>(a, s);
  }
  if (a.k_dtype == DT_F32) return launch_br_dh<MmaF32, DT_F32>(a, s);
  if (a.k_dtype == DT_BF16) return launch_br_dh<MmaF32, DT_BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace idx
