// Token-level refine of the hierarchical (block-pooled) indexer: each query scores only the
// tokens of the blocks it kept in the coarse stage, with the unchanged indexer score ("HISA:
// Efficient Hierarchical Indexing for Fine-Grained Sparse Attention", abstract: the token-level
// stage runs the original indexer inside the retained candidate blocks).
//
// A work-group takes a tile of up to 8 consecutive queries. Adjacent queries keep mostly the same
// blocks, so the group forms the union of their kept blocks (LDS bitmap + prefix popcounts),
// streams each union block's keys through LDS once, and every wave runs the MFMA tile only for
// 32-key steps that hold at least one of its own blocks. Score slot of query t for token
// o of its p-th kept block = p * block_size + o; tokens past the cache end or past the query's
// position get -inf.
#include "score_tile.h"

namespace idx {

constexpr int BR_UMAX = 2048;        // union blocks handled per round
constexpr int BR_NBW = 2048;         // bitmap words: blocks per sequence <= 65536

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

hipError_t launch_block_refine(const BlockRefineArgs& a, hipStream_t s) {
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_BF16) return launch_br_dh<MmaBf16, DT_BF16>(a, s);
  if (a.k_dtype == DT_F32) return launch_br_dh<MmaF32, DT_F32>(a, s);
  if (a.k_dtype == DT_BF16) return launch_br_dh<MmaF32, DT_BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace idx
