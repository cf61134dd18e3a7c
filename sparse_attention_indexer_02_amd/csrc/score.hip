// Indexer score kernel for prefill-shaped work (many queries per sequence): the q.k contraction
// over heads on MFMA, with ReLU and the head-weighted sum fused in registers, causal masking
// per tile, one fp32 score written per (query, slot).
//
// Work-group = one tile of up to 8 consecutive queries of one sequence (one query per wave);
// it streams the key set through LDS in tiles of 64 keys (double-buffered, XOR-swizzled 16-byte
// chunks so that the 32 key rows a wave reads per step hit distinct banks), and each wave runs
// the 64 keys x H heads x D contraction for its own query with the query's fragments held in
// registers. Tiles are dispatched heaviest (longest causal prefix) first.
//
// Score: I[t,s] = sum_h w[t,h] * max(q[t,h].k[s], 0) (DeepSeek Sparse Attention's lightning
// indexer, on which the ADIndex, Multi-layer Indexer, PIVOT, HISA and LatentIndex pages all
// build). FP8 keys carry one fp32 scale per token; because the scale is positive it factors out
// of the ReLU and the head sum, so it is applied once per key after the reduction.
#include "score_tile.h"

namespace idx {

template <class Mma, int D, int HB, int KST>
__global__ void __launch_bounds__(WavesFor<HB>::value * 64)
score_kernel(ScoreArgs a) {
  constexpr int NW = WavesFor<HB>::value;
  constexpr int NTHR = NW * 64;
  typedef Geo<Mma, D> G;
  typedef TileLoader<Mma, D, KST, NTHR> Loader;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tiles = smem;
  int32_t* skey = reinterpret_cast<int32_t*>(smem + 2 * G::TILE_BYTES);   // [2][KEY_TILE]
  float* sscale = reinterpret_cast<float*>(skey + 2 * KEY_TILE);           // [2][KEY_TILE]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lin = gridDim.x - 1 - blockIdx.x;       // heaviest tiles first
  const int b = lin % a.B;
  const int ti = lin / a.B;
  const bool list_mode = a.mode == MODE_LIST;

  int tb, te, lrow = 0, row0;
  if (!list_mode) {
    tb = a.c0 + ti * NW;
    te = min(tb + NW, a.c1);
    row0 = a.c0;
  } else {
    const int tpg = (a.group_size + NW - 1) / NW;
    const int g = a.c0 + ti / tpg, sub = ti % tpg;
    tb = g * a.group_size + sub * NW;
    te = min(min(tb + NW, g * a.group_size + a.group_size), a.T);
    lrow = b * a.n_groups + g;
    row0 = a.c0 * a.group_size;
  }

  const int kl = a.k_len ? max(0, min(a.k_len[b], a.tok_cap)) : a.tok_cap;
  const int nkeys_seq = (kl + a.count_div - 1) / a.count_div;
  auto count_of = [&](int pos) -> int {
    return pos < 0 ? 0 : min(nkeys_seq, pos / a.pos_stride + 1);
  };

  const int t = tb + wave;
  const bool active = t < te;
  const int my_pos = active ? a.q_pos[(int64_t)b * a.T + t] : -1;
  int my_count, key_end;
  if (!list_mode) {
    my_count = active ? count_of(my_pos) : 0;
    key_end = 0;
    for (int u = tb; u < te; ++u) key_end = max(key_end, count_of(a.q_pos[(int64_t)b * a.T + u]));
  } else {
    key_end = a.list_len[lrow];
    my_count = key_end;
  }
  if (blockIdx.y == 0 && active && lane == 0)
    a.row_len[(int64_t)b * a.rows_per_seq + (t - row0)] = my_count;

  const int kb0 = blockIdx.y * a.split_keys;
  const int kb1 = min(key_end, kb0 + a.split_keys);
  if (kb0 >= kb1) return;                           // uniform over the work-group

  // query fragments and head weights of this wave's query
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
                            (((int64_t)b * a.T + (ok ? t : 0)) * a.H + (ok ? head : 0)) * D * qeb;
#pragma unroll
      for (int kk = 0; kk < G::NKK; ++kk) {
        if (ok) qf[hb][kk] = load_frag<Mma>(qrow, a.q_dtype, hh * (D / 2) + kk * Mma::E);
        else qf[hb][kk] = typename Mma::frag_t{};
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = acc_head(hb, r, lane);
        wv[hb][r] = (active && h < a.H) ? a.w[((int64_t)b * a.T + t) * a.H + h] : 0.f;
      }
    }
  }

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)b * a.key_cap * (D * Loader::SRC_EB);
  auto key_at = [&](int base, int n) -> int {
    const int j = base + n;
    if (j >= kb1) return -1;
    return list_mode ? a.list[(int64_t)lrow * a.list_stride + j] : j;
  };
  auto scale_of = [&](int ki) -> float {
    if constexpr (KST == DT_FP8) return ki >= 0 ? a.k_scale[(int64_t)b * a.key_cap + ki] : 0.f;
    else return 1.f;
  };

  Loader ld;
  const int ntile = (kb1 - kb0 + KEY_TILE - 1) / KEY_TILE;
  ld.load(kseq, tid, [&](int n) { return key_at(kb0, n); });
  if (tid < KEY_TILE) {
    const int ki = key_at(kb0, tid);
    skey[tid] = ki;
    sscale[tid] = scale_of(ki);
  }
  ld.store(tiles, tid);
  __syncthreads();

  float* srow = a.scores + ((int64_t)b * a.rows_per_seq + (active ? t - row0 : 0)) * a.score_stride;

  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1;
    const int base = kb0 + it * KEY_TILE;
    const bool more = it + 1 < ntile;
    int nki = -1;
    float nsc = 0.f;
    if (more) {
      ld.load(kseq, tid, [&](int n) { return key_at(base + KEY_TILE, n); });
      if (tid < KEY_TILE) {
        nki = key_at(base + KEY_TILE, tid);
        nsc = scale_of(nki);
      }
    }
    if (active && base < my_count) {
      const uint8_t* tile = tiles + cur * G::TILE_BYTES;
#pragma unroll
      for (int sub = 0; sub < KEY_TILE / 32; ++sub) {
        const int sbase = base + sub * 32;
        if (sbase >= my_count || sbase >= kb1) break;
        f32x16_t acc[HB];
        tile_mma<Mma, D, HB>(qf, tile, sub * 32, lane, acc);
        const float tot = tile_epilogue<HB>(acc, wv);
        if (lane < 32) {
          const int j = sbase + lane;
          const int n = sub * 32 + lane;
          if (j < kb1 && j < my_count) {
            float v = tot;
            if constexpr (KST == DT_FP8) v *= sscale[cur * KEY_TILE + n];
            if (list_mode && skey[cur * KEY_TILE + n] > my_pos) v = -INFINITY;
            srow[j] = v;
          }
        }
      }
    }
    if (more) {
      ld.store(tiles + (cur ^ 1) * G::TILE_BYTES, tid);
      if (tid < KEY_TILE) {
        skey[(cur ^ 1) * KEY_TILE + tid] = nki;
        sscale[(cur ^ 1) * KEY_TILE + tid] = nsc;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// host dispatch

bool score_supported(int q_dtype, int k_dtype, int H, int D) {
  if (!(D == 32 || D == 64 || D == 128)) return false;
  if (H < 1 || H > 128) return false;
  if (q_dtype != DT_F32 && q_dtype != DT_BF16) return false;
  if (k_dtype != DT_F32 && k_dtype != DT_BF16 && k_dtype != DT_FP8) return false;
  return true;
}

template <class Mma, int D, int HB, int KST>
static hipError_t launch_one(const ScoreArgs& a, int n_splits, hipStream_t s) {
  constexpr int NW = WavesFor<HB>::value;
  typedef Geo<Mma, D> G;
  const size_t lds = 2 * G::TILE_BYTES + 4 * KEY_TILE * sizeof(int32_t);
  auto kfn = score_kernel<Mma, D, HB, KST>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.B * a.tiles_per_seq, n_splits);
  hipLaunchKernelGGL(kfn, grid, dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <class Mma, int KST>
static hipError_t launch_dh(const ScoreArgs& a, int n_splits, hipStream_t s) {
  const int HB = (a.H + 31) / 32;
#define IDX_CASE(DD, HH)                                                         \
  if (a.D == DD && HB <= HH) return launch_one<Mma, DD, HH, KST>(a, n_splits, s);
#define IDX_DCASES(DD) IDX_CASE(DD, 1) IDX_CASE(DD, 2) IDX_CASE(DD, 4)
  IDX_DCASES(32) IDX_DCASES(64) IDX_DCASES(128)
#undef IDX_DCASES
#undef IDX_CASE
  return hipErrorInvalidValue;
}

int score_queries_per_tile(int H) { return (H <= 64) ? 8 : 4; }

hipError_t launch_score(const ScoreArgs& a, int n_splits, hipStream_t s) {
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_BF16) return launch_dh<MmaBf16, DT_BF16>(a, n_splits, s);
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_FP8) return launch_dh<MmaBf16, DT_FP8>(a, n_splits, s);
  if (a.k_dtype == DT_F32) return launch_dh<MmaF32, DT_F32>(a, n_splits, s);
  if (a.k_dtype == DT_BF16) return launch_dh<MmaF32, DT_BF16>(a, n_splits, s);
  return launch_dh<MmaF32, DT_FP8>(a, n_splits, s);
}

}  // namespace idx
