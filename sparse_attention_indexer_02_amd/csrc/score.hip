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

template <class Mma, int KST> struct Direct {
  static constexpr bool value = sizeof(Mma) > 0 && Mma::E == 8 && KST == DT_BF16;
};
template <class Mma, int KST> struct TileKeys {
  static constexpr int value = Direct<Mma, KST>::value ? 128 : 64;
};

// One wave selects the top k slots of its own score row (n slots) from the row's 12-bit
// first-digit summary: tot finite slots, bin b1 of the k-th largest key, `above` slots in higher
// bins and `inbin` slots in bin b1. Pass 1 over the row writes the slots above bin b1 and keeps
// the slots of bin b1: when they fit (inbin <= CAP) as (key, slot) pairs in LDS (keys in `ck`,
// 16-bit slots in the upper half of `h`), otherwise as a histogram of their next 10 key bits. The
// k-th key is then resolved digit by digit: 10 more bits give its 22-bit prefix; slots above the
// prefix are written, and the slots sharing it (at most 256) are ranked exactly, higher key first,
// then lower slot (ties keep the lowest slots); a prefix shared by more slots takes a last 10-bit
// digit and keeps the lowest slots equal to the k-th key. Histograms use 1024 words of `h`. Without
// the LDS copy the row is read again from global memory for each step. Row reads are eight
// 16-byte loads per lane at a time. Output order: pass order, slot order within a pass.
template <int CAP>
__device__ __forceinline__ void wave_select_row(const float* srow, int n, int64_t stride, int k,
                                                uint32_t tot, int b1, uint32_t above, uint32_t inbin,
                                                uint32_t* h, uint32_t* ck, int32_t* oidx, float* osc) {
  static_assert(CAP <= 2048, "16-bit slots in 1024 words");
  constexpr int U = 8;
  const int lane = lane_id();
  const uint32_t kk = min((uint32_t)k, tot);
  const bool all = kk == tot;
  const bool gather = !all && inbin <= (uint32_t)CAP;
  uint16_t* cs = reinterpret_cast<uint16_t*>(h + 1024);
  const int last = (int)stride - 4;
  // visits the row 256 slots at a time: f(i0, key[4], v) with key 0 past the row
  auto stream = [&](auto f) {
    for (int i0 = 0; i0 < n; i0 += 256 * U) {
      f32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = *reinterpret_cast<const f32x4_t*>(srow + min(i0 + 256 * u + 4 * lane, last));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j0 = i0 + 256 * u;
        if (j0 >= n) break;
        uint32_t key[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) key[e] = j0 + 4 * lane + e < n ? f2key(v[u][e]) : 0u;
        f(j0, key, v[u]);
      }
    }
  };
  uint32_t pos = 0;
  // writes the slots flagged in sel[4] at pos, in slot order
  auto emit = [&](int i0, const bool (&sel)[4], const f32x4_t& v) {
    const uint32_t c = (sel[0] ? 1u : 0u) + (sel[1] ? 1u : 0u) + (sel[2] ? 1u : 0u) + (sel[3] ? 1u : 0u);
    const uint32_t inc = wave_scan_dpp(c);
    uint32_t p = pos + inc - c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (sel[e]) {
        oidx[p] = i0 + 4 * lane + e;
        if (osc) osc[p] = v[e];
      }
      p += sel[e] ? 1u : 0u;
    }
    pos += wave_bcast(inc, 63);
  };
  // writes one flagged slot per lane at pos, in lane order
  auto emit1 = [&](bool sel, uint32_t slot, uint32_t key) {
    const uint32_t inc = wave_scan_dpp(sel ? 1u : 0u);
    if (sel) {
      oidx[pos + inc - 1] = (int32_t)slot;
      if (osc) osc[pos + inc - 1] = key2f(key);
    }
    pos += wave_bcast(inc, 63);
  };
  auto zero_hist = [&] {
    for (int i = lane; i < 1024; i += 64) h[i] = 0u;
  };
  // ranks the c2 (key, slot) pairs in h[0..256) / h[256..512) and writes the best `need`
  auto rank_emit = [&](uint32_t c2, uint32_t need) {
    for (int j0 = 0; j0 < (int)c2; j0 += 64) {
      const int j = j0 + lane;
      uint32_t kj = 0, sj = 0, r = 0;
      if (j < (int)c2) {
        kj = h[j];
        sj = h[256 + j];
        for (int i = 0; i < (int)c2; ++i) {
          const uint32_t ki = h[i], si = h[256 + i];
          r += (ki > kj || (ki == kj && si < sj)) ? 1u : 0u;
        }
      }
      emit1(j < (int)c2 && r < need, sj, kj);
    }
  };
  const uint32_t ub1 = (uint32_t)b1;
  if (!all && !gather) zero_hist();
  uint32_t cb = 0;                                       // gathered slots
  stream([&](int i0, const uint32_t (&key)[4], const f32x4_t& v) {
    bool sel[4];
    uint32_t ce = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = all ? key[e] > KEY_NEG_INF : (key[e] >> 20) > ub1;
      ce += (key[e] >> 20) == ub1 ? 1u : 0u;
    }
    if (gather) {
      const uint32_t einc = wave_scan_dpp(ce);
      uint32_t p = cb + einc - ce;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((key[e] >> 20) == ub1 && p < (uint32_t)CAP) {   // p < inbin for finite keys
          ck[p] = key[e];
          cs[p] = (uint16_t)(i0 + 4 * lane + e);
        }
        p += (key[e] >> 20) == ub1 ? 1u : 0u;
      }
      cb += wave_bcast(einc, 63);
    } else if (!all) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((key[e] >> 20) == ub1) atomicAdd(&h[(key[e] >> 10) & 0x3FFu], 1u);
    }
    emit(i0, sel, v);
  });
  if (!all) {
    uint32_t need = kk - above;
    int b2, b3;
    uint32_t ab;
    if (gather) {
      zero_hist();
      for (int i = lane; i < (int)inbin; i += 64) atomicAdd(&h[(ck[i] >> 10) & 0x3FFu], 1u);
    }
    wave_hist_find(1024, need, [&](int q) { return h[q]; }, &b2, &ab);
    need -= ab;
    const uint32_t pre = (ub1 << 10) | (uint32_t)b2;
    const uint32_t c2 = h[b2];                           // slots sharing the 22-bit prefix
    if (gather) {
      if (c2 <= 256) {
        uint32_t eb = 0;
        for (int i0 = 0; i0 < (int)inbin; i0 += 64) {
          const int i = i0 + lane;
          const uint32_t key = i < (int)inbin ? ck[i] : 0u;
          const uint32_t slot = i < (int)inbin ? cs[i] : 0u;
          const bool eq = (key >> 10) == pre;
          const uint32_t einc = wave_scan_dpp(eq ? 1u : 0u);
          if (eq) {
            h[eb + einc - 1] = key;
            h[256 + eb + einc - 1] = slot;
          }
          eb += wave_bcast(einc, 63);
          emit1((key >> 10) > pre, slot, key);
        }
        rank_emit(c2, need);
      } else {
        zero_hist();
        for (int i = lane; i < (int)inbin; i += 64)
          if ((ck[i] >> 10) == pre) atomicAdd(&h[ck[i] & 0x3FFu], 1u);
        wave_hist_find(1024, need, [&](int q) { return h[q]; }, &b3, &ab);
        const uint32_t T = (pre << 10) | (uint32_t)b3;
        const uint32_t need_eq = need - ab;              // slots equal to T that are kept
        uint32_t eqb = 0;
        for (int i0 = 0; i0 < (int)inbin; i0 += 64) {
          const int i = i0 + lane;
          const uint32_t key = i < (int)inbin ? ck[i] : 0u;
          const uint32_t slot = i < (int)inbin ? cs[i] : 0u;
          const bool eq = key == T;
          const uint32_t einc = wave_scan_dpp(eq ? 1u : 0u);
          emit1(key > T || (eq && eqb + einc - 1 < need_eq), slot, key);
          eqb += wave_bcast(einc, 63);
        }
      }
    } else if (c2 <= 256) {
      uint32_t eb = 0;
      stream([&](int i0, const uint32_t (&key)[4], const f32x4_t& v) {
        bool sel[4];
        uint32_t ce = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sel[e] = (key[e] >> 20) == ub1 && (key[e] >> 10) > pre;
          ce += (key[e] >> 10) == pre ? 1u : 0u;
        }
        const uint32_t einc = wave_scan_dpp(ce);
        uint32_t p = eb + einc - ce;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((key[e] >> 10) == pre && p < 256u) {
            h[p] = key[e];
            h[256 + p] = (uint32_t)(i0 + 4 * lane + e);
          }
          p += (key[e] >> 10) == pre ? 1u : 0u;
        }
        eb += wave_bcast(einc, 63);
        emit(i0, sel, v);
      });
      rank_emit(c2, need);
    } else {
      zero_hist();
      stream([&](int, const uint32_t (&key)[4], const f32x4_t&) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((key[e] >> 10) == pre) atomicAdd(&h[key[e] & 0x3FFu], 1u);
      });
      wave_hist_find(1024, need, [&](int q) { return h[q]; }, &b3, &ab);
      const uint32_t T = (pre << 10) | (uint32_t)b3;
      const uint32_t need_eq = need - ab;                // slots equal to T that are kept
      uint32_t eqb = 0;                                  // equal slots seen so far
      stream([&](int i0, const uint32_t (&key)[4], const f32x4_t& v) {
        const uint32_t ce = (key[0] == T ? 1u : 0u) + (key[1] == T ? 1u : 0u) + (key[2] == T ? 1u : 0u) +
                            (key[3] == T ? 1u : 0u);
        const uint32_t einc = wave_scan_dpp(ce);
        uint32_t r = eqb + einc - ce;                    // rank of this lane's first equal slot
        bool sel[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool eq = key[e] == T;
          sel[e] = ((key[e] >> 20) == ub1 && key[e] > T) || (eq && r < need_eq);
          r += eq ? 1u : 0u;
        }
        eqb += wave_bcast(einc, 63);
        emit(i0, sel, v);
      });
    }
  }
  for (int p = (int)kk + lane; p < k; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
}

template <class Mma, int D, int HB, int KST, bool LISTM>
__global__ void __launch_bounds__(WavesFor<HB>::value * 64)
score_kernel(ScoreArgs a) {
  constexpr int NW = WavesFor<HB>::value;
  constexpr int NTHR = NW * 64;
  constexpr bool DIRECT = Direct<Mma, KST>::value;
  constexpr int KT = TileKeys<Mma, KST>::value;
  constexpr int NSUB = KT / 32;
  constexpr bool META = LISTM || KST == DT_FP8;
  static_assert(!Direct<Mma, KST>::value || NSUB >= 2, "direct tiles span several 32-key steps");
  typedef Geo<Mma, D, KT> G;
  typedef TileLoader<Mma, D, KST, NTHR, KT> Loader;
  typedef DirectLoader<D, NTHR, KT> DLoader;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tiles = smem;
  int32_t* skey = reinterpret_cast<int32_t*>(smem + 2 * G::TILE_BYTES);   // [2][KT]
  float* sscale = reinterpret_cast<float*>(skey + 2 * KT);                 // [2][KT]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-level values stay scalar
  // per-wave histogram of the first radix digit of the row's order-preserving score keys, from
  // which the wave writes its row's selection summary (the selector's first radix pass)
  uint32_t* whist = reinterpret_cast<uint32_t*>(sscale + 2 * KT) + wave * 2048;
  const bool fuse = a.row_meta != nullptr;
  const int lin = gridDim.x - 1 - blockIdx.x;       // heaviest tiles first
  const int b = lin % a.B;
  const int ti = lin / a.B;

  int tb, te, lrow = 0, row0;
  if constexpr (!LISTM) {
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
  if constexpr (!LISTM) {
    my_count = active ? count_of(my_pos) : 0;
    // the tile's key range: the longest prefix of its (at most 64) queries, one load per lane
    const int c = lane < te - tb ? count_of(a.q_pos[(int64_t)b * a.T + tb + lane]) : 0;
    key_end = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) key_end = max(key_end, __builtin_amdgcn_readlane(c, u));
  } else {
    key_end = a.list_len[lrow];
    my_count = key_end;
  }
  if (blockIdx.y == 0 && active && lane == 0)
    a.row_len[(int64_t)b * a.rows_per_seq + (t - row0)] = my_count;

  const int kb0 = blockIdx.y * a.split_keys;
  const int kb1 = min(key_end, kb0 + a.split_keys);
  if (kb0 >= kb1) return;                           // uniform over the work-group
  const int lim = min(my_count, kb1);               // this wave's last slot (exclusive)
  if (fuse)
    for (int i = lane; i < 512; i += 64) reinterpret_cast<u32x4_t*>(whist)[i] = u32x4_t{0u, 0u, 0u, 0u};

  // query fragments and head weights of this wave's query
  typename Mma::frag_t qf[HB][G::NKK];
  float wv[HB][16];
  {
    const int hh = lane >> 5, ln = lane & 31;
    const int qeb = dtype_bytes(a.q_dtype);
    const float* wrow = a.w + ((int64_t)b * a.T + (active ? t : 0)) * a.H;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 32 * hb + ln;
      const bool ok = active && head < a.H;
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                            (((int64_t)b * a.T + (ok ? t : 0)) * a.H + (ok ? head : 0)) * D * qeb;
      // a head block the query fills: plain loads (no per-lane branches); the weights of the
      // 16 heads a lane accumulates are 4 runs of 4 consecutive heads
      if (active && 32 * hb + 32 <= a.H) {
#pragma unroll
        for (int kk = 0; kk < G::NKK; ++kk)
          qf[hb][kk] = load_frag<Mma>(qrow, a.q_dtype, hh * (D / 2) + kk * Mma::E);
      } else {
#pragma unroll
        for (int kk = 0; kk < G::NKK; ++kk) {
          if (ok) qf[hb][kk] = load_frag<Mma>(qrow, a.q_dtype, hh * (D / 2) + kk * Mma::E);
          else qf[hb][kk] = typename Mma::frag_t{};
        }
      }
      if (active && 32 * hb + 32 <= a.H && (a.H & 3) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(wrow + 32 * hb + 8 * j + 4 * hh);
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[hb][4 * j + i] = v[i];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int h = acc_head(hb, r, lane);
          wv[hb][r] = (active && h < a.H) ? wrow[h] : 0.f;
        }
      }
    }
  }

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.keys) +
                        (int64_t)b * a.key_cap * (D * Loader::SRC_EB);
  const int32_t* lst = LISTM ? a.list + (int64_t)lrow * a.list_stride : nullptr;
  auto key_at = [&](int base, int n) -> int {       // key index of slot base + n, or -1
    const int j = base + n;
    if (j >= kb1) return -1;
    if constexpr (LISTM) return lst[j];
    else return j;
  };
  auto scale_of = [&](int ki) -> float {
    if constexpr (KST == DT_FP8) return ki >= 0 ? a.k_scale[(int64_t)b * a.key_cap + ki] : 0.f;
    else return 1.f;
  };

  const int ntile = (kb1 - kb0 + KT - 1) / KT;
  Loader ld;
  // direct path, key list: key indices of the rows this thread's DMA chunks fill, read one tile
  // ahead (a key range computes them when it issues the chunks)
  int kidx[DIRECT && LISTM ? DLoader::ITERS : 1];
  auto fetch_idx = [&](int base) {
    if constexpr (DIRECT && LISTM) {
#pragma unroll
      for (int i = 0; i < DLoader::ITERS; ++i) kidx[i] = key_at(base, DLoader::row_of(i, wave, lane));
    }
  };
  auto chunk_key = [&](int base, int i) -> int {
    if constexpr (LISTM) return kidx[i];
    else return key_at(base, DLoader::row_of(i, wave, lane));
  };
  auto issue_tile = [&](int buf, int base) {        // start filling LDS buffer `buf`
    if constexpr (DIRECT) {
#pragma unroll
      for (int i = 0; i < DLoader::ITERS; ++i)
        DLoader::load_chunk(i, kseq, tiles + buf * G::TILE_BYTES, wave, lane, chunk_key(base, i));
      if constexpr (LISTM) {
#pragma unroll
        for (int i = 0; i < DLoader::ITERS; ++i)
          if (DLoader::first_chunk(i, wave, lane)) skey[buf * KT + DLoader::row_of(i, wave, lane)] = kidx[i];
      }
    } else {
      ld.load(kseq, tid, [&](int n) { return key_at(base, n); });
      if (META && tid < KT) {
        const int ki = key_at(base, tid);
        skey[buf * KT + tid] = ki;
        sscale[buf * KT + tid] = scale_of(ki);
      }
    }
  };

  fetch_idx(kb0);
  issue_tile(0, kb0);
  if constexpr (DIRECT) {
    if (ntile > 1) fetch_idx(kb0 + KT);
    wait_vmem();
  } else {
    ld.store(tiles, tid);
  }
  __syncthreads();

  float* srow = a.scores + ((int64_t)b * a.rows_per_seq + (active ? t - row0 : 0)) * a.score_stride;
  bf16x8_t bfr[DIRECT ? G::NKK : 1];                 // rotating key fragments (bf16 path)

  // Scores of a full tile are counted and stored at the start of the next tile, before its
  // first load: the compiler waits for every outstanding vector memory operation before an LDS
  // access that follows the tiles' LDS loads, so the histogram adds must not come after a
  // load; and at the end of the tile they would hold every wave up at the tile barrier.
  float pv[NSUB / 2];
  int pbase = -1;                                     // first slot of the pending scores, or -1
#pragma unroll
  for (int p = 0; p < NSUB / 2; ++p) pv[p] = 0.f;
  // (a key list keeps the immediate stores: its registers are needed for the list indices)
  constexpr bool DEFER = !LISTM;
  auto flush = [&]() {
    if (DEFER && pbase >= 0) {
      if (fuse) {
#pragma unroll
        for (int p = 0; p < NSUB / 2; ++p) {
          const uint32_t key = f2key(pv[p]);
          hist1_add_if(whist, key, a.digit_bits, key > KEY_NEG_INF);
        }
      }
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) srow[pbase + p * 64 + lane] = pv[p];
      pbase = -1;
    }
  };

  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1;
    const int base = kb0 + it * KT;
    const bool more = it + 1 < ntile;
    flush();
    // bf16 full tiles issue the next tile's loads spread over their MFMA steps (8 waves issuing
    // all their loads at once queue behind each other and start the tile apart); other tiles
    // issue them all here
    const bool full = active && base + KT <= lim;
    const bool spread = DIRECT && full;
    if (more && !spread) {
      issue_tile(cur ^ 1, base + KT);
      if constexpr (DIRECT) {
        if (it + 2 < ntile) fetch_idx(base + 2 * KT);
      }
    }
    const uint8_t* tile = tiles + cur * G::TILE_BYTES;
    // scores of this tile, two 32-key steps per value (lanes 0-31: even step, 32-63: odd step)
    float ov[NSUB / 2];
#pragma unroll
    for (int p = 0; p < NSUB / 2; ++p) ov[p] = 0.f;
    if (full) {
      // full tile: the epilogue of each 32-key step overlaps the MFMAs of the next one, and
      // the next step's key fragments are read from LDS while this step's MFMAs run
      f32x16_t A[HB], Bq[HB];
      float t_prev = 0.f;
      auto mma_step = [&](int s, f32x16_t (&acc)[HB]) {
        if constexpr (DIRECT) {
          tile_mma_rot<D, HB, KT>(qf, bfr, tile, (s + 1) * 32, s + 1 < NSUB, lane, acc);
        } else {
          tile_mma<Mma, D, HB, KT>(qf, tile, s * 32, lane, acc);
        }
      };
      // the next tile's load chunks go out during the first NSUB - 1 steps (chunk i in step
      // i (NSUB - 1) / IT), so that the last has a whole step to land; on the last tile they
      // refill the idle buffer with rows already read (no branch inside the MFMA stream)
      constexpr int IT = DIRECT ? DLoader::ITERS : 0;
      auto dma_part = [&](int s) {
        if constexpr (DIRECT) {
#pragma unroll
          for (int i = (s * IT + NSUB - 2) / (NSUB - 1); i < ((s + 1) * IT + NSUB - 2) / (NSUB - 1) && i < IT; ++i)
            DLoader::load_chunk(i, kseq, tiles + (cur ^ 1) * G::TILE_BYTES, wave, lane,
                                chunk_key(base + KT, i));
        }
      };
      if constexpr (DIRECT) load_bfrag<D, KT>(tile, 0, lane, bfr);
      mma_step(0, A);
      dma_part(0);
#pragma unroll
      for (int s = 1; s < NSUB; ++s) {
        float tcur;
        if constexpr (DIRECT) __builtin_amdgcn_sched_barrier(0);
        if (s & 1) {
          mma_step(s, Bq);
          tcur = tile_epilogue<HB>(A, wv);
        } else {
          mma_step(s, A);
          tcur = tile_epilogue<HB>(Bq, wv);
        }
        dma_part(s);
        if constexpr (DIRECT) {
          // per key-fragment step: HB MFMAs, one LDS read of the next step, then a slice of
          // the previous step's epilogue; this step's load chunks go out after the first MFMAs
          constexpr int NL = IT / NSUB > 0 ? IT / NSUB : 1;
#pragma unroll
          for (int kk = 0; kk < G::NKK; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, HB, 0);
            if (s + 1 < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (kk == 1) __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (16 * HB * 2 + 8) / G::NKK + 1, 0);
          }
        }
        if ((s - 1) & 1) ov[(s - 2) / 2] = lane < 32 ? t_prev : tcur;
        else t_prev = tcur;
      }
      const float tl = tile_epilogue<HB>(Bq, wv);
      ov[NSUB / 2 - 1] = lane < 32 ? t_prev : tl;
      if constexpr (DIRECT) {
        if (more) {
          if constexpr (LISTM) {
#pragma unroll
            for (int i = 0; i < DLoader::ITERS; ++i)
              if (DLoader::first_chunk(i, wave, lane))
                skey[(cur ^ 1) * KT + DLoader::row_of(i, wave, lane)] = kidx[i];
          }
          if (it + 2 < ntile) fetch_idx(base + 2 * KT);
        }
      }
    } else if (active && base < lim) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (base + s * 32 >= lim) break;
        f32x16_t A[HB];
        tile_mma<Mma, D, HB, KT>(qf, tile, s * 32, lane, A);
        const float tot = tile_epilogue<HB>(A, wv);
        if ((s & 1) == (lane >> 5)) ov[s / 2] = tot;
      }
    }
    if constexpr (DIRECT) {
      if (more || spread) wait_vmem();
    } else {
      if (more) ld.store(tiles + (cur ^ 1) * G::TILE_BYTES, tid);
    }
    if (DEFER && full) {
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) {
        const int n = p * 64 + lane;
        pv[p] = ov[p];
        if constexpr (KST == DT_FP8) pv[p] *= sscale[cur * KT + n];
        if constexpr (LISTM) {
          if (skey[cur * KT + n] > my_pos) pv[p] = -INFINITY;
        }
      }
      pbase = base;
    } else if (active) {
      // partial tile: every LDS access (scale, key list, histogram) before the score stores
      float v[NSUB / 2];
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) {
        const int n = p * 64 + lane;
        v[p] = ov[p];
        if (base + n < lim) {
          if constexpr (KST == DT_FP8) v[p] *= sscale[cur * KT + n];
          if constexpr (LISTM) {
            if (skey[cur * KT + n] > my_pos) v[p] = -INFINITY;
          }
          if (fuse) {
            const uint32_t key = f2key(v[p]);
            if (key > KEY_NEG_INF) hist1_add(whist, key, a.digit_bits);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p)
        if (base + p * 64 + lane < lim) srow[base + p * 64 + lane] = v[p];
    }
    lds_barrier();
  }
  flush();
  if (fuse && active) {
    int bin;
    uint32_t above;
    const int bits = a.digit_bits;
    // bin q's count without a branch on the digit width (12 bits: bins q and q + 2048 are the
    // 16-bit halves of word q mod 2048)
    const uint32_t hm = bits == 12 ? 0xFFFFu : 0xFFFFFFFFu;
    const int hsh = bits == 12 ? 11 : 31;
    const uint32_t tot = wave_hist_find(1 << bits, (uint32_t)a.topk_k,
                                        [&](int q) { return (whist[q & 2047] >> ((q >> hsh) << 4)) & hm; },
                                        &bin, &above);
    if (lane == 0) {
      int32_t* m = a.row_meta + ((int64_t)b * a.rows_per_seq + (t - row0)) * 4;
      m[META_NVALID] = (int32_t)tot;
      m[META_BIN] = bin;
      m[META_ABOVE] = (int32_t)above;
      m[META_INBIN] = bin >= 0 ? (int32_t)hist1_count(whist, bin, bits) : 0;
    }
    if constexpr (!LISTM) {
      if (a.sel_idx != nullptr && bits == 12) {
        wait_vmem();                                     // this wave's score stores
        // the wave's share of the key tiles (idle after the last tile) holds bin b1's keys
        constexpr int SLICE = 2 * G::TILE_BYTES / NW / 4;
        const uint32_t inbin = bin >= 0 ? hist1_count(whist, bin, 12) : 0u;
        wave_select_row<SLICE < 2048 ? SLICE : 2048>(
            srow, my_count, a.score_stride, a.topk_k, tot, bin, above, inbin, whist,
            reinterpret_cast<uint32_t*>(tiles + wave * (2 * G::TILE_BYTES / NW)),
            a.sel_idx + ((int64_t)b * a.sel_T + t) * a.topk_k,
                        a.sel_score ? a.sel_score + ((int64_t)b * a.sel_T + t) * a.topk_k : nullptr);
      }
    }
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
  constexpr int KT = TileKeys<Mma, KST>::value;
  typedef Geo<Mma, D, KT> G;
  const size_t lds = 2 * G::TILE_BYTES + 4 * KT * sizeof(int32_t) +
                     (a.row_meta ? (size_t)NW * 2048 * sizeof(uint32_t) : 0);
  auto kfn = a.mode == MODE_LIST ? score_kernel<Mma, D, HB, KST, true>
                                 : score_kernel<Mma, D, HB, KST, false>;
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
