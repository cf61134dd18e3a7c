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
#pragma once
#include <type_traits>

#include "score_tile.h"

namespace idx {

// Keys already in the MFMA element format stream straight into LDS: bf16 keys for the bf16 MFMA,
// FP8 keys for the FP8 MFMA.
template <class Mma, int KST> struct Direct {
  static constexpr bool value = (std::is_same<Mma, MmaBf16>::value && KST == DT_BF16) ||
                                (std::is_same<Mma, MmaFp8>::value && KST == DT_FP8);
};
template <class Mma, int KST> struct TileKeys {
  static constexpr int value = Direct<Mma, KST>::value ? 128 : 64;
};

// One wave selects the top k slots of its own score row from the row's candidate list (LIST: n
// entries, entry i holding a score (srow[i]) and its 16-bit slot (sslot[i])) or from the row itself
// (!LIST: n slots, entry i is slot i; sslot is then only the room the compaction below uses). A
// list holds every
// finite slot at or above a bound no higher than the final first-digit bin b1 (the score kernel
// writes it while it scores the row), and the row's 12-bit first-digit summary counts every finite
// slot: tot finite slots, bin b1 of the k-th largest key, `above` slots in higher bins and `inbin`
// slots in bin b1. One pass over the list writes the entries above bin b1 to the output and keeps
// the entries of bin b1:
//   - when they fit (inbin <= CAP) as (key, slot) pairs in LDS (keys in `ck`, 16-bit slots in the
//     upper half of `h`);
//   - otherwise compacted into the list itself: entry p (key over srow[p], slot over sslot[p],
//     which this wave has already read, since p counts a subset of the entries read so far). The
//     10-bit histogram of the next digit is built during the pass.
// The k-th key is then resolved on the kept entries digit by digit: 10 more bits give its 22-bit
// prefix; entries above the prefix are written, and the entries sharing it (at most 256) are
// ranked exactly, higher key first, then lower slot (ties keep the lowest slots); a prefix shared
// by more entries takes a last 10-bit digit and keeps the lowest slots equal to the k-th key (the
// list is in ascending slot order). Histograms use 1024 words of `h`. List reads are eight
// 16-byte score loads and eight 8-byte slot loads per lane at a time; `last` is the highest
// index a 4-entry load may start at. Output order: pass order, list order within a pass.
template <int CAP, bool LIST>
__device__ __forceinline__ void wave_select_row(float* srow, uint16_t* sslot, int n, int last, int k,
                                                uint32_t tot, int b1, uint32_t above, uint32_t inbin,
                                                uint32_t* h, uint32_t* ck, int32_t* oidx, float* osc) {
  static_assert(CAP <= 2048, "16-bit slots in 1024 words");
  constexpr int U = 8;
  const int lane = lane_id();
  const uint32_t kk = min((uint32_t)k, tot);
  const bool all = kk == tot;
  const bool lds = !all && inbin <= (uint32_t)CAP;   // bin b1 kept as LDS pairs
  const bool glob = !all && !lds;                     // bin b1 compacted into the list
  uint16_t* cs = reinterpret_cast<uint16_t*>(h + 1024);
  uint32_t* crow = reinterpret_cast<uint32_t*>(srow);
  // visits the list 256 entries at a time: f(i0, key[4], v, slot[4]) with key 0 past the list.
  // The loads of the next 256 U entries are in flight while the current ones are processed (two
  // register buffers); indexes are clamped into the row's allocation. f may overwrite entries
  // below the end of the block it processes: the loads in flight are all at or above it.
  auto stream = [&](auto f) {
    f32x4_t va[U], vb[U];
    u32x2_t sa[U], sb[U];
    auto load = [&](int i0, f32x4_t (&v)[U], u32x2_t (&sv)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(i0 + 256 * u + 4 * lane, last);
        v[u] = *reinterpret_cast<const f32x4_t*>(srow + j);
        if constexpr (LIST) sv[u] = *reinterpret_cast<const u32x2_t*>(sslot + j);
      }
    };
    auto run = [&](int i0, const f32x4_t (&v)[U], const u32x2_t (&sv)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j0 = i0 + 256 * u;
        if (j0 >= n) break;
        uint32_t key[4], sl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          key[e] = j0 + 4 * lane + e < n ? f2key(v[u][e]) : 0u;
          if constexpr (LIST) sl[e] = (sv[u][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          else sl[e] = (uint32_t)(j0 + 4 * lane + e);
        }
        f(j0, key, v[u], sl);
      }
    };
    load(0, va, sa);
    for (int i0 = 0; i0 < n; i0 += 512 * U) {
      load(i0 + 256 * U, vb, sb);
      run(i0, va, sa);
      if (i0 + 256 * U >= n) break;
      load(i0 + 512 * U, va, sa);
      run(i0 + 256 * U, vb, sb);
    }
  };
  uint32_t pos = 0;
  // writes the entries flagged in sel[4] at pos, in list order (never past the k outputs,
  // whatever the summary says)
  auto emit = [&](const bool (&sel)[4], const f32x4_t& v, const uint32_t (&sl)[4]) {
    const uint32_t c = (sel[0] ? 1u : 0u) + (sel[1] ? 1u : 0u) + (sel[2] ? 1u : 0u) + (sel[3] ? 1u : 0u);
    const uint32_t inc = wave_scan_dpp(c);
    uint32_t p = pos + inc - c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (sel[e] && p < (uint32_t)k) {
        oidx[p] = (int32_t)sl[e];
        if (osc) osc[p] = v[e];
      }
      p += sel[e] ? 1u : 0u;
    }
    pos += wave_bcast(inc, 63);
  };
  // writes one flagged entry per lane at pos, in lane order
  auto emit1 = [&](bool sel, uint32_t slot, uint32_t key) {
    const uint32_t inc = wave_scan_dpp(sel ? 1u : 0u);
    if (sel && pos + inc - 1 < (uint32_t)k) {
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
  if (glob) zero_hist();
  uint32_t cb = 0;                                       // kept entries of bin b1
  stream([&](int i0, const uint32_t (&key)[4], const f32x4_t& v, const uint32_t (&sl)[4]) {
    bool sel[4];
    uint32_t ce = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = all ? key[e] > KEY_NEG_INF : (key[e] >> 20) > ub1;
      ce += (key[e] >> 20) == ub1 ? 1u : 0u;
    }
    if (lds) {
      const uint32_t einc = wave_scan_dpp(ce);
      uint32_t p = cb + einc - ce;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((key[e] >> 20) == ub1 && p < (uint32_t)CAP) {   // p < inbin for finite keys
          ck[p] = key[e];
          cs[p] = (uint16_t)sl[e];
        }
        p += (key[e] >> 20) == ub1 ? 1u : 0u;
      }
      cb += wave_bcast(einc, 63);
    } else if (glob) {
      const uint32_t einc = wave_scan_dpp(ce);
      uint32_t p = cb + einc - ce;                       // p < i0 + 256: entries already read
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((key[e] >> 20) == ub1 && p < (uint32_t)n) {
          crow[p] = key[e];
          sslot[p] = (uint16_t)sl[e];
          atomicAdd(&h[(key[e] >> 10) & 0x3FFu], 1u);
        }
        p += (key[e] >> 20) == ub1 ? 1u : 0u;
      }
      cb += wave_bcast(einc, 63);
    }
    emit(sel, v, sl);
  });
  if (!all) {
    if (glob) {
      // the compacted entries are read back: wait for the stores, and drop any stale copy of
      // the list the vector L1 cache still holds
      wait_vmem();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    // kept entry i of bin b1: its key and slot
    auto get = [&](int i, uint32_t& key, uint32_t& slot) {
      if (lds) {
        key = ck[i];
        slot = cs[i];
      } else {
        key = crow[i];
        slot = sslot[i];
      }
    };
    inbin = min(inbin, min(cb, lds ? (uint32_t)CAP : (uint32_t)n));   // slots actually kept
    uint32_t need = kk - above;
    int b2, b3;
    uint32_t ab;
    if (lds) {
      zero_hist();
      for (int i = lane; i < (int)inbin; i += 64) atomicAdd(&h[(ck[i] >> 10) & 0x3FFu], 1u);
    }
    wave_hist_find(1024, need, [&](int q) { return h[q]; }, &b2, &ab);
    need -= ab;
    const uint32_t pre = (ub1 << 10) | (uint32_t)b2;
    const uint32_t c2 = h[b2];                           // slots sharing the 22-bit prefix
    if (c2 <= 256) {
      uint32_t eb = 0;
      for (int i0 = 0; i0 < (int)inbin; i0 += 64) {
        const int i = i0 + lane;
        uint32_t key = 0, slot = 0;
        if (i < (int)inbin) get(i, key, slot);
        const bool eq = (key >> 10) == pre;
        const uint32_t einc = wave_scan_dpp(eq ? 1u : 0u);
        if (eq && eb + einc - 1 < 256u) {
          h[eb + einc - 1] = key;
          h[256 + eb + einc - 1] = slot;
        }
        eb += wave_bcast(einc, 63);
        emit1((key >> 10) > pre, slot, key);
      }
      rank_emit(c2, need);
    } else {
      zero_hist();
      for (int i = lane; i < (int)inbin; i += 64) {
        uint32_t key, slot;
        get(i, key, slot);
        if ((key >> 10) == pre) atomicAdd(&h[key & 0x3FFu], 1u);
      }
      wave_hist_find(1024, need, [&](int q) { return h[q]; }, &b3, &ab);
      const uint32_t T = (pre << 10) | (uint32_t)b3;
      const uint32_t need_eq = need - ab;                // slots equal to T that are kept
      uint32_t eqb = 0;
      for (int i0 = 0; i0 < (int)inbin; i0 += 64) {
        const int i = i0 + lane;
        uint32_t key = 0, slot = 0;
        if (i < (int)inbin) get(i, key, slot);
        const bool eq = key == T;
        const uint32_t einc = wave_scan_dpp(eq ? 1u : 0u);
        emit1(key > T || (eq && eqb + einc - 1 < need_eq), slot, key);
        eqb += wave_bcast(einc, 63);
      }
    }
  }
  for (int p = (int)kk + lane; p < k; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
}

template <class Mma, int D, int HB, int KST, bool LISTM, bool CMP>
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
  typedef DirectLoader<Mma, D, NTHR, KT> DLoader;
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
  if (kb0 >= kb1) {                                 // uniform over the work-group
    // every query of the tile has an empty prefix: its summary says "nothing to select", and a
    // self-selecting kernel writes the padded output row itself (nothing else will)
    if (blockIdx.y == 0 && fuse && active) {
      if (lane == 0) {
        int32_t* m = a.row_meta + ((int64_t)b * a.rows_per_seq + (t - row0)) * 4;
        m[META_NVALID] = 0;
        m[META_BIN] = -1;
        m[META_ABOVE] = 0;
        m[META_INBIN] = 0;
      }
      if constexpr (!LISTM) {
        if (a.sel_idx != nullptr && a.digit_bits == 12) {
          if (a.sel_cnt != nullptr && lane == 0) a.sel_cnt[(int64_t)b * a.sel_T + t] = 0;
          int32_t* oi = a.sel_idx + ((int64_t)b * a.sel_T + t) * a.topk_k;
          float* os = a.sel_score ? a.sel_score + ((int64_t)b * a.sel_T + t) * a.topk_k : nullptr;
          for (int p = lane; p < a.topk_k; p += 64) {
            oi[p] = -1;
            if (os) os[p] = -INFINITY;
          }
        }
      }
    }
    return;
  }
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
      // FP8 queries: each head's query scale is a factor of that head's weight (both >= 0 under
      // ReLU: w ReLU(c x) = (w c) ReLU(x))
      if constexpr (std::is_same<Mma, MmaFp8>::value) {
        const float* qsrow = a.q_scale + ((int64_t)b * a.T + (active ? t : 0)) * a.H;
#pragma unroll
        for (int r = 0; r < 16; ++r) wv[hb][r] *= qsrow[min(acc_head(hb, r, lane), a.H - 1)];
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
  typename Mma::frag_t bfr[DIRECT ? G::NKK : 1];     // rotating key fragments (direct paths)

  // Scores of a full tile are counted and stored at the start of the next tile, before its
  // first load: the compiler waits for every outstanding vector memory operation before an LDS
  // access that follows the tiles' LDS loads, so the histogram adds must not come after a
  // load; and at the end of the tile they would hold every wave up at the tile barrier.
  // 12-bit digits count in 16-bit halves: slot 65535 (only rows of 65536 slots have it) is kept
  // out of the histogram so that no count reaches 65536; the summary adds it back
  const int xslot = a.digit_bits == 12 ? 65535 : -1;
  // A wave that selects its own row keeps a candidate list instead of the row: every finite
  // score at or above a running bound cbin (the first-digit bin of the k-th largest score counted
  // so far, which never exceeds the row's final bin b1: the k-th largest of a subset is at most
  // that of the whole), in slot order, with the 16-bit slots after the scores (sslot). The
  // selection then reads the list instead of the whole row.
  const bool cmp = CMP && !LISTM && fuse && a.sel_idx != nullptr && a.digit_bits == 12;   // uniform
  uint16_t* sslot = reinterpret_cast<uint16_t*>(srow + a.slot_off);
  uint32_t ccnt = 0, cbin = 0;                        // list entries; bound (12-bit bin)
  // one score per lane at `slot` (inside the prefix when ok), by every lane of the wave. Without
  // a branch: the listed scores go to the list's end, the others right after them, where the
  // next listed scores overwrite them (the row has 64 entries of room past its slot count), so
  // that every lane stores and the 64 stores are contiguous
  auto put = [&](float v, int slot, bool ok) {
    if (cmp) {
      const uint32_t key = f2key(v);
      const bool f = ok && key > KEY_NEG_INF && (key >> 20) >= cbin;
      const uint64_t m = __ballot(f);
      const uint32_t nf = (uint32_t)__popcll(m);
      const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t at = f ? ccnt + r : ccnt + nf + ((uint32_t)lane - r);
      srow[at] = v;
      sslot[at] = (uint16_t)slot;
      ccnt += nf;
    } else if (ok) {
      srow[slot] = v;
    }
  };
  // raises the bound every 32 stored tiles: a scan of the histogram from the highest bin down,
  // 64 bins per step, to the bin holding the k-th largest counted score (a short loop with one
  // LDS read per lane, so that it costs the tile loop no registers). The histogram counts the
  // listed scores only (every finite score while fewer than k are counted, then those at or
  // above the bound): it holds every score at or above the current bound, so the k-th largest it
  // counts is the k-th largest seen so far; and its total reaches k exactly only if those k are
  // the row's top k, since every later score is below the bound.
  int nflush = 0;
  auto raise_bound = [&]() {
    ++nflush;
    if (cmp && (nflush & 31) == 0) {
      uint32_t run = 0;
      for (int top = 4095; top >= (int)cbin; top -= 64) {
        const int q = top - lane;                        // lane 0: the highest bin of the step
        const uint32_t c = q >= (int)cbin ? (whist[q & 2047] >> ((q >> 11) << 4)) & 0xFFFFu : 0u;
        const uint32_t inc = wave_scan_dpp(c);
        const uint64_t hit = __ballot(run + inc >= (uint32_t)a.topk_k);
        if (hit) {
          cbin = (uint32_t)(top - (int)__builtin_ctzll(hit));
          break;
        }
        run += wave_bcast(inc, 63);
      }
    }
  };
  float pv[NSUB / 2];
  int pbase = -1;                                     // first slot of the pending scores, or -1
#pragma unroll
  for (int p = 0; p < NSUB / 2; ++p) pv[p] = 0.f;
  // (a key list keeps the immediate stores: its registers are needed for the list indices)
  constexpr bool DEFER = !LISTM;
  auto flush = [&]() {
    if (DEFER && pbase >= 0) {
      if (fuse) {
        raise_bound();
#pragma unroll
        for (int p = 0; p < NSUB / 2; ++p) {
          const uint32_t key = f2key(pv[p]);
          hist1_add_if(whist, key, a.digit_bits,
                       key > KEY_NEG_INF && pbase + p * 64 + lane != xslot && (!cmp || (key >> 20) >= cbin));
        }
      }
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) put(pv[p], pbase + p * 64 + lane, true);
      pbase = -1;
    }
  };

  // bf16 key ranges carry the last 32-key step of a full tile into the next tile: its epilogue
  // runs under the MFMAs of the next tile's first step (which otherwise has no epilogue to hide)
  // instead of after the tile's MFMAs, where both waves of a SIMD would run it at once, between
  // two barriers. The carried tile's scores are then complete after that first step and are
  // flushed at the start of the tile after (stores and histogram adds stay ahead of every load).
  constexpr bool CARRY = DIRECT && !LISTM;
  f32x16_t A[HB], Bq[HB];                             // step accumulators (Bq: the carried step)
  bool carry = false;
  float c_ov0 = 0.f, c_tprev = 0.f;                   // the carried tile's other scores
  float c_ks[NSUB / 2] = {};                          // and its FP8 key scales
  int c_base = 0;
  auto finish_carry = [&]() {                         // carried step's epilogue without MFMAs
    if (CARRY && carry) {
      const float tl = tile_epilogue<HB>(Bq, wv);
      pv[0] = c_ov0;
      pv[1] = lane < 32 ? c_tprev : tl;
      if constexpr (KST == DT_FP8) {
        pv[0] *= c_ks[0];
        pv[1] *= c_ks[1];
      }
      pbase = c_base;
      carry = false;
      flush();
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
    if (!full) finish_carry();
    if (more && !spread) {
      issue_tile(cur ^ 1, base + KT);
      if constexpr (DIRECT) {
        if (it + 2 < ntile) fetch_idx(base + 2 * KT);
      }
    }
    const uint8_t* tile = tiles + cur * G::TILE_BYTES;
    // FP8 keys: the per-token scale multiplies a key's reduced score. Direct key ranges load the
    // scales of this tile's slots into registers here, used once the tile's scores are done;
    // staged tiles keep them in LDS next to the key indices
    float ksc[NSUB / 2];
#pragma unroll
    for (int p = 0; p < NSUB / 2; ++p) ksc[p] = 1.f;
    if constexpr (DIRECT && KST == DT_FP8 && !LISTM) {
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p)
        ksc[p] = a.k_scale[(int64_t)b * a.key_cap + min(base + p * 64 + lane, a.key_cap - 1)];
    }
    auto tile_scale = [&](int p) -> float {           // scale of slot base + 64 p + lane
      if constexpr (KST != DT_FP8) {
        return 1.f;
      } else if constexpr (!DIRECT) {
        return sscale[cur * KT + p * 64 + lane];
      } else if constexpr (LISTM) {
        const int ki = skey[cur * KT + p * 64 + lane];
        return ki >= 0 ? a.k_scale[(int64_t)b * a.key_cap + ki] : 0.f;
      } else {
        return ksc[p];
      }
    };
    // scores of this tile, two 32-key steps per value (lanes 0-31: even step, 32-63: odd step)
    float ov[NSUB / 2];
#pragma unroll
    for (int p = 0; p < NSUB / 2; ++p) ov[p] = 0.f;
    if (full && DIRECT) {
      // full bf16 tile: each 32-key step's MFMAs carry the previous step's epilogue, fragment by
      // fragment, and refill the key fragments for the next step from LDS; the next tile's load
      // chunks go out during the first NSUB - 1 steps (chunk i in step i (NSUB - 1) / IT, at odd
      // fragments), so that the last has a whole step to land; on the last tile they refill the
      // idle buffer with rows already read (no branch inside the MFMA stream)
      float t_prev = 0.f;
      constexpr int IT = DIRECT ? DLoader::ITERS : 1;
      // (the j-th chunk of a step goes out at fragment 2 j + 1, or at the step's last fragment
      // when the step has fewer fragments: every chunk is issued in every case)
      auto dma = [&](int s, int kk) {
        if constexpr (DIRECT) {
          const int i0 = (s * IT + NSUB - 2) / (NSUB - 1);
          const int i1 = min(IT, ((s + 1) * IT + NSUB - 2) / (NSUB - 1));
#pragma unroll
          for (int i = i0; i < i1; ++i)
            if (min(2 * (i - i0) + 1, G::NKK - 1) == kk)
              DLoader::load_chunk(i, kseq, tiles + (cur ^ 1) * G::TILE_BYTES, wave, lane, chunk_key(base + KT, i));
        }
      };
      if constexpr (DIRECT) {
        static_assert(NSUB == 4, "the carried step is the odd step 3 (accumulator Bq)");
        load_bfrag<Mma, D, KT>(tile, 0, lane, bfr);
        const float tc = tile_mma_epi<Mma, D, HB, KT>(qf, bfr, tile, 32, true, CARRY && carry, lane, A, Bq, wv,
                                                 [&](int kk) { dma(0, kk); });
        if (CARRY && carry) {                           // the carried tile is complete
          pv[0] = c_ov0;
          pv[1] = lane < 32 ? c_tprev : tc;
          if constexpr (KST == DT_FP8) {
            pv[0] *= c_ks[0];
            pv[1] *= c_ks[1];
          }
          pbase = c_base;
          carry = false;
        }
#pragma unroll
        for (int s = 1; s < NSUB; ++s) {
          float tcur;
          if (s & 1)
            tcur = tile_mma_epi<Mma, D, HB, KT>(qf, bfr, tile, (s + 1) * 32, s + 1 < NSUB, true, lane, Bq, A, wv,
                                           [&](int kk) { dma(s, kk); });
          else
            tcur = tile_mma_epi<Mma, D, HB, KT>(qf, bfr, tile, (s + 1) * 32, s + 1 < NSUB, true, lane, A, Bq, wv,
                                           [&](int kk) { dma(s, kk); });
          if ((s - 1) & 1) ov[(s - 2) / 2] = lane < 32 ? t_prev : tcur;
          else t_prev = tcur;
        }
        if constexpr (CARRY) {
          carry = true;
          c_ov0 = ov[0];
          c_tprev = t_prev;
          c_base = base;
#pragma unroll
          for (int p = 0; p < NSUB / 2; ++p) c_ks[p] = ksc[p];
        } else {
          const float tl = tile_epilogue<HB>(Bq, wv);
          ov[NSUB / 2 - 1] = lane < 32 ? t_prev : tl;
        }
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
    } else if (full) {
      // full tile (keys staged through registers): the epilogue of each 32-key step overlaps the
      // MFMAs of the next one
      float t_prev = 0.f;
      tile_mma<Mma, D, HB, KT>(qf, tile, 0, lane, A);
#pragma unroll
      for (int s = 1; s < NSUB; ++s) {
        float tcur;
        if (s & 1) {
          tile_mma<Mma, D, HB, KT>(qf, tile, s * 32, lane, Bq);
          tcur = tile_epilogue<HB>(A, wv);
        } else {
          tile_mma<Mma, D, HB, KT>(qf, tile, s * 32, lane, A);
          tcur = tile_epilogue<HB>(Bq, wv);
        }
        if ((s - 1) & 1) ov[(s - 2) / 2] = lane < 32 ? t_prev : tcur;
        else t_prev = tcur;
      }
      const float tl = tile_epilogue<HB>(Bq, wv);
      ov[NSUB / 2 - 1] = lane < 32 ? t_prev : tl;
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
    if (DEFER && full && !CARRY) {
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) {
        const int n = p * 64 + lane;
        pv[p] = ov[p];
        if constexpr (KST == DT_FP8) pv[p] *= tile_scale(p);
        if constexpr (LISTM) {
          if (skey[cur * KT + n] > my_pos) pv[p] = -INFINITY;
        }
      }
      pbase = base;
    } else if (active && !(CARRY && full)) {
      // partial tile (and a key list's full tile): every LDS access (scale, key list, histogram)
      // before the score stores
      float v[NSUB / 2];
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) {
        const int n = p * 64 + lane;
        v[p] = ov[p];
        if (base + n < lim) {
          if constexpr (KST == DT_FP8) v[p] *= tile_scale(p);
          if constexpr (LISTM) {
            if (skey[cur * KT + n] > my_pos) v[p] = -INFINITY;
          }
          if (fuse) {
            const uint32_t key = f2key(v[p]);
            if (key > KEY_NEG_INF && base + n != xslot && (!cmp || (key >> 20) >= cbin))
              hist1_add(whist, key, a.digit_bits);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < NSUB / 2; ++p) put(v[p], base + p * 64 + lane, base + p * 64 + lane < lim);
    }
    lds_barrier();
  }
  flush();
  finish_carry();
  if (fuse && active) {
    int bin;
    uint32_t above;
    const int bits = a.digit_bits;
    wait_vmem();                                         // this wave's score stores
    // the bin of slot 65535's key, which the histogram left out (-1 if none)
    int xbin = -1;
    if (cmp) {
      // slot 65535 is the list's last entry when it was kept; a key below the bound is not
      // counted, like every other one (see raise_bound)
      if (ccnt > 0 && lim > xslot && xslot >= 0 && sslot[ccnt - 1] == (uint16_t)xslot) {
        const uint32_t xk = f2key(srow[ccnt - 1]);
        if (xk > KEY_NEG_INF) xbin = (int)digit1(xk, bits);
      }
    } else if (lim > xslot && xslot >= 0) {
      const uint32_t xk = f2key(srow[xslot]);
      if (xk > KEY_NEG_INF) xbin = (int)digit1(xk, bits);
    }
    // bin q's count without a branch on the digit width (12 bits: bins q and q + 2048 are the
    // 16-bit halves of word q mod 2048)
    const uint32_t hm = bits == 12 ? 0xFFFFu : 0xFFFFFFFFu;
    const int hsh = bits == 12 ? 11 : 31;
    const uint32_t tot = wave_hist_find(
        1 << bits, (uint32_t)a.topk_k,
        [&](int q) { return ((whist[q & 2047] >> ((q >> hsh) << 4)) & hm) + (q == xbin ? 1u : 0u); }, &bin,
        &above);
    const uint32_t inbin = bin >= 0 ? hist1_count(whist, bin, bits) + (bin == xbin ? 1u : 0u) : 0u;
    if (lane == 0) {
      int32_t* m = a.row_meta + ((int64_t)b * a.rows_per_seq + (t - row0)) * 4;
      m[META_NVALID] = (int32_t)tot;
      m[META_BIN] = bin;
      m[META_ABOVE] = (int32_t)above;
      m[META_INBIN] = (int32_t)inbin;
    }
    if constexpr (!LISTM) {
      if (a.sel_idx != nullptr && bits == 12) {
        if (a.sel_cnt != nullptr && lane == 0)
          a.sel_cnt[(int64_t)b * a.sel_T + t] = (int32_t)min((uint32_t)a.topk_k, tot);
        // the wave's share of the key tiles (idle after the last tile) holds bin b1's keys
        constexpr int SLICE = 2 * G::TILE_BYTES / NW / 4;
        wave_select_row<SLICE < 2048 ? SLICE : 2048, CMP>(
            srow, sslot, CMP ? (int)ccnt : my_count, a.slot_off - 4, a.topk_k, tot, bin, above, inbin, whist,
            reinterpret_cast<uint32_t*>(tiles + wave * (2 * G::TILE_BYTES / NW)),
            a.sel_idx + ((int64_t)b * a.sel_T + t) * a.topk_k,
                        a.sel_score ? a.sel_score + ((int64_t)b * a.sel_T + t) * a.topk_k : nullptr);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launchers, instantiated per (MFMA flavour, key storage, head dim) in the score_*.hip units

template <class Mma, int D, int HB, int KST>
hipError_t launch_one(const ScoreArgs& a, int n_splits, hipStream_t s) {
  constexpr int NW = WavesFor<HB>::value;
  constexpr int KT = TileKeys<Mma, KST>::value;
  typedef Geo<Mma, D, KT> G;
  const size_t lds = 2 * G::TILE_BYTES + 4 * KT * sizeof(int32_t) +
                     (a.row_meta ? (size_t)NW * 2048 * sizeof(uint32_t) : 0);
  auto kfn = a.mode == MODE_LIST ? score_kernel<Mma, D, HB, KST, true, false>
             : a.sel_list       ? score_kernel<Mma, D, HB, KST, false, true>
                                : score_kernel<Mma, D, HB, KST, false, false>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.B * a.tiles_per_seq, n_splits);
  hipLaunchKernelGGL(kfn, grid, dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

// head blocks of 32 heads: 1, 2 or 4 (up to 128 heads)
template <class Mma, int KST, int D>
hipError_t launch_score_d(const ScoreArgs& a, int n_splits, hipStream_t s) {
  const int HB = (a.H + 31) / 32;
  if (HB <= 1) return launch_one<Mma, D, 1, KST>(a, n_splits, s);
  if (HB <= 2) return launch_one<Mma, D, 2, KST>(a, n_splits, s);
  if (HB <= 4) return launch_one<Mma, D, 4, KST>(a, n_splits, s);
  return hipErrorInvalidValue;
}

}  // namespace idx
