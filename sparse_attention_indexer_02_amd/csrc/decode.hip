// Decode-shaped indexer: a few multi-token-prediction queries per sequence (T <= 4) against a
// long key cache, usually FP8 E4M3 with one fp32 scale per token. At long context the indexer's
// scan of the cache, not the sparse attention it feeds, sets the decode time ("Multi-layer
// Indexer", abstract; "PIVOT", abstract), so this path is built around streaming the cache from
// HBM exactly once per step, with both queries of a step sharing every key read.
//
// decode_scan_kernel: work-group = (sequence, chunk of keys, pair of queries), 4 waves, one per
//   SIMD. A wave keeps both queries' bf16 fragments (2 x 64 heads x 128) in the accumulation
//   registers and the head weights in vector registers, so that both queries share every key
//   load and conversion, and walks 16-key blocks of its chunk:
//   - each lane issues 16-byte loads of its key's bytes so that the 4 lanes of a key cover one
//     64-byte segment per instruction; PF blocks are in flight, a block is re-issued as soon as
//     it is consumed (the loop issues no global stores, so each wait is for one block only);
//   - FP8 -> bf16 in registers by the hardware converter (every E4M3 value is a bf16 value, so
//     the MFMA operand is exact); the per-token scale is positive and factors out of ReLU and
//     the head sum, so it multiplies the reduced score;
//   - 16x16x32 bf16 MFMAs (heads = rows, keys = columns), the epilogue of the previous block
//     (ReLU, head weights, cross-lane head sum) interleaved with them;
//   - the fp32 scores of up to DC_SUB keys stay in LDS with a histogram of their first radix
//     digit (12 bits of the order-preserving key). At the end of each sub-chunk the bin of the
//     sub-chunk's own k-th largest score is found, and only the keys in that bin or above are
//     written to the row's candidate list (at the sub-chunk's own slots, with their count). The
//     row's top-k is inside the union of the sub-chunks' top-k, so every key the selection can
//     take is a candidate.
//   With a table of kept blocks (the block filter of "HISA ...", abstract, at decode) the same
//   scan walks the tokens of a row's kept blocks instead of its whole prefix: slot j of the row
//   is the j-th kept token (blocks ascending, so slot order is token order), a 16-key block never
//   straddles two kept blocks (blocks of 16 tokens or more, a power of two), and a query's
//   visible slots are those of its causal prefix, a prefix of the slots.
// decode_select_kernel: work-group = row. The top-k of the row's candidates (radix select over
//   the order-preserving keys, ties to the lowest slots) and the padding; kept-block slots are
//   written out as their tokens.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace idx {

constexpr int DC_BINS = DECODE_BINS;             // 12-bit first digit
constexpr int DC_KB = 16;                        // keys per block (MFMA columns)
constexpr int DC_SUB = DECODE_SUB;               // keys per sub-chunk held in LDS
// blocks in flight per wave (FP8 keys: 2 KB per block per wave; bf16 keys: 4 KB), 8 per SIMD
template <int KST, int W> constexpr int dc_pf() { return (KST == DT_FP8 ? 8 : 4) * 4 / W; }
// waves per scan work-group: one per SIMD at D = 128; two per SIMD at D = 64, where the query
// fragments take half the registers and a second wave per SIMD measured 7-10% faster

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v_t;

// Two E4M3 bytes (bytes 0-1 or 2-3 of a word) -> two bf16 in one word; exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// f2key in three operations (shift, or, xor): the sign bit selects complement or top bit
__device__ __forceinline__ uint32_t f2key3(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ (uint32_t)((int32_t)u >> 31 | (int32_t)0x80000000);
}

// Element placement (the same permutation of d is used for queries and keys, so dot products
// are unchanged). Lane = 16 * g + n: n = key (B operand column) or head (A operand row), g = the
// lane group holding 8 consecutive elements of each K=32 step s.
//   FP8 keys:  d = 64 * (s / 2) + 16 * g + 8 * (s % 2) + e   (lane loads bytes 64 j + 16 g)
//   bf16 keys: d = 32 * s + 8 * g + e                        (lane loads bytes 64 s + 16 g)
template <int KST>
__device__ __forceinline__ int frag_d0(int s, int g) {
  return KST == DT_FP8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
}


// NQ: queries per work-group in the block loop (1 when every work-group scans for one query);
// W: waves per work-group (4: one per SIMD; 8: two per SIMD, a wave's MFMAs beside the other's
// vector work)
template <int D, int HB, int KST, int PF, bool BLK, int NQ, int W>
__global__ void __launch_bounds__(W * 64, 1) decode_scan_kernel(DecodeArgs a) {
  constexpr int NW = W, NT = W * 64;
  constexpr int NS = D / 32;                      // K=32 MFMA steps
  constexpr int KEB = KST == DT_FP8 ? 1 : 2;      // key bytes per element
  constexpr int NLD = D * KEB / 64;               // 16-byte loads per lane per block
  static_assert(PF % 2 == 0, "blocks alternate between two accumulator sets");
  extern __shared__ __align__(16) uint8_t lds[];
  // scores [2][sub] (an area of 2 DC_SUB, so that a row's reads of DC_SUB slots stay inside it)
  float* ssc = reinterpret_cast<float*>(lds);
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds + 8 * DC_SUB);  // [2][2048] 16-bit bins
  uint32_t* misc = hist + 2 * 2048;                                // [32]
  uint32_t* sink = misc + 32;                                      // [2][64] per-lane sinks
  int32_t* btab = reinterpret_cast<int32_t*>(sink + 128);          // BLK: [keep_stride] kept blocks

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int b = blockIdx.x / a.nchunk, chunk = blockIdx.x % a.nchunk;
  const int t0 = a.pair * blockIdx.y;
  const bool two = a.pair == 2 && t0 + 1 < a.T;
  const int nrows = two ? 2 : 1;
  const int kl = a.k_len ? max(0, min(a.k_len[b], a.N)) : a.N;
  const int64_t r0 = (int64_t)b * a.T + t0, r1 = two ? r0 + 1 : r0;
  const int p0 = a.q_pos[r0], p1 = a.q_pos[r1];
  const int P0 = p0 < 0 ? 0 : min(p0 + 1, kl), P1 = p1 < 0 ? 0 : min(p1 + 1, kl);
  // visible slots of each query: its prefix, or with kept blocks the kept tokens inside it
  int V0 = P0, V1 = P1, vmax = kl;
  if constexpr (BLK) {
    const int64_t lrow = (int64_t)b * a.n_groups + t0 / a.group_size;
    const int nk = max(0, min(a.n_kept[lrow], a.keep_stride));
    const int bsz = 1 << a.blk_shift;
    uint32_t s0 = 0, s1 = 0;
    for (int j = tid; j < nk; j += NT) {
      const int blk = a.blocks[lrow * a.keep_stride + j];
      btab[j] = blk;
      const int base = blk << a.blk_shift;
      s0 += (uint32_t)min(max(P0 - base, 0), bsz);
      s1 += (uint32_t)min(max(P1 - base, 0), bsz);
    }
    s0 = wave_bcast(wave_scan_dpp(s0), 63);
    s1 = wave_bcast(wave_scan_dpp(s1), 63);
    if (lane == 0) {
      misc[wave] = s0;
      misc[8 + wave] = s1;
    }
    __syncthreads();
    V0 = V1 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      V0 += (int)misc[w];
      V1 += (int)misc[8 + w];
    }
    vmax = nk << a.blk_shift;
    __syncthreads();
  }
  const int c0 = chunk * a.chunk;
  const int c1 = min(c0 + a.chunk, max(V0, V1));
  {
    // sub-chunks of this chunk past the causal limit have no candidates
    const int s_lo = c0 >= c1 ? c0 / a.sub : (c1 + a.sub - 1) / a.sub;
    const int s_hi = min(c0 + a.chunk, a.vn);
    for (int sg = s_lo + tid; sg * a.sub < s_hi; sg += NT) {
      a.ccount[r0 * a.nsegs + sg] = 0u;
      if (two) a.ccount[r1 * a.nsegs + sg] = 0u;
    }
  }
  if (c0 >= c1) return;

  // query fragments and head weights of both queries (a lone query is repeated): all loads
  // first, then the fragments move to the accumulation registers (they are only MFMA operands
  // there, which leaves the vector registers to the key stream and the epilogue)
  bf16x8_t qf[NQ][HB][NS];
  float wv[NQ][HB][4];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int64_t rr = j == 0 ? r0 : r1;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 16 * hb + n;
      const bool ok = head < a.H;
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (rr * a.H + (ok ? head : 0)) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + frag_d0<KST>(s, g));
        qf[j][hb][s] = ok ? __builtin_bit_cast(bf16x8_t, v) : bf16x8_t{};
      }
      const int h0 = 16 * hb + 4 * g;                              // 4 consecutive heads
      if ((a.H & 3) == 0) {
        const f32x4_t v = h0 < a.H ? *reinterpret_cast<const f32x4_t*>(a.w + rr * a.H + h0) : f32x4_t{};
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[j][hb][r] = v[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          wv[j][hb][r] = a.w[rr * a.H + min(h0 + r, a.H - 1)] * (h0 + r < a.H ? 1.f : 0.f);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int s = 0; s < NS; ++s) asm volatile("" : "+a"(qf[j][hb][s]));

  // uniform bases with 32-bit per-lane byte offsets (one sequence's keys stay below 2^31 bytes)
  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.keys) + (int64_t)b * a.N * (D * KEB);
  const uint8_t* sseq = a.k_scale ? reinterpret_cast<const uint8_t*>(a.k_scale + (int64_t)b * a.N) : nullptr;
  const uint32_t lane_koff = 16u * g;
  const bool owner = g == 0 || (g == 1 && two);                    // lanes that emit a score
  const int oq = (g == 1 && two) ? 1 : 0;                          // and the row they emit for
  float* my_ssc = ssc + oq * a.sub;
  float* sink_f = reinterpret_cast<float*>(sink) + lane;            // writes of masked lanes

  for (int sub0 = c0; sub0 < c1; sub0 += a.sub) {
    const int sub1 = min(sub0 + a.sub, c1);
    for (int i = tid; i < 2 * 2048; i += NT) hist[i] = 0u;
    if (tid < 2) misc[12 + tid] = 0u;                               // candidates written
    __syncthreads();

    // ---- scores of the sub-chunk into LDS
    const int nblk = (sub1 - sub0 + DC_KB - 1) / DC_KB;
    const int per_wave = (nblk + NW - 1) / NW;
    const int iters = (per_wave + PF - 1) / PF * PF;               // extra blocks are masked
    // slot u of raw holds the bytes of a block from its issue until its MFMAs; slot u of scl
    // holds a block's scale until its epilogue, one slot later, so that no loaded register is
    // ever copied (a copy would wait for the load)
    u32x4_t raw[PF][NLD];
    float scl[PF];
    // token of lane n's key in block i (clamped: always issued; with kept blocks, slot -> token
    // through the LDS table, the same entry for a whole 16-key block)
    auto key_of = [&](int i) {
      const int blk = min(i * NW + wave, nblk - 1);
      int v = sub0 + blk * DC_KB + n;
      if constexpr (BLK) {
        v = min(v, vmax - 1);
        v = max((btab[v >> a.blk_shift] << a.blk_shift) | (v & ((1 << a.blk_shift) - 1)), 0);
      }
      return min(v, kl - 1);
    };
    auto issue_keys_at = [&](int tok, u32x4_t (&dst)[NLD]) {
      const uint32_t off = (uint32_t)tok * (D * KEB) + lane_koff;
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        dst[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kseq + off + 64 * j));
    };
    auto issue_scale_at = [&](int tok, float& sc) {
      if constexpr (KST == DT_FP8) sc = *reinterpret_cast<const float*>(sseq + (uint32_t)tok * 4u);
      else sc = 1.f;
    };
    // with kept blocks, slot u's token is kept from the issue of its keys to that of its scale
    // (the table read happens at the top of the slot, well before the issue)
    int ktok[PF];
    // the previous sub-chunk's candidate stores are complete here, so that the block loop
    // below only ever waits for its own, in-order loads; the prologue issues in the loop's
    // order (slot u: keys of its block, then the scale of the previous slot's block)
    __builtin_amdgcn_s_waitcnt(0x0F70);                            // vmcnt(0)
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int up = (u + PF - 1) % PF;
      ktok[u] = key_of(u);
      issue_keys_at(ktok[u], raw[u]);
      if constexpr (W == 8) issue_scale_at(ktok[u], scl[u]);
      else if constexpr (BLK) issue_scale_at(ktok[u == 0 ? 0 : up], scl[up]);
      else issue_scale_at(key_of(up), scl[up]);
      __builtin_amdgcn_sched_barrier(0);
    }

    f32x4v_t acc[2][NQ][HB];                                       // [set][query][head block]
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[x][j][hb] = f32x4v_t{};

    // Epilogue of a block in pieces that the slot loop spreads between the MFMAs of the next
    // block (a wave issues in order, so its VALU work overlaps the matrix core only when it sits
    // between MFMAs). Pieces 0 .. NE-1: ReLU and head weight of one accumulator element (query
    // q, head block hb, row r), in the order the MFMAs produced them; then the head sum over the
    // 4 lane groups, the scale, the LDS store and the histogram.
    constexpr int NE = NQ * HB * 4;
    constexpr int NPIECE = NE + 4;
    // A lane's 16 heads of a query are summed in one chain (consecutive links of a chain are
    // NQ pieces, at least one MFMA, apart).
    struct Epi {
      float p[NQ];
      float x[NQ];
    };
    auto piece = [&](int k, Epi& st, int i, const f32x4v_t (&ac)[NQ][HB], float sc) {
      if (k < NE) {
        const int q = k % NQ, hb = (k / NQ) % HB, r = k / (NQ * HB);
        const float t = __int_as_float(max(__float_as_int(ac[q][hb][r]), 0));
        st.p[q] = k < NQ ? wv[q][hb][r] * t : fmaf(wv[q][hb][r], t, st.p[q]);
      } else if (k == NE) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) st.x[q] = st.p[q];
      } else if (k == NE + 1) {
        if constexpr (NQ == 2) {
          // one swap for both queries: row 2m + 1 of query 0 trades places with row 2m of query
          // 1, so the sum of the outputs holds in row r the pair sum of query r % 2
          const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(st.x[0]), __float_as_uint(st.x[1]), false, false);
          st.x[0] = __uint_as_float(w[0]) + __uint_as_float(w[1]);
        } else {
          // sum of both swap outputs: the pair's total in every lane, whichever way it swaps
          const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(st.x[0]), __float_as_uint(st.x[0]), false, false);
          st.x[0] = __uint_as_float(w[0]) + __uint_as_float(w[1]);
        }
      } else if (k == NE + 2) {
        // rows r and r + 2 meet: every row holds its query's total
        const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.x[0]), __float_as_uint(st.x[0]), false, false);
        st.x[0] = __uint_as_float(w[0]) + __uint_as_float(w[1]);
      } else {
        // branch-free (a branch would end the interleave): masked lanes write to their own sink
        // words; a block before the first (i = -1) has a negative offset. Row g holds the total
        // of query g % 2 (the only one with one query)
        const float v = st.x[0] * sc;
        const int jl = (i * NW + wave) * DC_KB + n;             // offset in the sub-chunk
        const bool valid = owner & ((unsigned)jl < (unsigned)(sub1 - sub0));
        *(valid ? my_ssc + jl : sink_f) = v;
      }
    };
    auto epilogue = [&](int i, const f32x4v_t (&ac)[NQ][HB], float sc) {
      Epi st;
#pragma unroll
      for (int k = 0; k < NPIECE; ++k) piece(k, st, i, ac, sc);
    };
    auto convert = [&](const u32x4_t (&src)[NLD], int s) -> bf16x8_t {
      if constexpr (KST == DT_FP8) {
        const u32x4_t v = src[s >> 1];
        const uint32_t w0 = v[(s & 1) * 2], w1 = v[(s & 1) * 2 + 1];
        u32x4_t o;
        o[0] = fp8x2_to_bf16x2<false>(w0);
        o[1] = fp8x2_to_bf16x2<true>(w0);
        o[2] = fp8x2_to_bf16x2<false>(w1);
        o[3] = fp8x2_to_bf16x2<true>(w1);
        return __builtin_bit_cast(bf16x8_t, o);
      } else {
        return __builtin_bit_cast(bf16x8_t, src[s]);
      }
    };

    constexpr int NM = NQ * HB * NS;                                // MFMAs per block
    if constexpr (W == 8) {
      // Two waves per SIMD: one wave's MFMAs run beside the other's vector work, so a block is
      // scored in program order (convert, MFMAs, epilogue) and its head blocks are pipelined
      // (the MFMAs of head block hb + 1 are issued before the ReLU and weights of hb).
      for (int i0 = 0; i0 < iters; i0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int i = i0 + u;
          int ntok = 0;
          if constexpr (BLK) ntok = key_of(i + PF);
          bf16x8_t bfr[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) bfr[s] = convert(raw[u], s);
          // the slot's keys are converted: refill it with block i + PF
          if constexpr (BLK) {
            ktok[u] = ntok;
            issue_keys_at(ntok, raw[u]);
          } else {
            issue_keys_at(key_of(i + PF), raw[u]);
          }
          float p[NQ];
          f32x4v_t ac[2][NQ];
          auto mm = [&](int hb, f32x4v_t (&o)[NQ]) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int q = 0; q < NQ; ++q)
                o[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[q][hb][s], bfr[s], s == 0 ? f32x4v_t{} : o[q], 0, 0, 0);
          };
          auto ep = [&](int hb, const f32x4v_t (&o)[NQ]) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int q = 0; q < NQ; ++q) {
                const float t = __int_as_float(max(__float_as_int(o[q][r]), 0));
                p[q] = hb == 0 && r == 0 ? wv[q][hb][r] * t : fmaf(wv[q][hb][r], t, p[q]);
              }
          };
          mm(0, ac[0]);
#pragma unroll
          for (int hb = 1; hb < HB; ++hb) {
            mm(hb, ac[hb & 1]);
            ep(hb - 1, ac[(hb - 1) & 1]);
          }
          ep(HB - 1, ac[(HB - 1) & 1]);
          Epi st;
#pragma unroll
          for (int q = 0; q < NQ; ++q) st.p[q] = p[q];
#pragma unroll
          for (int k = NE; k < NPIECE; ++k) piece(k, st, i, acc[0], scl[u]);   // (no accumulator read)
          // the slot's scale is used: refill it with block i + PF's
          if constexpr (BLK) issue_scale_at(ktok[u], scl[u]);
          else issue_scale_at(key_of(i + PF), scl[u]);
        }
      }
    } else {
    for (int i0 = 0; i0 < iters; i0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int i = i0 + u;
        const int x = u & 1;
        const int up = (u + PF - 1) % PF;                            // slot of block i - 1
        int ntok = 0;
        if constexpr (BLK) ntok = key_of(i + PF);
        bf16x8_t bfr[NS];
        bfr[0] = convert(raw[u], 0);
        Epi st;
        __builtin_amdgcn_sched_barrier(0);
        // MFMAs of block i into set x (t = (s, hb, q), q fastest); between them the conversion
        // of the next K step, the refill of this slot once converted, and the epilogue of block
        // i - 1 from set x ^ 1
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          const int s = t / (NQ * HB), hb = (t / NQ) % HB, q = t % NQ;
          acc[x][q][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[q][hb][s], bfr[s], s == 0 ? f32x4v_t{} : acc[x][q][hb], 0, 0, 0);
          if (t % (NQ * HB) == 0 && s + 1 < NS) bfr[s + 1] = convert(raw[u], s + 1);
          if (t == (NS - 2) * NQ * HB) {
            if constexpr (BLK) {
              ktok[u] = ntok;
              issue_keys_at(ntok, raw[u]);
            } else {
              issue_keys_at(key_of(i + PF), raw[u]);
            }
          }
#pragma unroll
          for (int k = t * NPIECE / NM; k < (t + 1) * NPIECE / NM; ++k) piece(k, st, i - 1, acc[x ^ 1], scl[up]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (BLK) issue_scale_at(ktok[up], scl[up]);
        else issue_scale_at(key_of(i - 1 + PF), scl[up]);
      }
    }
    epilogue(iters - 1, acc[1], scl[PF - 1]);                      // iters is a multiple of even PF
    }
    __syncthreads();

    // ---- the sub-chunk's scores of row qq as order-preserving keys in registers, CST steps of
    // 4 NT slots at a time (the nck chunks that hold the sub-chunk): thread tid takes slots
    // j = 4 NT st + 4 tid + e (0, below every score's key, past the row's visible slots; loads
    // past them stay inside the score area)
    constexpr int CST = 4;
    const int len = sub1 - sub0;
    const int nck = (len + CST * 4 * NT - 1) / (CST * 4 * NT);
    auto load_keys = [&](int qq, int h, uint32_t (&kr)[CST][4]) {
      int lim = min(len, (qq ? V1 : V0) - sub0);                   // visible slots
      asm volatile("" : "+s"(lim));       // the masks are recomputed per call, not kept (64 pairs)
      const float* row = ssc + qq * a.sub + 4 * tid;
      f32x4_t v[CST];
#pragma unroll
      for (int u = 0; u < CST; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(row + (h * CST + u) * 4 * NT);
      __builtin_amdgcn_sched_barrier(0);         // the loads in flight together
      if (lim >= (h + 1) * CST * 4 * NT) {                         // every slot visible
#pragma unroll
        for (int u = 0; u < CST; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) kr[u][e] = f2key3(v[u][e]);
      } else {
#pragma unroll
        for (int u = 0; u < CST; ++u) {
          const int j = (h * CST + u) * 4 * NT + 4 * tid;
#pragma unroll
          for (int e = 0; e < 4; ++e) kr[u][e] = j + e < lim ? f2key3(v[u][e]) : 0u;
          __builtin_amdgcn_sched_barrier(0);     // a few compare masks live at a time, not 32
        }
      }
    };
    // first-digit histogram of each row's visible finite scores (kept out of the block loop,
    // whose VALU issue is the bottleneck)
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      if (qq < nrows) {
        uint32_t* hq = hist + qq * 2048;
        uint32_t* hsink = sink + 64 + lane;
        for (int h = 0; h < nck; ++h) {
          uint32_t kr[CST][4];
          load_keys(qq, h, kr);
#pragma unroll
          for (int u = 0; u < CST; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // branch-free: a hidden or -inf slot adds to the lane's own sink word
              const uint32_t x = kr[u][e];
              atomicAdd(x > KEY_NEG_INF ? hq + ((x >> 20) & 2047u) : hsink, 1u << ((x >> 27) & 16u));
            }
          }
        }
      }
    }
    __syncthreads();

    // ---- end of the sub-chunk. Thread t owns first-digit bins [4096 - BPT (t+1), 4096 - BPT t)
    // of both rows and finds the bin b of each row's k-th largest score in this sub-chunk (both
    // rows' counts packed in one word: each <= DC_SUB).
    // The keys in bins >= b are this sub-chunk's candidates.
    constexpr int BPT = DC_BINS / NT;                       // bins per thread
    static_assert(BPT % 8 == 0, "whole 16-byte reads of packed bins");
    uint32_t bins[2][BPT];
    uint32_t part = 0;
    const int seg = sub0 / a.sub;
    const int blo = DC_BINS - BPT * (tid + 1);                     // bins [blo, blo + BPT)
    const int w0 = blo & 2047, hsh = blo >= 2048 ? 16 : 0;         // their words and half
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      uint32_t sum = 0;
      // the selector sums the sub-chunks' histograms (every key in a bin at or above a
      // sub-chunk's bound is one of its candidates); the first half of the threads holds every
      // word once
      uint32_t* hout = a.shist + ((qq ? r1 : r0) * a.nsegs + seg) * (DC_BINS / 2) + w0;
#pragma unroll
      for (int c = 0; c < BPT / 4; ++c) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(hist + qq * 2048 + w0 + 4 * c);
        if ((qq < nrows) & (tid < NT / 2)) reinterpret_cast<u32x4_t*>(hout)[c] = w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bins[qq][4 * c + e] = (w[e] >> hsh) & 0xFFFFu;
          sum += bins[qq][4 * c + e];
        }
      }
      part |= sum << (16 * qq);
    }
    const uint32_t inc = wave_scan_dpp(part);      // thread order = descending bins
    if (lane == 63) misc[16 + wave] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? misc[16 + w] : 0u;
      total += misc[16 + w];
    }
    const uint32_t ex = before + inc - part;
    const uint32_t k = (uint32_t)a.k;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      if (tid == 0) {
        misc[4 * qq + 0] = KEY_NEG_INF + 1u;     // every finite score, unless cut below
        misc[4 * qq + 1] = (total >> (16 * qq)) & 0xFFFFu;
      }
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const uint32_t exq = (ex >> (16 * qq)) & 0xFFFFu, sq = (part >> (16 * qq)) & 0xFFFFu;
      if (exq < k && k <= exq + sq) {
        uint32_t run = exq;
#pragma unroll
        for (int e = BPT - 1; e >= 0; --e) {
          if (run + bins[qq][e] >= k) {
            misc[4 * qq + 0] = (uint32_t)(DC_BINS - BPT * (tid + 1) + e) << 20;
            misc[4 * qq + 1] = run + bins[qq][e];
            break;
          }
          run += bins[qq][e];
        }
      }
    }
    __syncthreads();
    // ---- candidates (order-preserving key, slot) at or above each row's bound, written to the
    // sub-chunk's own slots of the row's candidate list (a key is a candidate of one sub-chunk
    // only) in any order: a wave reserves its run with one LDS atomic, then writes its entries
    // one register at a time, the lanes that hold one at consecutive positions (ballot rank)
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      if (qq < nrows) {
        // a candidate: a finite score's key at or above the bound (keys of hidden slots are 0)
        const uint32_t thr = max(misc[4 * qq], KEY_NEG_INF + 1u);
        uint32_t n = 0;                                              // the wave's count
        for (int h = 0; h < nck; ++h) {
          uint32_t kr[CST][4];
          load_keys(qq, h, kr);
#pragma unroll
          for (int u = 0; u < CST; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) n += (uint32_t)__popcll(__ballot(kr[u][e] >= thr));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        uint32_t pos = 0;
        if (lane == 0 && n) pos = atomicAdd(&misc[12 + qq], n);
        pos = (uint32_t)sub0 + wave_bcast(pos, 0);
        const int64_t rr = qq ? r1 : r0;
        // byte offsets below 2^32 from uniform bases (one row's list)
        uint8_t* ck = reinterpret_cast<uint8_t*>(a.cand_key + rr * a.cand_cap);
        uint8_t* ci = reinterpret_cast<uint8_t*>(a.cand_idx + rr * a.cand_cap);
        const uint32_t slot0 = (uint32_t)(sub0 + 4 * tid);
        for (int h = 0; h < nck; ++h) {
          uint32_t kr[CST][4];
          load_keys(qq, h, kr);
#pragma unroll
          for (int u = 0; u < CST; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = kr[u][e];
              const bool f = x >= thr;
              const uint64_t m = __ballot(f);
              if (f) {
                const uint32_t at = 4u * (pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)));
                *reinterpret_cast<uint32_t*>(ck + at) = x;
                *reinterpret_cast<uint32_t*>(ci + at) = slot0 + (uint32_t)((h * CST + u) * 4 * NT + e);
              }
              pos += (uint32_t)__popcll(m);
              __builtin_amdgcn_sched_barrier(0);                   // one register's masks live at a time
            }
          }
        }
      }
    }
    __syncthreads();
    // the sub-chunk's candidate count (read by thread qq, the one that clears the row's counter
    // at the next sub-chunk's start)
    if (tid < nrows) a.ccount[(tid ? r1 : r0) * a.nsegs + seg] = misc[12 + tid];
  }
}

// Bin of the need-th largest element of a 4096-bin histogram in LDS, by all RS_THREADS threads
// (thread t holds the 8 bins below 4096 - 8 t): out = {bin or ~0u if need exceeds the total, count
// in higher bins}. sh: RS_WAVES words of scratch.
constexpr int RS_THREADS = 512;
constexpr int RS_WAVES = RS_THREADS / 64;
constexpr int RS_LDS_CAND = 4096;
constexpr int RS_R = 64;                                  // candidate chunks held in registers

__device__ __forceinline__ void block_find_desc(const uint32_t* h, uint32_t need, uint32_t* sh, uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = DC_BINS - 8 * (tid + 1);                 // bins [lo, lo + 8)
  const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(h + lo);
  const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(h + lo + 4);
  const uint32_t c[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) sum += c[e];
  const uint32_t inc = wave_scan_dpp(sum);
  if (lane == 63) sh[wave] = inc;
  if (tid == 0) {
    out[0] = ~0u;
    out[1] = 0u;
  }
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < RS_WAVES; ++w) before += w < wave ? sh[w] : 0u;
  const uint32_t ex = before + inc - sum;                 // count in higher bins than mine
  if (ex < need && need <= ex + sum) {
    uint32_t run = ex;
#pragma unroll
    for (int e = 7; e >= 0; --e) {
      if (run + c[e] >= need) {
        out[0] = (uint32_t)(lo + e);
        out[1] = run;
        break;
      }
      run += c[e];
    }
  }
  __syncthreads();
}

// One work-group per row. The row's candidates (per sub-chunk lists written by the scan) hold
// every key the selection can take, and at least min(k, finite slots) keys, so the selection
// is the top min(k, M) of the M candidates: the 12-bit bin b1 of the k-th largest from their
// histogram, candidates above b1 written out, the ones in b1 resolved exactly with two more
// 10-bit digits and, for ties at the k-th key, three digits of the complemented slot (lowest
// slots first); then the padding.

__global__ void __launch_bounds__(RS_THREADS) decode_select_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint32_t hist[DC_BINS + 128];       // + per-lane sink words (staging)
  __shared__ uint32_t ckey[RS_LDS_CAND + 64];                     // + per-lane sink entries
  __shared__ uint32_t cpos[RS_LDS_CAND + 64];
  __shared__ uint32_t sh[RS_WAVES];
  __shared__ uint32_t wsum[2 * RS_WAVES];
  __shared__ __align__(16) uint32_t cbase[RS_R];
  __shared__ __align__(16) int clim[RS_R];
  __shared__ uint32_t bc[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const uint32_t* counts = a.ccount + r * a.nsegs;
  const uint32_t* gk = a.cand_key + r * a.cand_cap;
  const uint32_t* gi = a.cand_idx + r * a.cand_cap;
  uint32_t* g2k = a.cand2_key + r * a.cand_cap;
  uint32_t* g2p = a.cand2_idx + r * a.cand_cap;
  int32_t* oidx = a.out_idx + r * a.k;
  float* osc = a.out_score ? a.out_score + r * a.k : nullptr;
  // slot -> token (kept-block slots through the row's table; the selected slots are visible, so
  // inside the kept blocks)
  const int32_t* tab = a.blocks ? a.blocks + ((r / a.T) * a.n_groups + (r % a.T) / a.group_size) * a.keep_stride
                                : nullptr;
  auto tok = [&](uint32_t sl) -> int32_t {
    if (!tab) return (int32_t)sl;
    return (tab[sl >> a.blk_shift] << a.blk_shift) | (int32_t)(sl & ((1u << a.blk_shift) - 1u));
  };

  // ---- candidate count M
  uint32_t M = 0;
  {
    uint32_t part = 0;
    for (int sg = tid; sg < a.nsegs; sg += RS_THREADS) part += counts[sg];
    const uint32_t inc = wave_scan_dpp(part);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) M += sh[w];
    __syncthreads();
  }
  const uint32_t kk = min((uint32_t)a.k, M);
  const bool all = kk == M;

  for (int i = tid; i < DC_BINS; i += RS_THREADS) hist[i] = 0u;
  if (tid == 0) {
    bc[4] = 0u;                                  // written
    bc[5] = 0u;                                  // bin-b1 candidates
  }
  __syncthreads();

  // Visits the candidates in batches of RS_U * RS_THREADS of one segment (key, and slot when
  // IDX), the next batch's loads in flight while f runs on the current one: f(ok[], x[], i[]).
  constexpr int RS_U = 4;
  struct Batch {
    uint32_t x[RS_U], i[RS_U];
    bool ok[RS_U];
  };
  auto advance = [&](int& sg, int& j0) {                  // next batch (uniform)
    j0 += RS_U * RS_THREADS;
    while (sg < a.nsegs && j0 >= (int)counts[sg]) {
      ++sg;
      j0 = 0;
    }
  };
  auto for_batches = [&](auto f, auto idx_tag) {
    constexpr bool IDX = decltype(idx_tag)::value;
    auto load = [&](int sg, int j0, Batch& bt) {
      const int c = (int)counts[sg];
      const uint32_t base = (uint32_t)sg * (uint32_t)a.sub;
#pragma unroll
      for (int u = 0; u < RS_U; ++u) {
        const int j = j0 + u * RS_THREADS + tid;
        const uint32_t p = base + (uint32_t)min(j, c - 1);
        bt.ok[u] = j < c;
        bt.x[u] = gk[p];
        if constexpr (IDX) bt.i[u] = gi[p];
        else bt.i[u] = 0u;
      }
    };
    int sg = 0, j0 = -RS_U * RS_THREADS;
    advance(sg, j0);
    Batch A, B;
    if (sg < a.nsegs) load(sg, j0, A);
    while (sg < a.nsegs) {
      advance(sg, j0);
      if (sg < a.nsegs) load(sg, j0, B);
      f(A);
      if (sg >= a.nsegs) break;
      advance(sg, j0);
      if (sg < a.nsegs) load(sg, j0, A);
      f(B);
    }
  };

  // ---- first-digit histogram and bin b1 of the kk-th largest: the sum of the sub-chunks'
  // histograms, exact in every bin at or above the highest sub-chunk bound. Some sub-chunk
  // holds k keys at or above its own bound when M > kk, so b1 is at or above every bound.
  if (!all) {
    const int lo = DC_BINS - 8 * (tid + 1);               // this thread's bins [lo, lo + 8)
    uint32_t hs[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    const uint32_t* src = a.shist + r * a.nsegs * (DC_BINS / 2) + (lo & 2047);
    const int hsh = lo >= 2048 ? 16 : 0;
#pragma unroll 4
    for (int sg = 0; sg < a.nsegs; ++sg) {
      // a sub-chunk without candidates has no keys (and a histogram that was never written)
      const uint32_t keep = counts[sg] ? 0xFFFFu : 0u;
      const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(src + (size_t)sg * (DC_BINS / 2));
      const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(src + (size_t)sg * (DC_BINS / 2) + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hs[e] += (v0[e] >> hsh) & keep;
        hs[4 + e] += (v1[e] >> hsh) & keep;
      }
    }
    *reinterpret_cast<u32x4_t*>(hist + lo) = u32x4_t{hs[0], hs[1], hs[2], hs[3]};
    *reinterpret_cast<u32x4_t*>(hist + lo + 4) = u32x4_t{hs[4], hs[5], hs[6], hs[7]};
  }
  __syncthreads();
  uint32_t b1 = 0, above = 0;
  if (!all) {
    block_find_desc(hist, kk, sh, bc);
    b1 = bc[0];
    above = bc[1];
  }

  // ---- pass 2: candidates above b1 out (all when every candidate is selected), bin b1 kept
  // as (key, slot). Up to RS_R chunks of RS_THREADS candidates (one segment each) are loaded
  // at once and held in registers; a row with more streams them in batches instead.
  // chunk table: chunk u = candidates [cbase[u], cbase[u] + clim[u]) of one segment, at most
  // RS_THREADS; held when every candidate is in the first RS_R chunks (and there are at most
  // 64 segments: lane g of wave 0 lays out segment g's chunks)
  if (wave == 0) {
    const int c = lane < a.nsegs ? (int)counts[lane] : 0;
    const uint32_t nch = (uint32_t)(c + RS_THREADS - 1) / RS_THREADS;
    const uint32_t inc = wave_scan_dpp(nch);
    const uint32_t tot = wave_bcast(inc, 63);
    const bool fits = a.nsegs <= 64 && tot <= (uint32_t)RS_R;
    if (fits) {
      for (uint32_t q = 0; q < nch; ++q) {
        const uint32_t u = inc - nch + q;
        cbase[u] = (uint32_t)lane * (uint32_t)a.sub + q * RS_THREADS;
        clim[u] = min(c - (int)(q * RS_THREADS), RS_THREADS);
      }
      for (uint32_t u = tot + lane; u < (uint32_t)RS_R; u += 64) {
        cbase[u] = 0u;
        clim[u] = 0;
      }
    }
    if (lane == 0) {
      bc[6] = fits ? 1u : 0u;
      bc[7] = tot;                                         // chunks in use
    }
  }
  __syncthreads();
  const bool held = kk > 0 && bc[6] != 0u;
  // the held path's selections above b1 (fewer than kk) are staged in the histogram's LDS (free
  // until the bin-b1 passes) and written out together: stores into global memory inside its loop
  // made every iteration wait for the previous ones
  const bool stage = held && kk <= (uint32_t)(DC_BINS / 2);
  if (held) {
    // keys; 0 (below every finite score's key) where a chunk has no candidate. The loops stop
    // at the chunks in use (a uniform bound; the register arrays stay statically indexed)
    const int nchk = (int)bc[7];
    uint32_t xr[RS_R], ir[RS_R];                           // key and slot
#pragma unroll
    for (int u = 0; u < RS_R; ++u) {
      xr[u] = 0u;
      ir[u] = 0u;
    }
#pragma unroll
    for (int u = 0; u < RS_R; u += 4) {
      if (u < nchk) {
        const u32x4_t cb = *reinterpret_cast<const u32x4_t*>(cbase + u);
        const int4 cl = *reinterpret_cast<const int4*>(clim + u);
        const int lim[4] = {cl.x, cl.y, cl.z, cl.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (tid < lim[e]) {
            xr[u + e] = gk[cb[e] + (uint32_t)tid];
            ir[u + e] = gi[cb[e] + (uint32_t)tid];
          }
        }
      }
    }
    // selected: above b1 (every candidate when all are taken); bin-b1 candidates: in b1. One
    // compare each on the key (candidates are finite, so b1 >= 8 unless all are taken; an empty
    // register holds 0, neither)
    const uint32_t sel_gt = all ? KEY_NEG_INF : (uint32_t)(((uint64_t)b1 + 1u << 20) - 1u);
    const uint32_t clo = b1 << 20, cwid = all ? 0u : (1u << 20);
    auto is_sel = [&](uint32_t x, uint32_t) { return x > sel_gt; };
    auto is_cand = [&](uint32_t x, uint32_t) { return x - clo < cwid; };
    // per-wave counts, then each wave writes its candidates from its own offsets
    uint32_t cs = 0, cq = 0;                               // this lane's counts
#pragma unroll
    for (int u = 0; u < RS_R; ++u) {
      if (u < nchk) {
        cs += is_sel(xr[u], b1) ? 1u : 0u;
        cq += is_cand(xr[u], b1) ? 1u : 0u;
      }
    }
    const uint32_t cs_own = cs, cq_own = cq;
    cs = wave_scan_dpp(cs);
    cq = wave_scan_dpp(cq);
    if (lane == 63) {
      wsum[wave] = cs;
      wsum[RS_WAVES + wave] = cq;
    }
    __syncthreads();
    uint32_t ps = 0, pc = 0;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) {
      ps += w < wave ? wsum[w] : 0u;
      pc += w < wave ? wsum[RS_WAVES + w] : 0u;
    }
    if (tid == 0) {
      uint32_t ts = 0, tq = 0;
#pragma unroll
      for (int w = 0; w < RS_WAVES; ++w) {
        ts += wsum[w];
        tq += wsum[RS_WAVES + w];
      }
      bc[4] = ts;
      bc[5] = tq;
    }
    // the masks are recomputed below rather than kept from the count loop (RS_R x 2 masks)
    uint32_t b1x = b1;
    asm volatile("" : "+v"(b1x));
#pragma unroll
    for (int u = 0; u < RS_R; ++u) asm volatile("" : "+v"(xr[u]));
    if (stage) {
      // lane order instead of chunk order: each lane writes its own entries from its offset (the
      // exclusive scan of the counts above), without ballots, without branches (an entry a lane
      // does not keep goes to its own sink words); chunks in groups of 4 (one uniform test each)
      uint32_t ls = ps + cs - cs_own, lc = pc + cq - cq_own;
      auto emit = [&](auto spill_tag) {
        constexpr bool SPILL = decltype(spill_tag)::value;       // bin-b1 candidates past the LDS
#pragma unroll
        for (int u0 = 0; u0 < RS_R; u0 += 4) {
          if (u0 >= nchk) break;
#pragma unroll
          for (int u = u0; u < u0 + 4; ++u) {
            const bool sel = is_sel(xr[u], b1x), cand = is_cand(xr[u], b1x);
            // (fewer than kk <= DC_BINS / 2 are selected here, so ls stays inside the staging area)
            const uint32_t at = sel ? 2u * ls : (uint32_t)DC_BINS + 2u * (uint32_t)lane;
            hist[at] = ir[u];
            hist[at + 1] = xr[u];
            const uint32_t cl = (cand && (!SPILL || lc < (uint32_t)RS_LDS_CAND)) ? lc : (uint32_t)RS_LDS_CAND + (uint32_t)lane;
            ckey[cl] = xr[u];
            cpos[cl] = ir[u];
            if (SPILL && cand && lc >= (uint32_t)RS_LDS_CAND) {
              g2k[lc] = xr[u];
              g2p[lc] = ir[u];
            }
            ls += sel ? 1u : 0u;
            lc += cand ? 1u : 0u;
          }
        }
      };
      if (pc + (uint32_t)__builtin_amdgcn_readfirstlane(wsum[RS_WAVES + wave]) <= (uint32_t)RS_LDS_CAND) emit(std::false_type{});
      else emit(std::true_type{});
    }
#pragma unroll
    for (int u = 0; u < RS_R; ++u) {
      if (stage || u >= nchk) continue;
      const bool sel = is_sel(xr[u], b1x), cand = is_cand(xr[u], b1x);
      const uint64_t ms = __ballot(sel), mc = __ballot(cand);
      const uint32_t sl = ir[u];
      if (sel) {
        const uint32_t pos = ps + __builtin_amdgcn_mbcnt_hi((uint32_t)(ms >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ms, 0u));
        oidx[pos] = tok(sl);
        if (osc) osc[pos] = key2f(xr[u]);
      }
      if (cand) {
        const uint32_t cp = pc + __builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0u));
        if (cp < (uint32_t)RS_LDS_CAND) {
          ckey[cp] = xr[u];
          cpos[cp] = sl;
        } else {
          g2k[cp] = xr[u];
          g2p[cp] = sl;
        }
      }
      ps += (uint32_t)__popcll(ms);
      pc += (uint32_t)__popcll(mc);
    }
  }
  if (kk > 0 && !held) {
    for_batches([&](const Batch& bt) {
      uint64_t ms[RS_U], mc[RS_U];
      uint32_t ns = 0, nq = 0;
#pragma unroll
      for (int u = 0; u < RS_U; ++u) {
        ms[u] = __ballot(bt.ok[u] && (all || (bt.x[u] >> 20) > b1));
        mc[u] = __ballot(bt.ok[u] && !all && (bt.x[u] >> 20) == b1);
        ns += (uint32_t)__popcll(ms[u]);
        nq += (uint32_t)__popcll(mc[u]);
      }
      uint32_t ps = 0, pc = 0;
      if (lane == 0) {
        if (ns) ps = atomicAdd(&bc[4], ns);
        if (nq) pc = atomicAdd(&bc[5], nq);
      }
      ps = wave_bcast(ps, 0);
      pc = wave_bcast(pc, 0);
#pragma unroll
      for (int u = 0; u < RS_U; ++u) {
        const uint32_t bs = __builtin_amdgcn_mbcnt_hi((uint32_t)(ms[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ms[u], 0u));
        const uint32_t bq = __builtin_amdgcn_mbcnt_hi((uint32_t)(mc[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mc[u], 0u));
        if ((ms[u] >> lane) & 1u) {
          oidx[ps + bs] = tok(bt.i[u]);
          if (osc) osc[ps + bs] = key2f(bt.x[u]);
        }
        if ((mc[u] >> lane) & 1u) {
          const uint32_t cp = pc + bq;
          if (cp < (uint32_t)RS_LDS_CAND) {
            ckey[cp] = bt.x[u];
            cpos[cp] = bt.i[u];
          } else {
            g2k[cp] = bt.x[u];
            g2p[cp] = bt.i[u];
          }
        }
        ps += (uint32_t)__popcll(ms[u]);
        pc += (uint32_t)__popcll(mc[u]);
      }
    }, std::true_type{});
  }
  __syncthreads();
  if (stage) {
    for (uint32_t i = tid; i < min(bc[4], (uint32_t)(DC_BINS / 2)); i += RS_THREADS) {
      const uint32_t sl = hist[2 * i], x = hist[2 * i + 1];
      oidx[i] = tok(sl);
      if (osc) osc[i] = key2f(x);
    }
    __syncthreads();
  }

  if (kk > 0 && !all) {
    const uint32_t nc = bc[5];
    auto get = [&](uint32_t j, uint32_t& x, uint32_t& i) {
      if (j < (uint32_t)RS_LDS_CAND) {
        x = ckey[j];
        i = cpos[j];
      } else {
        x = g2k[j];
        i = g2p[j];
      }
    };
    // one radix pass over the bin-b1 candidates: histogram of digit(x, i) over the matching
    // ones, then the bin holding the need-th largest; out = {bin, count above it, count in it}
    auto pass = [&](auto match, auto digit, int nb, uint32_t need, uint32_t* out) {
      __syncthreads();
      for (int q = tid; q < nb; q += RS_THREADS) hist[q] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < nc; j += RS_THREADS) {
        uint32_t x, i;
        get(j, x, i);
        if (match(x, i)) atomicAdd(&hist[digit(x, i)], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        int bn;
        uint32_t ab;
        wave_hist_find(hist, nb, need, &bn, &ab);
        if (lane == 0) {
          bc[0] = (uint32_t)max(bn, 0);
          bc[1] = ab;
          bc[2] = bn >= 0 ? hist[bn] : 0u;
        }
      }
      __syncthreads();
      out[0] = bc[0];
      out[1] = bc[1];
      out[2] = bc[2];
    };
    uint32_t need = kk - above;
    uint32_t rr[3];
    pass([&](uint32_t, uint32_t) { return true; },
         [&](uint32_t x, uint32_t) { return (x >> 10) & 0x3FFu; }, 1024, need, rr);
    const uint32_t pre2 = (b1 << 10) | rr[0];
    need -= rr[1];
    pass([&](uint32_t x, uint32_t) { return (x >> 10) == pre2; },
         [&](uint32_t x, uint32_t) { return x & 0x3FFu; }, 1024, need, rr);
    const uint32_t T = (pre2 << 10) | rr[0];
    const uint32_t need_eq = need - rr[1], n_eq = rr[2];
    uint32_t CI = 0u;                         // ties kept: complemented slot >= CI
    if (n_eq != need_eq) {
      pass([&](uint32_t x, uint32_t) { return x == T; },
           [&](uint32_t, uint32_t i) { return (~i) >> 21; }, 2048, need_eq, rr);
      const uint32_t d4 = rr[0];
      uint32_t ne = need_eq - rr[1];
      pass([&](uint32_t x, uint32_t i) { return x == T && ((~i) >> 21) == d4; },
           [&](uint32_t, uint32_t i) { return ((~i) >> 10) & 0x7FFu; }, 2048, ne, rr);
      const uint32_t d5 = (d4 << 11) | rr[0];
      ne -= rr[1];
      pass([&](uint32_t x, uint32_t i) { return x == T && ((~i) >> 10) == d5; },
           [&](uint32_t, uint32_t i) { return (~i) & 0x3FFu; }, 1024, ne, rr);
      CI = (d5 << 10) | rr[0];
    }
    // the rest follow the candidates above b1
    for (uint32_t j0 = 0; j0 < nc; j0 += RS_THREADS) {
      const uint32_t j = j0 + tid;
      bool sel = false;
      uint32_t x = 0, i = 0;
      if (j < nc) {
        get(j, x, i);
        sel = x > T || (x == T && ~i >= CI);
      }
      const uint64_t m = __ballot(sel);
      uint32_t pb = 0;
      if (lane == 0 && m) pb = atomicAdd(&bc[4], (uint32_t)__popcll(m));
      pb = wave_bcast(pb, 0);
      if (sel) {
        const uint32_t pos = pb + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        oidx[pos] = tok(i);
        if (osc) osc[pos] = key2f(x);
      }
    }
  }
  if (a.out_cnt != nullptr && tid == 0) a.out_cnt[r] = (int32_t)kk;
  for (int p = (int)kk + tid; p < a.k; p += RS_THREADS) {
    oidx[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
}

bool decode_supported(int q_dtype, int k_dtype, int H, int D, int T, int N) {
  // 32-bit byte offsets within one sequence's keys
  const int64_t seq_bytes = (int64_t)N * D * (k_dtype == DT_FP8 ? 1 : 2);
  return q_dtype == DT_BF16 && (k_dtype == DT_FP8 || k_dtype == DT_BF16) && H <= 64 &&
         (D == 64 || D == 128) && T <= 4 && N >= 2048 && seq_bytes < (int64_t(1) << 31);
}

bool decode_blocks_supported(int q_dtype, int k_dtype, int H, int D, int T, int N, int block_size, int keep) {
  return decode_supported(q_dtype, k_dtype, H, D, T, N) && block_size >= DC_KB &&
         (block_size & (block_size - 1)) == 0 && keep <= DECODE_KEEP_MAX;
}

size_t decode_scan_lds(int keep) {
  return (size_t)8 * DC_SUB + 2 * 2048 * 4 + (32 + 128) * 4 + (size_t)4 * keep;
}

template <int D, int HB, int KST>
static hipError_t launch_scan(const DecodeArgs& a, hipStream_t s) {
  constexpr int W = D == 64 ? 8 : 4, PF = dc_pf<KST, W>();
  const bool blk = a.blocks != nullptr;
  // one query per work-group (pairs of one, or a single query per sequence): half the MFMAs and
  // epilogue per key block
  const bool one = a.pair == 1 || a.T == 1;
  auto kfn = blk ? (one ? decode_scan_kernel<D, HB, KST, PF, true, 1, W> : decode_scan_kernel<D, HB, KST, PF, true, 2, W>)
                 : (one ? decode_scan_kernel<D, HB, KST, PF, false, 1, W> : decode_scan_kernel<D, HB, KST, PF, false, 2, W>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)decode_scan_lds(blk ? DECODE_KEEP_MAX : 0));
  if (e != hipSuccess) return e;
  dim3 grid(a.B * a.nchunk, (a.T + a.pair - 1) / a.pair);
  hipLaunchKernelGGL(kfn, grid, dim3(W * 64), decode_scan_lds(blk ? a.keep_stride : 0), s, a);
  return hipGetLastError();
}

template <int D, int KST>
static hipError_t launch_scan_h(const DecodeArgs& a, hipStream_t s) {
  const int hb = (a.H + 15) / 16;
  if (hb == 1) return launch_scan<D, 1, KST>(a, s);
  if (hb == 2) return launch_scan<D, 2, KST>(a, s);
  return launch_scan<D, 4, KST>(a, s);
}

hipError_t launch_decode_scan(const DecodeArgs& a, hipStream_t s) {
  if (a.sub < DC_KB || a.sub > DC_SUB || a.sub % 64) return hipErrorInvalidValue;
  if (a.pair != 1 && a.pair != 2) return hipErrorInvalidValue;
  if (a.blocks && (a.keep_stride < 1 || a.keep_stride > DECODE_KEEP_MAX || a.blk_shift < 4 ||
                   a.group_size < 1 || (a.pair == 2 && a.group_size % 2) || !a.n_kept))
    return hipErrorInvalidValue;
  if (a.k_dtype == DT_FP8)
    return a.D == 128 ? launch_scan_h<128, DT_FP8>(a, s) : launch_scan_h<64, DT_FP8>(a, s);
  return a.D == 128 ? launch_scan_h<128, DT_BF16>(a, s) : launch_scan_h<64, DT_BF16>(a, s);
}

hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_select_kernel, dim3(a.B * a.T), dim3(RS_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
