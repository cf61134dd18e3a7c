// LDS key tiles and the per-wave MFMA tile + fused epilogue, shared by the score kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace idx {

template <class Mma, int D, int KT>
struct Geo {
  static constexpr int EB = Mma::kElemBytes;
  static constexpr int ROW_BYTES = D * EB;
  static constexpr int CPR = ROW_BYTES / 16;          // 16-byte chunks per key row
  static constexpr int EPC = 16 / EB;                 // elements per chunk
  static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  // rows shorter than the 256-byte bank cycle: consecutive rows share it, so the XOR key is the
  // row index with those rows folded together (then 16 rows read by one phase of a 16-byte
  // read land in 16 distinct 16-byte bank groups)
  static constexpr int SWZ_SH = ROW_BYTES >= 256 ? 0 : (ROW_BYTES == 128 ? 1 : 2);
  static constexpr int TILE_BYTES = KT * ROW_BYTES;
  static constexpr int NKK = D / 2 / Mma::E;          // MFMA steps per 32x32 tile
  static constexpr int CPF = Mma::E * EB / 16;        // 16-byte chunks per lane per fragment
};

template <int HB> struct WavesFor { static constexpr int value = (HB <= 2) ? 8 : 4; };

// Byte offset inside a tile of logical 16-byte chunk c of key row n (XOR swizzle: the 32 rows a
// wave reads in one step start in different banks).
template <class G>
__device__ __forceinline__ int swz(int n) { return (n >> G::SWZ_SH) & G::SWZ; }

template <class G>
__device__ __forceinline__ int chunk_off(int n, int c) {
  return n * G::ROW_BYTES + ((c ^ swz<G>(n)) << 4);
}

// Stages one tile of KT keys from global memory (any key storage format) into LDS in the MFMA
// element format, through registers. Global loads are issued early (load) and written to LDS
// later (store) so that their latency overlaps the current tile's MFMA work.
template <class Mma, int D, int KST, int NTHR, int KT>
struct TileLoader {
  typedef Geo<Mma, D, KT> G;
  static constexpr int NCH = KT * G::CPR;
  static constexpr int ITERS = (NCH + NTHR - 1) / NTHR;
  static constexpr int SRC_EB = (KST == DT_F32 ? 4 : (KST == DT_BF16 ? 2 : 1));
  static constexpr int SRC_BYTES = G::EPC * SRC_EB;
  u32x4_t raw[ITERS];

  template <class KeyAt>
  __device__ __forceinline__ void load(const uint8_t* kseq, int tid, KeyAt key_at) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int cid = tid + i * NTHR;
      raw[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (NCH % NTHR == 0 || cid < NCH) {
        const int n = cid / G::CPR, c = cid % G::CPR;
        const int ki = key_at(n);
        if (ki >= 0) {
          const uint8_t* src = kseq + (int64_t)ki * (D * SRC_EB) + c * SRC_BYTES;
          if constexpr (SRC_BYTES == 16) {
            raw[i] = *reinterpret_cast<const u32x4_t*>(src);
          } else if constexpr (SRC_BYTES == 8) {
            u32x2_t v = *reinterpret_cast<const u32x2_t*>(src);
            raw[i][0] = v[0];
            raw[i][1] = v[1];
          } else {
            raw[i][0] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
      }
    }
  }

  __device__ __forceinline__ static u32x4_t convert(u32x4_t v) {
    if constexpr (Mma::E == 8) {              // -> 8 bf16
      if constexpr (KST == DT_BF16) {
        return v;
      } else {                                 // fp8: 8 bytes in v[0], v[1]
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t word = v[p >> 1] >> ((p & 1) * 16);
          o[p] = e4m3_to_bf16_bits(word & 0xFFu) | (e4m3_to_bf16_bits((word >> 8) & 0xFFu) << 16);
        }
        return o;
      }
    } else {                                   // -> 4 fp32
      if constexpr (KST == DT_F32) {
        return v;
      } else if constexpr (KST == DT_BF16) {   // 4 bf16 in v[0], v[1]
        u32x4_t o;
        o[0] = v[0] << 16; o[1] = v[0] & 0xFFFF0000u;
        o[2] = v[1] << 16; o[3] = v[1] & 0xFFFF0000u;
        return o;
      } else {                                 // 4 fp8 in v[0]
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = e4m3_to_bf16_bits((v[0] >> (8 * p)) & 0xFFu) << 16;
        return o;
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int cid = tid + i * NTHR;
      if (NCH % NTHR == 0 || cid < NCH) {
        const int n = cid / G::CPR, c = cid % G::CPR;
        *reinterpret_cast<u32x4_t*>(tile + chunk_off<G>(n, c)) = convert(raw[i]);
      }
    }
  }
};

// Direct global->LDS staging (global_load_lds_dwordx4) for keys already in the MFMA element
// format: no staging registers. Each load instruction of a wave fills 1 KB of LDS, lane i
// writing bytes [16 i, 16 i + 16); the lane therefore fetches the global chunk that the
// swizzled layout puts at that position. Invalid keys fetch key row 0 of the sequence (finite
// data whose scores are never stored). Completion: s_waitcnt vmcnt(0) before the barrier.
template <class Mma, int D, int NTHR, int KT>
struct DirectLoader {
  typedef Geo<Mma, D, KT> G;
  static constexpr int NCH = KT * G::CPR;
  static constexpr int NWAVE = NTHR / 64;
  static constexpr int ITERS = NCH / NTHR > 0 ? NCH / NTHR : 1;

  // key row and logical chunk that this lane's i-th load fills
  __device__ __forceinline__ static int phys(int i, int wave, int lane) {
    return (i * NWAVE + wave) * 64 + lane;
  }
  __device__ __forceinline__ static int row_of(int i, int wave, int lane) {
    return phys(i, wave, lane) / G::CPR;
  }
  __device__ __forceinline__ static bool first_chunk(int i, int wave, int lane) {
    return phys(i, wave, lane) % G::CPR == 0;
  }

  // The i-th of this lane's chunks: ki = key index (row of the sequence's key array) of
  // row_of(i), or -1 for an unused row (then row 0 is read and never used).
  __device__ __forceinline__ static void load_chunk(int i, const uint8_t* kseq, uint8_t* tile,
                                                    int wave, int lane, int ki) {
    static_assert(NCH % NTHR == 0, "tile chunks must divide over the work-group");
    const int blk = i * NWAVE + wave;                // 1 KB LDS block written by this instr
    const int p = blk * 64 + lane;
    const int n = p / G::CPR, cp = p % G::CPR;
    const int c = cp ^ swz<G>(n);                    // logical chunk stored at p
    const uint8_t* src = kseq + (int64_t)(ki >= 0 ? ki : 0) * G::ROW_BYTES + c * 16;
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                              reinterpret_cast<uintptr_t>(tile + blk * 1024)),
                                     16, 0, 0);
  }

  template <int N>
  __device__ __forceinline__ static void load_idx(const uint8_t* kseq, uint8_t* tile, int wave,
                                                  int lane, const int (&kidx)[N]) {
    static_assert(N == ITERS, "one key index per chunk");
#pragma unroll
    for (int i = 0; i < ITERS; ++i) load_chunk(i, kseq, tile, wave, lane, kidx[i]);
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work-group barrier for reusing LDS tiles: waits for this wave's LDS operations only, then
// s_barrier. Unlike __syncthreads() it does not first wait for the wave's global stores (the
// score rows) to complete, which would put a store round trip on every tile.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}

// ReLU through an integer max: an IEEE float is negative iff its bit pattern is negative as an
// int32, so max(bits, 0) is bits(x) for x >= +0 and +0 otherwise (one VALU op, no NaN quieting).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// B fragment kk of key row n for lane half hh (direct paths): CPF consecutive logical chunks,
// starting at chunk CPF (hh NKK + kk); queries are loaded with the same element order.
template <class Mma, class G>
__device__ __forceinline__ typename Mma::frag_t read_frag(const uint8_t* tile, int n, int hh, int kk) {
  if constexpr (G::CPF == 1) {
    return *reinterpret_cast<const typename Mma::frag_t*>(tile + chunk_off<G>(n, hh * G::NKK + kk));
  } else {
    static_assert(G::CPF == 2, "one or two 16-byte chunks per fragment");
    const int c = 2 * (hh * G::NKK + kk);
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(tile + chunk_off<G>(n, c));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(tile + chunk_off<G>(n, c + 1));
    return typename Mma::frag_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

// One wave: x = q(32*HB heads) . k(32 keys of the tile starting at row n0) accumulated in acc.
template <class Mma, int D, int HB, int KT>
__device__ __forceinline__ void tile_mma(const typename Mma::frag_t (&qf)[HB][Geo<Mma, D, KT>::NKK],
                                         const uint8_t* tile, int n0, int lane,
                                         f32x16_t (&acc)[HB]) {
  typedef Geo<Mma, D, KT> G;
  const int hh = lane >> 5;
  const int n = n0 + (lane & 31);
  if constexpr (Mma::E > 1) {
    typename Mma::frag_t bf[G::NKK];
#pragma unroll
    for (int kk = 0; kk < G::NKK; ++kk) bf[kk] = read_frag<Mma, G>(tile, n, hh, kk);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = Mma::mma(qf[hb][0], bf[0], f32x16_t{});
#pragma unroll
    for (int kk = 1; kk < G::NKK; ++kk)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = Mma::mma(qf[hb][kk], bf[kk], acc[hb]);
  } else {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16_t{};
#pragma unroll
    for (int c4 = 0; c4 < G::NKK / 4; ++c4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(tile + chunk_off<G>(n, hh * (G::CPR / 2) + c4));
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = Mma::mma(qf[hb][c4 * 4 + e], v[e], acc[hb]);
    }
  }
}

// B fragments (the 32 keys' halves of the head dimension) of one 32-key step, direct paths.
template <class Mma, int D, int KT>
__device__ __forceinline__ void load_bfrag(const uint8_t* tile, int n0, int lane,
                                           typename Mma::frag_t (&bf)[Geo<Mma, D, KT>::NKK]) {
  typedef Geo<Mma, D, KT> G;
  const int hh = lane >> 5;
  const int n = n0 + (lane & 31);
#pragma unroll
  for (int kk = 0; kk < G::NKK; ++kk) bf[kk] = read_frag<Mma, G>(tile, n, hh, kk);
}

// bf16 path: MFMAs of one 32-key step from fragments already in registers; when `next` is
// set, each fragment register is refilled with the next step's fragment right after its last
// use, so that the LDS latency of the next step hides behind this step's MFMAs.
template <int D, int HB, int KT>
__device__ __forceinline__ void tile_mma_rot(const bf16x8_t (&qf)[HB][Geo<MmaBf16, D, KT>::NKK],
                                             bf16x8_t (&bf)[Geo<MmaBf16, D, KT>::NKK],
                                             const uint8_t* tile, int next_n0, bool next, int lane,
                                             f32x16_t (&acc)[HB]) {
  typedef Geo<MmaBf16, D, KT> G;
  const int hh = lane >> 5;
  const int n = next_n0 + (lane & 31);
#pragma unroll
  for (int kk = 0; kk < G::NKK; ++kk) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      acc[hb] = MmaBf16::mma(qf[hb][kk], bf[kk], kk == 0 ? f32x16_t{} : acc[hb]);
    if (next) bf[kk] = read_frag<MmaBf16, G>(tile, n, hh, kk);
  }
}

// Order of the head-weighted sum: the 16 accumulator registers of each head block are taken in
// 8 slices of 2 registers; slice by slice, head block by head block, register r goes into partial
// sum r % 4. Every evaluation of the epilogue (interleaved with MFMAs or not) uses this order, so
// that a key's score does not depend on the path that computed it.
constexpr int EPI_SLICES = 8;

template <int HB>
__device__ __forceinline__ void epi_slice(const f32x16_t (&acc)[HB], const float (&wv)[HB][16], int sl,
                                          float (&p)[4]) {
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int r = 2 * sl; r < 2 * sl + 2; ++r) p[r & 3] = fmaf(wv[hb][r], relu(acc[hb][r]), p[r & 3]);
}

// Cross-lane finish: lanes l and l+32 hold complementary heads of key l % 32; the permlane32 swap
// exchanges the halves so that both lanes end with the same total.
__device__ __forceinline__ float epi_finish(const float (&p)[4]) {
  const float part = (p[0] + p[1]) + (p[2] + p[3]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                   false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// ReLU + head-weighted sum of one 32x32 tile per head block; returns the full score of key
// (lane % 32) in every lane.
template <int HB>
__device__ __forceinline__ float tile_epilogue(const f32x16_t (&acc)[HB], const float (&wv)[HB][16]) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < EPI_SLICES; ++sl) epi_slice<HB>(acc, wv, sl, p);
  return epi_finish(p);
}

// One 32-key step of the bf16 path with the previous step's epilogue woven in. Per key fragment
// kk: the HB MFMAs of this step, the refill of fragment register kk with the next step's
// fragment from LDS (when `next`), the fragment's share of the previous step's epilogue (when
// `prev`; slices of epi_slice, in order) and the hook extra(kk) (the next tile's load issue). A
// scheduling barrier closes each fragment's group, so that the compiler keeps VALU work behind
// every pair of MFMAs instead of running the MFMAs back to back and the epilogue after them (a
// wave issues in order: the matrix core is idle while the wave works through a run of VALU
// instructions). Returns the previous step's scores (when `prev`).
template <class Mma, int D, int HB, int KT, class Extra>
__device__ __forceinline__ float tile_mma_epi(const typename Mma::frag_t (&qf)[HB][Geo<Mma, D, KT>::NKK],
                                              typename Mma::frag_t (&bf)[Geo<Mma, D, KT>::NKK],
                                              const uint8_t* tile, int next_n0, bool next, bool prev,
                                              int lane, f32x16_t (&acc)[HB], const f32x16_t (&pacc)[HB],
                                              const float (&wv)[HB][16], Extra extra) {
  typedef Geo<Mma, D, KT> G;
  constexpr int NKK = G::NKK;
  static_assert(EPI_SLICES % NKK == 0 || NKK % EPI_SLICES == 0, "epilogue slices per fragment");
  const int hh = lane >> 5;
  const int n = next_n0 + (lane & 31);
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      acc[hb] = Mma::mma(qf[hb][kk], bf[kk], kk == 0 ? f32x16_t{} : acc[hb]);
    if (next) bf[kk] = read_frag<Mma, G>(tile, n, hh, kk);
    if (prev) {
#pragma unroll
      for (int sl = kk * EPI_SLICES / NKK; sl < (kk + 1) * EPI_SLICES / NKK; ++sl) epi_slice<HB>(pacc, wv, sl, p);
      // the partial sums are materialised here: without this the compiler sinks the whole
      // epilogue to its single use after the last fragment
      asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
    }
    extra(kk);
    __builtin_amdgcn_sched_barrier(0);
  }
  return prev ? epi_finish(p) : 0.f;
}

}  // namespace idx
