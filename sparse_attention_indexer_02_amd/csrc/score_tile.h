// LDS key tiles and the per-wave MFMA tile + fused epilogue, shared by the score kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace idx {

template <class Mma, int D>
struct Geo {
  static constexpr int EB = Mma::kElemBytes;
  static constexpr int ROW_BYTES = D * EB;
  static constexpr int CPR = ROW_BYTES / 16;          // 16-byte chunks per key row
  static constexpr int EPC = 16 / EB;                 // elements per chunk
  static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;
  static constexpr int TILE_BYTES = KEY_TILE * ROW_BYTES;
  static constexpr int NKK = D / 2 / Mma::E;          // MFMA steps per 32x32 tile
};

template <int HB> struct WavesFor { static constexpr int value = (HB <= 2) ? 8 : 4; };

// Stages one tile of KEY_TILE keys from global memory (any key storage format) into LDS in the
// MFMA element format. Global loads are issued early (load) and written to LDS later (store)
// so that their latency overlaps the current tile's MFMA work.
template <class Mma, int D, int KST, int NTHR>
struct TileLoader {
  typedef Geo<Mma, D> G;
  static constexpr int NCH = KEY_TILE * G::CPR;
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
        const int phys = c ^ (n & G::SWZ);
        *reinterpret_cast<u32x4_t*>(tile + n * G::ROW_BYTES + phys * 16) = convert(raw[i]);
      }
    }
  }
};

// One wave: x = q(32*HB heads) . k(32 keys of the tile starting at row n0) accumulated in acc.
template <class Mma, int D, int HB>
__device__ __forceinline__ void tile_mma(const typename Mma::frag_t (&qf)[HB][Geo<Mma, D>::NKK],
                                         const uint8_t* tile, int n0, int lane,
                                         f32x16_t (&acc)[HB]) {
  typedef Geo<Mma, D> G;
  const int hh = lane >> 5;
  const int n = n0 + (lane & 31);
  const uint8_t* krow = tile + n * G::ROW_BYTES;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16_t{};
  if constexpr (Mma::E == 8) {
    bf16x8_t bf[G::NKK];
#pragma unroll
    for (int kk = 0; kk < G::NKK; ++kk)
      bf[kk] = *reinterpret_cast<const bf16x8_t*>(
          krow + (((hh * (G::CPR / 2) + kk) ^ (n & G::SWZ)) << 4));
#pragma unroll
    for (int kk = 0; kk < G::NKK; ++kk)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = Mma::mma(qf[hb][kk], bf[kk], acc[hb]);
  } else {
#pragma unroll
    for (int c4 = 0; c4 < G::NKK / 4; ++c4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(
          krow + (((hh * (G::CPR / 2) + c4) ^ (n & G::SWZ)) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = Mma::mma(qf[hb][c4 * 4 + e], v[e], acc[hb]);
    }
  }
}

// ReLU + head-weighted sum of one 32x32 tile per head block; returns the full score of key
// (lane % 32) in every lane.
template <int HB>
__device__ __forceinline__ float tile_epilogue(const f32x16_t (&acc)[HB], const float (&wv)[HB][16]) {
  float part = 0.f;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) part = fmaf(wv[hb][r], fmaxf(acc[hb][r], 0.f), part);
  return part + __shfl_xor(part, 32, 64);
}

}  // namespace idx
