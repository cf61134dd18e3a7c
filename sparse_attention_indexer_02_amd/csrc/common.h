// Device-side building blocks shared by the indexer kernels (gfx950 / CDNA4).
//
// Score contraction: for one query t and a block of 32 keys, the head dot products
// x[h, n] = q[t,h,:] . k[n,:] are one 32x32 MFMA tile per group of 32 heads (rows = heads,
// columns = keys), accumulated in fp32 over D. The fused epilogue reduces the tile to one score
// per key, I[t,n] = sum_h w[t,h] * max(x[h,n], 0), in registers: each lane holds 16 heads of one
// key per tile, lanes l and l+32 hold complementary heads, one cross-lane add finishes the sum.
// (DeepSeek Sparse Attention's lightning-indexer score; the five indexer pages build on it.)
//
// Operand layout: lane l works on key/head row (l % 32) and on HALF of the head dimension,
// hh = l / 32 covers d in [hh*D/2, (hh+1)*D/2). Step kk of the contraction consumes E
// consecutive elements of that half (E = 8 for bf16 32x32x16, E = 1 for fp32 32x32x2). The same
// permutation of d is applied to queries and keys, so the dot products are unchanged.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// ---------------------------------------------------------------------------------------------
// number formats

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// OCP FP8 E4M3FN byte -> bf16 bits, exact (every E4M3 value is a bf16 value). Normal codes:
// exponent rebias 7 -> 127 and mantissa moved to the top of bf16's 7 bits. Subnormal codes
// m * 2^-9 are normalised by a 3-entry shift. The NaN code (S.1111.111) maps to a bf16 NaN.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t b) {
  uint32_t s = (b & 0x80u) << 8;
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  uint32_t mag;
  if (e != 0) {
    mag = ((e + 120u) << 7) | (m << 4);
    if (e == 15u && m == 7u) mag = 0x7FC0u;
  } else if (m == 0) {
    mag = 0;
  } else {
    // m in 1..7: value m*2^-9; leading bit position p = floor(log2 m)
    uint32_t p = 31u - __builtin_clz(m);
    uint32_t frac = (m << (7u - p)) & 0x7Fu;        // bits below the leading one, left-aligned
    mag = ((118u + p) << 7) | frac;                 // 2^-9 * 2^p -> biased exponent 118 + p
  }
  return s | mag;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __uint_as_float(e4m3_to_bf16_bits(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even, NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Order-preserving map float -> uint32 (larger float <=> larger key). 0 is below every
// non-NaN float (-inf maps to 0x007FFFFF) and marks "no score" slots.
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
constexpr uint32_t KEY_NONE = 0u;
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;    // f2key(-inf): slots without a candidate

// ---------------------------------------------------------------------------------------------
// MFMA flavours. Elements live in LDS in the flavour's element type.

struct MmaBf16 {
  static constexpr int kElemBytes = 2;
  static constexpr int E = 8;                  // elements per lane per instruction
  typedef bf16x8_t frag_t;
  static __device__ __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// FP8 x FP8 (OCP E4M3FN both): 32x32x64 with fp32 accumulation, 32 elements (bytes) per lane
// per operand; the block scales of the instruction are 1 (E8M0 127).
struct MmaFp8 {
  static constexpr int kElemBytes = 1;
  static constexpr int E = 32;
  typedef i32x8_t frag_t;
  static __device__ __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

struct MmaF32 {
  static constexpr int kElemBytes = 4;
  static constexpr int E = 1;
  typedef float frag_t;
  static __device__ __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Head held by accumulator register r of lane l in head block hb (32x32 MFMA C layout:
// row = 8*(r/4) + 4*(l/32) + r%4, column = l%32).
__device__ __forceinline__ int acc_head(int hb, int r, int lane) {
  return 32 * hb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Load E elements of a query/key row, converting from its storage format into the MFMA
// element type. `row` points at the row start, `e0` is the first element.
template <class Mma>
__device__ __forceinline__ typename Mma::frag_t load_frag(const void* row, int dtype, int e0);

template <>
__device__ __forceinline__ bf16x8_t load_frag<MmaBf16>(const void* row, int dtype, int e0) {
  // only bf16 storage reaches here (queries of the bf16 path)
  u32x4_t v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(row) + e0);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <>
__device__ __forceinline__ i32x8_t load_frag<MmaFp8>(const void* row, int dtype, int e0) {
  // only E4M3 bytes reach here (queries of the FP8 path)
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(row) + e0);
  const u32x4_t lo = src[0], hi = src[1];
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <>
__device__ __forceinline__ float load_frag<MmaF32>(const void* row, int dtype, int e0) {
  if (dtype == DT_F32) return reinterpret_cast<const float*>(row)[e0];
  if (dtype == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[e0]);
  return e4m3_to_f32(reinterpret_cast<const uint8_t*>(row)[e0]);
}

// Bytes per element of a storage dtype.
__host__ __device__ __forceinline__ int dtype_bytes(int dt) {
  return dt == DT_F32 ? 4 : (dt == DT_BF16 ? 2 : 1);
}

// ---------------------------------------------------------------------------------------------
// Wave-level helpers (wave64)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(v, o, 64);
    if (l >= o) v += u;
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes with DPP (row shifts, then row broadcasts): no LDS
// round trips.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_bcast(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Wave-level search over a histogram of nbins bins (a power of two, at least 64), highest bin
// first: the bin holding the need-th largest element (need >= 1) and the count in higher bins.
// count(b) reads bin b. Returns the total count; *bin_out = -1 when need exceeds it.
// Lane l sums the contiguous range of nbins/64 bins below nbins - l*nbins/64; the lanes walk
// their ranges from different offsets, so that one read instruction of the wave touches
// consecutive bins (distinct LDS banks) instead of 64 bins a bank-count multiple apart. The
// range that holds the bin is then searched by the whole wave, 64 bins per prefix scan.
template <class CountFn>
__device__ __forceinline__ uint32_t wave_hist_find(int nbins, uint32_t need, CountFn count,
                                                   int* bin_out, uint32_t* above_out) {
  const int lane = lane_id();
  const int per = nbins >> 6;
  const int hi = nbins - 1 - lane * per;
  uint32_t sum = 0;
#pragma unroll 8
  for (int i = 0; i < per; ++i) sum += count(hi - ((i + lane) & (per - 1)));
  const uint32_t inc = wave_scan_dpp(sum);
  const uint32_t tot = wave_bcast(inc, 63);
  const uint64_t m = __ballot(need > 0 && inc - sum < need && need <= inc);
  *bin_out = -1;
  *above_out = 0;
  if (m) {
    const int src = __builtin_ctzll(m);
    const int shi = nbins - 1 - src * per;
    uint32_t base = wave_bcast(inc - sum, src);
    for (int c = 0; c < per; c += 64) {
      const int j = c + lane;
      const uint32_t h = j < per ? count(shi - j) : 0u;
      const uint32_t s = wave_scan_dpp(h);
      const uint64_t hit = __ballot(base + s >= need);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        *bin_out = shi - c - f;
        *above_out = base + wave_bcast(s - h, f);
        break;
      }
      base += wave_bcast(s, 63);
    }
  }
  return tot;
}

__device__ __forceinline__ uint32_t wave_hist_find(const uint32_t* hist, int nbins, uint32_t need,
                                                   int* bin_out, uint32_t* above_out) {
  return wave_hist_find(nbins, need, [&](int b) { return hist[b]; }, bin_out, above_out);
}

// First radix digit of a selection: the top `bits` (11 or 12) bits of the order-preserving key.
// With 12 bits the 4096 counters are 16-bit halves of 2048 words (valid for rows of fewer than
// 65536 slots, so that no half can carry into its neighbour); bins b and b + 2048 (keys of
// opposite sign) share a word, so that neighbouring bins, which a row's scores crowd into, sit
// in different words and banks and atomic adds to them do not serialise.
__device__ __forceinline__ uint32_t digit1(uint32_t key, int bits) { return key >> (32 - bits); }

__device__ __forceinline__ void hist1_add(uint32_t* words, uint32_t key, int bits) {
  if (bits == 12) atomicAdd(&words[(key >> 20) & 2047u], 1u << ((key >> 31) * 16));
  else atomicAdd(&words[key >> 21], 1u);
}

// hist1_add without a branch: adds 0 when `ok` is false.
__device__ __forceinline__ void hist1_add_if(uint32_t* words, uint32_t key, int bits, bool ok) {
  const uint32_t w = bits == 12 ? (key >> 20) & 2047u : key >> 21;
  const uint32_t inc = bits == 12 ? 1u << ((key >> 31) * 16) : 1u;
  atomicAdd(&words[w], ok ? inc : 0u);
}

__device__ __forceinline__ uint32_t hist1_count(const uint32_t* words, int bin, int bits) {
  if (bits == 12) return (words[bin & 2047] >> ((bin >> 11) * 16)) & 0xFFFFu;
  return words[bin];
}

}  // namespace idx
