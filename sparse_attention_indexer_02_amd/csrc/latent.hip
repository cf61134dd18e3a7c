// absorb_kernel: absorbed queries for scoring a shared latent cache ("LatentIndex: Cross-Layer
//   Sharing with Layer-Specific Selection for Sparse Attention", abstract: each layer scores the
//   shared cache by absorbing its key decoder into its queries). A layer's key is the latent row
//   times its decoder Wk [Dc, D], so q . k = (Wk q) . latent. The absorbed query of row m
//   (= query * H + head) is q_lat[m, j] = bf16_rne(sum_d q[m, d] * Wk[j, d]): bf16 products,
//   fp32 accumulation on the 32x32x16 bf16 matrix cores (A = 32 query rows, B = 32 decoder rows,
//   K = D), rounded once to bf16 since the result is itself an indexer query.
//   Work-group = 4 waves; a wave holds the whole decoder as B fragments (read once) and walks
//   ABS_TILES tiles of 32 query rows. The contraction is small (Dc / D of a pass over the
//   queries), so the kernel is bound by reading the queries.
#include "common.h"
#include "kernels.h"

namespace idx {

constexpr int ABS_TILES = 8;

template <int D, int DC>
__global__ void __launch_bounds__(256) absorb_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ wk,
                                                     uint16_t* __restrict__ out, int64_t M) {
  constexpr int NK = D / 16;           // K steps; lane half hh takes elements hh * D/2 + 8 kk ..
  constexpr int NC = DC / 32;          // 32-column blocks of the output
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, ln = lane & 31;
  const int64_t m0 = ((int64_t)blockIdx.x * 4 + wave) * (32 * ABS_TILES);
  if (m0 >= M) return;
  bf16x8_t bf[NC][NK];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      bf[cb][kk] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(wk + (int64_t)(32 * cb + ln) * D + hh * (D / 2) + kk * 8));
  for (int tt = 0; tt < ABS_TILES; ++tt) {
    const int64_t mb = m0 + 32 * tt;
    if (mb >= M) break;
    const int64_t r = min(mb + ln, M - 1);
    bf16x8_t af[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      af[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(q + r * D + hh * (D / 2) + kk * 8));
    f32x16_t acc[NC];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) acc[cb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) acc[cb] = MmaBf16::mma(af[kk], bf[cb][kk], acc[cb]);
    // C layout: lane column ln, row 8 (i / 4) + 4 hh + i % 4 of the 32-row tile
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = mb + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (row < M) out[row * DC + 32 * cb + ln] = f32_to_bf16_rne(acc[cb][i]);
      }
  }
}

template <int D>
static hipError_t launch_absorb_d(const uint16_t* q, const uint16_t* wk, uint16_t* out, int64_t M, int Dc,
                                  hipStream_t s) {
  const int64_t per_wg = 4 * 32 * ABS_TILES;
  dim3 grid((unsigned)((M + per_wg - 1) / per_wg));
  if (Dc == 32) hipLaunchKernelGGL((absorb_kernel<D, 32>), grid, dim3(256), 0, s, q, wk, out, M);
  else if (Dc == 64) hipLaunchKernelGGL((absorb_kernel<D, 64>), grid, dim3(256), 0, s, q, wk, out, M);
  else hipLaunchKernelGGL((absorb_kernel<D, 128>), grid, dim3(256), 0, s, q, wk, out, M);
  return hipGetLastError();
}

hipError_t launch_absorb(const void* q, const void* wk, void* out, int64_t M, int D, int Dc, hipStream_t s) {
  if ((D != 32 && D != 64 && D != 128) || (Dc != 32 && Dc != 64 && Dc != 128) || M < 1 ||
      (M + 1023) / 1024 > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  auto qq = static_cast<const uint16_t*>(q);
  auto ww = static_cast<const uint16_t*>(wk);
  auto oo = static_cast<uint16_t*>(out);
  if (D == 32) return launch_absorb_d<32>(qq, ww, oo, M, Dc, s);
  if (D == 64) return launch_absorb_d<64>(qq, ww, oo, M, Dc, s);
  return launch_absorb_d<128>(qq, ww, oo, M, Dc, s);
}

}  // namespace idx
