// Host dispatch of the score kernel (score_kernel.h): the (MFMA flavour, key storage, head dim)
// launchers are compiled in separate units (score_*.hip) so that the library builds in parallel.
#include "common.h"
#include "kernels.h"

namespace idx {

template <class Mma, int KST, int D>
hipError_t launch_score_d(const ScoreArgs& a, int n_splits, hipStream_t s);

bool score_supported(int q_dtype, int k_dtype, int H, int D) {
  if (!(D == 32 || D == 64 || D == 128)) return false;
  if (H < 1 || H > 128) return false;
  if (q_dtype == DT_FP8) return k_dtype == DT_FP8 && D >= 64;   // FP8 x FP8 MFMA, K = 64 per step
  if (q_dtype != DT_F32 && q_dtype != DT_BF16) return false;
  if (k_dtype != DT_F32 && k_dtype != DT_BF16 && k_dtype != DT_FP8) return false;
  return true;
}

template <class Mma, int KST>
static hipError_t launch_dh(const ScoreArgs& a, int n_splits, hipStream_t s) {
  if (a.D == 128) return launch_score_d<Mma, KST, 128>(a, n_splits, s);
  if (a.D == 64) return launch_score_d<Mma, KST, 64>(a, n_splits, s);
  if (a.D == 32) return launch_score_d<Mma, KST, 32>(a, n_splits, s);
  return hipErrorInvalidValue;
}

int score_queries_per_tile(int H) { return (H <= 64) ? 8 : 4; }

hipError_t launch_score(const ScoreArgs& a, int n_splits, hipStream_t s) {
  if (a.q_dtype == DT_FP8) {
    if (a.k_dtype != DT_FP8) return hipErrorInvalidValue;
    if (a.D == 128) return launch_score_d<MmaFp8, DT_FP8, 128>(a, n_splits, s);
    if (a.D == 64) return launch_score_d<MmaFp8, DT_FP8, 64>(a, n_splits, s);
    return hipErrorInvalidValue;
  }
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_BF16) return launch_dh<MmaBf16, DT_BF16>(a, n_splits, s);
  if (a.q_dtype == DT_BF16 && a.k_dtype == DT_FP8) return launch_dh<MmaBf16, DT_FP8>(a, n_splits, s);
  if (a.k_dtype == DT_F32) return launch_dh<MmaF32, DT_F32>(a, n_splits, s);
  if (a.k_dtype == DT_BF16) return launch_dh<MmaF32, DT_BF16>(a, n_splits, s);
  return launch_dh<MmaF32, DT_FP8>(a, n_splits, s);
}

}  // namespace idx
