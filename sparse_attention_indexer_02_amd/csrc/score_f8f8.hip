// Score kernel launchers: FP8 x FP8 MFMA (FP8 queries and keys) at D=64 and D=128.
#include "score_kernel.h"

namespace idx {

template hipError_t launch_score_d<MmaFp8, DT_FP8, 64>(const ScoreArgs&, int, hipStream_t);
template hipError_t launch_score_d<MmaFp8, DT_FP8, 128>(const ScoreArgs&, int, hipStream_t);

}  // namespace idx
