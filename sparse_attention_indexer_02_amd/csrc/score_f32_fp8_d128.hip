// Score kernel launchers: fp32 MFMA with FP8 keys at D=128.
#include "score_kernel.h"

namespace idx {

template hipError_t launch_score_d<MmaF32, DT_FP8, 128>(const ScoreArgs&, int, hipStream_t);

}  // namespace idx
