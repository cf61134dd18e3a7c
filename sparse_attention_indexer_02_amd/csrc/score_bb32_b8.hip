// Score kernel launchers: bf16 MFMA with bf16 keys at D=32, bf16 MFMA with FP8 keys at D=32, bf16 MFMA with FP8 keys at D=64, bf16 MFMA with FP8 keys at D=128.
#include "score_kernel.h"

namespace idx {

template hipError_t launch_score_d<MmaBf16, DT_BF16, 32>(const ScoreArgs&, int, hipStream_t);
template hipError_t launch_score_d<MmaBf16, DT_FP8, 32>(const ScoreArgs&, int, hipStream_t);
template hipError_t launch_score_d<MmaBf16, DT_FP8, 64>(const ScoreArgs&, int, hipStream_t);
template hipError_t launch_score_d<MmaBf16, DT_FP8, 128>(const ScoreArgs&, int, hipStream_t);

}  // namespace idx
