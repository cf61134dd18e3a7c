// Score kernel launchers: bf16 MFMA with bf16 keys at D=64.
#include "score_kernel.h"

namespace idx {

template hipError_t launch_score_d<MmaBf16, DT_BF16, 64>(const ScoreArgs&, int, hipStream_t);

}  // namespace idx
