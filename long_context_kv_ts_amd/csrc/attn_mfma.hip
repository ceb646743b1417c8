// Matrix-core split-K attention (placeholder until the bf16 MFMA kernel lands).
#include "common.h"

namespace ts {
hipError_t launch_attn_split_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ts
