// Placeholder: the bf16 matrix-core prefill is not written yet; bf16 inputs
// use the fp32 vector-ALU kernel.
#include "kda_internal.h"

namespace kda {
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t st) {
    return launch_prefill_valu(a, st);
}
}  // namespace kda
