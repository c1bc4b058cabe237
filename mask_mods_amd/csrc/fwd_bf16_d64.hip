// Forward MFMA kernel instantiations: bf16 inputs, head dim 64.
#include "fwd_mfma.h"

namespace mm {
hipError_t launch_fwd_mfma_bf16_d64(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
    return launch_fwd_mfma<BF16, 64>(p, alibi, mask, s);
}
}  // namespace mm
