// Forward MFMA kernel instantiations: bf16 inputs, head dim 128.
#include "fwd_mfma.h"

namespace mm {
hipError_t launch_fwd_mfma_bf16_d128(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
    return launch_fwd_mfma<BF16, 128>(p, alibi, mask, s);
}
}  // namespace mm
