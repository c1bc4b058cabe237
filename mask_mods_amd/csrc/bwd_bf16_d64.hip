// Backward kernel instantiations: bf16 inputs, head dim 64.
#include "bwd.h"

namespace mm {
hipError_t launch_bwd_bf16_d64(const BwdParams &p, bool alibi, int mask, hipStream_t s) {
    return launch_bwd_t<BF16, 64>(p, alibi, mask, s);
}
}  // namespace mm
