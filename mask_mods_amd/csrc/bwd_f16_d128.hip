// Backward kernel instantiations: f16 inputs, head dim 128.
#include "bwd.h"

namespace mm {
hipError_t launch_bwd_f16_d128(const BwdParams &p, bool alibi, int mask, hipStream_t s) {
    return launch_bwd_t<F16, 128>(p, alibi, mask, s);
}
}  // namespace mm
