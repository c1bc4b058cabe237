// Forward MFMA kernel instantiations: bf16 inputs, head dim 128.
#include "fwd_pingpong.h"

namespace mm {
hipError_t launch_fwd_mfma_bf16_d128(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
    #if MM_FWD_PP
    return launch_fwd_pp<BF16, 128>(p, alibi, mask, s);
#else
    return launch_fwd_mfma<BF16, 128>(p, alibi, mask, s);
#endif
}
}  // namespace mm
