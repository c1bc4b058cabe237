// Backward dispatch over dtype and head dim.
#include "kernels.h"

namespace mm {
hipError_t launch_bwd_bf16_d64(const BwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_bwd_bf16_d128(const BwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_bwd_f16_d64(const BwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_bwd_f16_d128(const BwdParams &p, bool alibi, int mask, hipStream_t s);

hipError_t launch_bwd(const BwdParams &p, int dtype, int D, bool alibi, int mask, hipStream_t s) {
    if (dtype == 2) return D == 64 ? launch_bwd_bf16_d64(p, alibi, mask, s) : launch_bwd_bf16_d128(p, alibi, mask, s);
    return D == 64 ? launch_bwd_f16_d64(p, alibi, mask, s) : launch_bwd_f16_d128(p, alibi, mask, s);
}
}  // namespace mm
