// fp8 (e4m3) forward, D = 64: the launcher for every mod combination.
#include "fwd_fp8.h"

namespace mm {
hipError_t launch_fwd_fp8_d64(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
    return launch_fwd_fp8<64>(p, alibi, mask, s);
}
}  // namespace mm
