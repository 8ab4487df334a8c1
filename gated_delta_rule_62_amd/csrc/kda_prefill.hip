// kda_prefill.hip -- chunkwise KDA prefill (gfx950).  (kernels follow)
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

PrefillPlan plan_prefill(int B, int T, int H, int D, int N, bool varlen) {
    PrefillPlan p;
    (void)B; (void)T; (void)H; (void)D; (void)N; (void)varlen;
    return p;
}

hipError_t launch_prefill(const PrefillArgs&, const PrefillPlan&, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace kda
