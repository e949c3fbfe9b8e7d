// moe_shared_gux.hip -- the shared-read gate/up launch with no staging launch: every workgroup converts
// its expert's rows from x itself (calls of up to four tokens with no norm weight, where a separate
// staging launch would cost more than the conversion it saves).
#include "moe_small.h"

namespace moe {

hipError_t launch_shared_gateup_direct(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev) {
    return launch_gu_sh<false>(a, s, ev);
}

}  // namespace moe
