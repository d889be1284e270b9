// K3: R-SWA-masked prefill (bf16 MFMA). Not built yet: the launcher reports "not supported".
#include "kernels.h"

namespace rswa {

hipError_t launch_prefill(const PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace rswa
