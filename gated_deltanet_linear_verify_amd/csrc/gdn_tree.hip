// gdn_tree.hip - tree verify (placeholder until the kernel lands).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

size_t verify_tree_lds_bytes(int d, int T) { return sizeof(float) * (size_t)T * d; }

hipError_t launch_verify_tree(const VerifyArgs &, const LaunchCfg &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
