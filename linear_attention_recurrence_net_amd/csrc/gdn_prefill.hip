// gdn_prefill.hip -- chunked prefill (placeholder until the MFMA kernels land).
#include "device_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

size_t prefill_workspace_bytes(int B, int T, int H, int d) {
    (void)B; (void)T; (void)H; (void)d;
    return 256;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    (void)a; (void)stream;
    return hipErrorNotSupported;
}

}  // namespace gdn
