// kd_topk.hip - top-k three-term kernels (placeholder until the streaming
// selection kernel lands).
#include "kd_internal.h"

namespace kd {
size_t topk_workspace_bytes(const Plan& p, int32_t k) { return 256; }
hipError_t run_topk(const Plan&, const TopkIO&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kd
