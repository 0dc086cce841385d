// admit.hip -- which reductions take the host-slot all-reduce (host code).
//
// The 1Cat-vLLM pull request "[Kernel] Two-rank FP16 all-reduce through
// pinned host memory for GPUs without P2P" admits a reduction to the host
// path only when it is FP16, the group has two ranks, the GPUs have no peer
// access and the payload is at most 256 KiB, with a switch that turns the
// path off; everything else stays on the caller's existing collective
// (sections "Purpose" and "Path coverage").  The SGLang pull request "[SM120]
// Add optional FlashInfer PCIe-IPC all-reduce for switch-free hosts" sizes
// its bound for the decode phase, rows = max batch x tokens per request per
// step (speculative draft tokens included), times hidden (sections
// "Modifications" and the review thread on workspace width), and warns that
// silent declines read as slow kernels -- so every decline here names its
// reason.
//
// The policy widens the page's defaults only on request: bfloat16 and groups
// of up to HR_MAX_WORLD ranks are admitted when the caller asks for them.
#include "hr_internal.h"

extern "C" HR_API hr_route hr_admit(const hr_admit_policy *policy, hr_dtype dtype, int world_size,
                                    int peer_access, size_t numel) {
    const size_t max_bytes = (policy && policy->max_bytes) ? policy->max_bytes : HR_DEFAULT_MAX_NUMEL * 2;
    const int max_world = (policy && policy->max_world) ? policy->max_world : 2;
    if (policy != nullptr && !policy->enabled) return HR_DECLINE_DISABLED;
    const bool dtype_ok = dtype == HR_DTYPE_F16 || (dtype == HR_DTYPE_BF16 && policy && policy->allow_bf16);
    if (!dtype_ok) return HR_DECLINE_DTYPE;
    if (world_size < 2 || world_size > max_world || world_size > HR_MAX_WORLD) return HR_DECLINE_WORLD_SIZE;
    if (peer_access) return HR_DECLINE_PEER_ACCESS;
    if (numel > max_bytes / 2) return HR_DECLINE_TOO_LARGE;
    return HR_ROUTE_HOST;
}

extern "C" HR_API const char *hr_route_str(hr_route r) {
    switch (r) {
        case HR_ROUTE_HOST: return "HR_ROUTE_HOST";
        case HR_DECLINE_DISABLED: return "HR_DECLINE_DISABLED";
        case HR_DECLINE_DTYPE: return "HR_DECLINE_DTYPE";
        case HR_DECLINE_WORLD_SIZE: return "HR_DECLINE_WORLD_SIZE";
        case HR_DECLINE_PEER_ACCESS: return "HR_DECLINE_PEER_ACCESS";
        case HR_DECLINE_TOO_LARGE: return "HR_DECLINE_TOO_LARGE";
    }
    return "HR_ROUTE_UNKNOWN";
}

extern "C" HR_API size_t hr_decode_numel(size_t max_batch, size_t tokens_per_request, size_t hidden) {
    const size_t rows = max_batch * (tokens_per_request ? tokens_per_request : 1);
    return rows * hidden;
}
