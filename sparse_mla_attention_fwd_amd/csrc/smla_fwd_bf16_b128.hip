// bf16 KV, B_TOPK 128 (every head count).
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_bf16_b128<1>(const FwdArgs&, hipStream_t);
template hipError_t launch_bf16_b128<2>(const FwdArgs&, hipStream_t);
template hipError_t launch_bf16_b128<4>(const FwdArgs&, hipStream_t);
}  // namespace smla
