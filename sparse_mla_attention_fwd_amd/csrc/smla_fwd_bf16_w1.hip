// bf16 KV, h_q 16, B_TOPK 32 and 64.
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_bf16<1, 32>(const FwdArgs&, hipStream_t);
template hipError_t launch_bf16<1, 64>(const FwdArgs&, hipStream_t);
}  // namespace smla
