// bf16 KV, h_q 32, B_TOPK 32 and 64.
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_bf16<2, 32>(const FwdArgs&, hipStream_t);
template hipError_t launch_bf16<2, 64>(const FwdArgs&, hipStream_t);
}  // namespace smla
