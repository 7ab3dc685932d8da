// bf16 KV, 64 heads per workgroup (h_q 64 and 128), B_TOPK 64.
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_bf16<4, 64>(const FwdArgs&, hipStream_t);
}  // namespace smla
