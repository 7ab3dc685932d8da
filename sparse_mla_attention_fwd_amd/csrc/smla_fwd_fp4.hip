// fp4 (E2M1) KV cache, every head count (16, 32 and 64 heads per workgroup).
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_fp4<1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fp4<2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fp4<4>(const FwdArgs&, hipStream_t);
}  // namespace smla
