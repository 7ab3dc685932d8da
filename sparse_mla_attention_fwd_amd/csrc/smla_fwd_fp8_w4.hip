// fp8 E4M3 KV, 64 heads per workgroup (h_q 64 and 128).
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_fp8<4>(const FwdArgs&, hipStream_t);
}  // namespace smla
