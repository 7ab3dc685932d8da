// fp8 E4M3 KV, h_q 16 and 32.
#include "smla_fwd_launch.cuh"

namespace smla {
template hipError_t launch_fp8<1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fp8<2>(const FwdArgs&, hipStream_t);
}  // namespace smla
