// Launchers of the forward kernels per configuration (instantiated by the
// smla_fwd_*.hip units).
#pragma once

#include "smla_fwd_q_pipe.cuh"

namespace smla {

template <int NW, int BT>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t stream) {
  const bool split = a.num_splits > 1, buf = a.kv_window_bytes != 0;
  if constexpr (NW == 4 && BT == 32) {
    // 64 heads per workgroup, B_TOPK 32, long splits: the pipelined d_v-split
    // kernel (its prologue costs more; short decode splits keep the other one)
    if (a.slots_per_split >= kPipeMinSlots) {
      const dim3 grid(grid_size(a)), block(256);
      if (a.token_blocks)   // one split, 32-bit window, block counts computed ahead
        hipLaunchKernelGGL((smla_fwd_bf16_pipe_kernel<false, true, true>), grid, block, 0, stream, a);
      else if (split && buf)
        hipLaunchKernelGGL((smla_fwd_bf16_pipe_kernel<true, true>), grid, block, 0, stream, a);
      else if (split)
        hipLaunchKernelGGL((smla_fwd_bf16_pipe_kernel<true, false>), grid, block, 0, stream, a);
      else if (buf)
        hipLaunchKernelGGL((smla_fwd_bf16_pipe_kernel<false, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((smla_fwd_bf16_pipe_kernel<false, false>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (split)
    buf ? launch_bf16_variant<NW, BT, true, true>(a, stream) : launch_bf16_variant<NW, BT, true, false>(a, stream);
  else
    buf ? launch_bf16_variant<NW, BT, false, true>(a, stream) : launch_bf16_variant<NW, BT, false, false>(a, stream);
  return hipGetLastError();
}

// bf16 KV, B_TOPK 128: short splits (at most 128 slots) in the one-block
// kernel, longer ones in the 128-slot block loop.
template <int NW>
hipError_t launch_bf16_b128(const FwdArgs& a, hipStream_t stream) {
  const bool split = a.num_splits > 1, buf = a.kv_window_bytes != 0;
  if (a.slots_per_split <= kShortSlots) {
    if (split)
      buf ? launch_bf16_short<NW, true, true>(a, stream) : launch_bf16_short<NW, true, false>(a, stream);
    else
      buf ? launch_bf16_short<NW, false, true>(a, stream) : launch_bf16_short<NW, false, false>(a, stream);
    return hipGetLastError();
  }
  const dim3 grid(grid_size(a)), block(NW * 64);
  if (split && buf)
    hipLaunchKernelGGL((smla_fwd_bf16_b128_kernel<NW, true, true>), grid, block, 0, stream, a);
  else if (split)
    hipLaunchKernelGGL((smla_fwd_bf16_b128_kernel<NW, true, false>), grid, block, 0, stream, a);
  else if (buf)
    hipLaunchKernelGGL((smla_fwd_bf16_b128_kernel<NW, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((smla_fwd_bf16_b128_kernel<NW, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_fp4(const FwdArgs& a, hipStream_t stream) {
  const bool split = a.num_splits > 1, buf = a.kv_window_bytes != 0;
  if constexpr (NW == 4) {
    // 64 heads per workgroup: the pipelined kernel with one conversion per
    // block and workgroup
    const dim3 grid(grid_size(a)), block(256);
    if (split && buf)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<true, true, KvFp4Format>), grid, block, 0, stream, a);
    else if (split)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<true, false, KvFp4Format>), grid, block, 0, stream, a);
    else if (buf)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<false, true, KvFp4Format>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<false, false, KvFp4Format>), grid, block, 0, stream, a);
    return hipGetLastError();
  } else {
    if (split)
      buf ? launch_fp8_variant<NW, true, true, KvFp4Format>(a, stream)
          : launch_fp8_variant<NW, true, false, KvFp4Format>(a, stream);
    else
      buf ? launch_fp8_variant<NW, false, true, KvFp4Format>(a, stream)
          : launch_fp8_variant<NW, false, false, KvFp4Format>(a, stream);
    return hipGetLastError();
  }
}

template <int NW>
hipError_t launch_fp8(const FwdArgs& a, hipStream_t stream) {
  const bool split = a.num_splits > 1, buf = a.kv_window_bytes != 0;
  if constexpr (NW == 4) {
    // 64 heads per workgroup: the pipelined kernel with one conversion per
    // block and workgroup
    const dim3 grid(grid_size(a)), block(256);
    if (split && buf)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<true, true, KvFp8Format>), grid, block, 0, stream, a);
    else if (split)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<true, false, KvFp8Format>), grid, block, 0, stream, a);
    else if (buf)
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<false, true, KvFp8Format>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((smla_fwd_q_pipe_kernel<false, false, KvFp8Format>), grid, block, 0, stream, a);
    return hipGetLastError();
  } else {
    if (split)
      buf ? launch_fp8_variant<NW, true, true>(a, stream) : launch_fp8_variant<NW, true, false>(a, stream);
    else
      buf ? launch_fp8_variant<NW, false, true>(a, stream) : launch_fp8_variant<NW, false, false>(a, stream);
    return hipGetLastError();
  }
}

}  // namespace smla
