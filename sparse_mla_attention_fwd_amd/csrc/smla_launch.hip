// Host dispatch of the forward pass and the split-topk combine kernel.
//
// Combine (page "Ascend Sparse Attention Forward 算法与优化技术简析", section
// 数学建模: tokens are independent and the softmax over a token's slots can be
// merged from parts by their log-sum-exp): out = Σ_s e^{lse_s − lse} out_s,
// lse = log Σ_s e^{lse_s}; an empty part (lse = −∞) has weight 0.
#include "smla_common.cuh"

namespace smla {
namespace {

// Log-sum-exp merge of split partials (bf16 O/l and fp32 lse per part): one
// thread per (token, head, 8 columns).  Parts are merged four at a time: the
// four lse values and partial rows of a chunk are all loaded before any is
// used (one memory round trip per chunk), then folded into the running
// merge with the chunk's max.  A part with lse = −∞ (no valid slot) gets
// weight 0; its partial row, written as zeros, is still loaded, and loads
// past the last part repeat the last part with weight 0.
__global__ __launch_bounds__(256) void smla_combine_kernel(FwdArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.s_q * a.h_q * (kDv / 8);
  if (t >= total) return;
  const int q8 = (int)(t % (kDv / 8));
  const int64_t th = t / (kDv / 8);
  const int head = (int)(th % a.h_q);
  const int64_t token = th / a.h_q;
  const int ns = a.num_splits;
  const int64_t part0 = token * ns * a.h_q + head;
  float m = kNegInf, z = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int s0 = 0; s0 < ns; s0 += 4) {
    float ls[4];
    i32x4 pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t part = part0 + (int64_t)min(s0 + j, ns - 1) * a.h_q;
      ls[j] = a.ws_lse[part];
      pv[j] = *(const i32x4*)(a.ws_o + part * kDv + 8 * q8);
    }
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (s0 + j >= ns) ls[j] = kNegInf;
    const float mc = fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3]));
    const float mn = fmaxf(m, mc);
    if (mn == kNegInf) continue;                 // every part so far is empty
    if (m != kNegInf && mn != m) {
      const float r = __expf(m - mn);
      z *= r;
      acc0 *= r;
      acc1 *= r;
    }
    m = mn;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float wgt = ls[j] == kNegInf ? 0.f : __expf(ls[j] - m);
      z += wgt;
      // eight bf16 partial values -> fp32 (exact: bf16 is the top half of fp32)
      f32x4 lo4, hi4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        lo4[2 * k] = __uint_as_float((uint32_t)pv[j][k] << 16);
        lo4[2 * k + 1] = __uint_as_float((uint32_t)pv[j][k] & 0xFFFF0000u);
        hi4[2 * k] = __uint_as_float((uint32_t)pv[j][k + 2] << 16);
        hi4[2 * k + 1] = __uint_as_float((uint32_t)pv[j][k + 2] & 0xFFFF0000u);
      }
      acc0 += wgt * lo4;
      acc1 += wgt * hi4;
    }
  }
  const float inv = z > 0.f ? 1.0f / z : 0.f;
  i32x4 v;
  v[0] = (int)pack2_bf16(acc0[0] * inv, acc0[1] * inv);
  v[1] = (int)pack2_bf16(acc0[2] * inv, acc0[3] * inv);
  v[2] = (int)pack2_bf16(acc1[0] * inv, acc1[1] * inv);
  v[3] = (int)pack2_bf16(acc1[2] * inv, acc1[3] * inv);
  *(i32x4*)(a.out + token * a.out_st + (int64_t)head * a.out_sh + 8 * q8) = v;
  if (q8 == 0) a.lse[token * a.lse_st + head] = z > 0.f ? m + __logf(z) : kNegInf;
}

// Paged KV cache (page "Flash Attention Infer算子性能优化", section
// 优化Paged Attention路径: pages of contiguous rows reached through a block
// table).  One thread per slot: logical position v of token t is row
// v % page_size of physical page block_table[t][v / page_size]; positions
// outside [0, table_width * page_size) and blocks whose entry is outside
// [0, num_pages) give -1 (masked by the forward kernels).
__global__ __launch_bounds__(256) void smla_paged_translate_kernel(
    const int32_t* __restrict__ idx, int64_t idx_st, const int32_t* __restrict__ bt, int64_t bt_st,
    int32_t table_width, int32_t page_size, int64_t num_pages, int32_t s_q, int32_t topk,
    int32_t* __restrict__ phys) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)s_q * topk) return;
  const int64_t t = i / topk, j = i - t * topk;
  const int32_t v = idx[t * idx_st + j];
  int32_t r = -1;
  if (v >= 0 && (int64_t)v < (int64_t)table_width * page_size) {
    const int32_t blk = v / page_size;
    const int32_t page = bt[t * bt_st + blk];
    if (page >= 0 && (int64_t)page < num_pages) r = page * page_size + (v - blk * page_size);
  }
  phys[i] = r;
}

// Blocks of each token up to its last valid slot, at least 1 (an empty
// token still takes one fully masked block): one wave per token reads the
// token's index row.
__global__ __launch_bounds__(256) void smla_token_blocks_kernel(const int32_t* __restrict__ idx, int64_t idx_st,
                                                                int32_t s_q, int32_t topk, int64_t s_kv,
                                                                int32_t* __restrict__ nb) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= s_q) return;
  const int32_t* __restrict__ irow = idx + t * idx_st;
  int last = -1;
  int j = lane;
  for (; j + 7 * 64 < topk; j += 8 * 64) {
    int v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = irow[j + 64 * k];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (v[k] >= 0 && (int64_t)v[k] < s_kv) last = j + 64 * k;
  }
  for (; j < topk; j += 64) {
    const int v = irow[j];
    if (v >= 0 && (int64_t)v < s_kv) last = j;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off));
  if (lane == 0) nb[t] = last < 0 ? 1 : last / 32 + 1;
}

}  // namespace

hipError_t launch_token_blocks(const FwdArgs& a, int32_t* nb, hipStream_t stream) {
  hipLaunchKernelGGL(smla_token_blocks_kernel, dim3((unsigned)((a.s_q + 3) / 4)), dim3(256), 0, stream, a.idx,
                     a.idx_st, a.s_q, a.topk, a.s_kv, nb);
  return hipGetLastError();
}

hipError_t launch_paged_translate(const int32_t* idx, int64_t idx_st, const int32_t* block_table,
                                  int64_t bt_st, int32_t table_width, int32_t page_size,
                                  int64_t num_pages, int32_t s_q, int32_t topk, int32_t* phys,
                                  hipStream_t stream) {
  const int64_t n = (int64_t)s_q * topk;
  hipLaunchKernelGGL(smla_paged_translate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, idx, idx_st, block_table, bt_st, table_width, page_size, num_pages, s_q,
                     topk, phys);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int b_topk, int kv_format, hipStream_t stream) {
  hipError_t e;
  const bool b64 = b_topk == 64;
  if (kv_format == kKvFp4) {
    switch (a.h_q) {
      case 16: e = launch_fp4<1>(a, stream); break;
      case 32: e = launch_fp4<2>(a, stream); break;
      case 64:
      case 128: e = launch_fp4<4>(a, stream); break;   // 128: two head groups
      default: return hipErrorInvalidValue;
    }
  } else if (kv_format == kKvFp8) {
    switch (a.h_q) {
      case 16: e = launch_fp8<1>(a, stream); break;
      case 32: e = launch_fp8<2>(a, stream); break;
      case 64:
      case 128: e = launch_fp8<4>(a, stream); break;   // 128: two head groups
      default: return hipErrorInvalidValue;
    }
  } else if (b_topk == 128) {
    switch (a.h_q) {
      case 16: e = launch_bf16_b128<1>(a, stream); break;
      case 32: e = launch_bf16_b128<2>(a, stream); break;
      case 64:
      case 128: e = launch_bf16_b128<4>(a, stream); break;   // 128: two head groups
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.h_q) {
      case 16: e = b64 ? launch_bf16<1, 64>(a, stream) : launch_bf16<1, 32>(a, stream); break;
      case 32: e = b64 ? launch_bf16<2, 64>(a, stream) : launch_bf16<2, 32>(a, stream); break;
      case 64:
      case 128:   // 128: two head groups
        e = b64 ? launch_bf16<4, 64>(a, stream) : launch_bf16<4, 32>(a, stream); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess || a.num_splits <= 1) return e;
  const int64_t threads = (int64_t)a.s_q * a.h_q * (kDv / 8);
  hipLaunchKernelGGL(smla_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace smla
