// Phase timestamps of the short-split bf16 decode kernel on the 128-head decode
// workload (64 tokens, topk 512 in 4 splits, 32768 KV rows per token).  Built by
// phase_probe.py, which generates phase_probe_gen.cuh from the library source.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "phase_probe_gen.cuh"

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

__global__ void fill_bf16(uint16_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0x3c00 + (uint16_t)((i * 2654435761u) >> 25);   // small positive values
}
__global__ void read_all(const smla::i32x4* p, size_t n, int* sink) {
  smla::i32x4 acc = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) acc += p[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x7fffffff) sink[0] = 1;
}

int main() {
  const int s_q = 64, h = 128, topk = 512, per_seq = 32768, ns = 4, G = 256;
  const size_t s_kv = (size_t)s_q * per_seq;
  uint16_t *q, *kv, *out, *wso;
  int *idx, *sink;
  float *lse, *wsl;
  unsigned long long* dbg;
  char* flush;
  const size_t flush_bytes = (size_t)512 << 20;
  CK(hipMalloc(&q, (size_t)s_q * h * 576 * 2));
  CK(hipMalloc(&kv, s_kv * 1152));
  CK(hipMalloc(&idx, (size_t)s_q * topk * 4));
  CK(hipMalloc(&out, (size_t)s_q * h * 512 * 2));
  CK(hipMalloc(&lse, (size_t)s_q * h * 4));
  CK(hipMalloc(&wso, (size_t)s_q * ns * h * 512 * 2));
  CK(hipMalloc(&wsl, (size_t)s_q * ns * h * 4));
  CK(hipMalloc(&dbg, (size_t)G * 16 * 8));
  CK(hipMalloc(&flush, flush_bytes));
  CK(hipMalloc(&sink, 64));
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, q, (size_t)s_q * h * 576);
  hipLaunchKernelGGL(fill_bf16, dim3(8192), dim3(256), 0, 0, kv, s_kv * 576);
  std::vector<int> hidx((size_t)s_q * topk), perm(per_seq);
  std::mt19937 rng(1);
  for (int i = 0; i < per_seq; ++i) perm[i] = i;
  for (int t = 0; t < s_q; ++t) {
    std::shuffle(perm.begin(), perm.end(), rng);
    for (int j = 0; j < topk; ++j) hidx[(size_t)t * topk + j] = t * per_seq + perm[j];
  }
  CK(hipMemcpy(idx, hidx.data(), hidx.size() * 4, hipMemcpyHostToDevice));

  smla::FwdArgs a{};
  a.q = q; a.q_st = h * 576; a.q_sh = 576;
  a.kv = (const char*)kv; a.kv_row_bytes = 1152;
  a.idx = idx; a.idx_st = topk;
  a.out = out; a.out_st = h * 512; a.out_sh = 512; a.lse = lse; a.lse_st = h;
  a.ws_o = wso; a.ws_lse = wsl;
  a.s_q = s_q; a.h_q = h; a.topk = topk; a.slots_per_split = topk / ns; a.num_splits = ns;
  a.head_groups = 1; a.inner_groups = 2; a.s_kv = (int64_t)s_kv; a.scale_log2 = 1.4426950408889634f / 24;
  a.kv_window_bytes = (uint32_t)(s_kv * 1152); a.token_blocks = nullptr;
  // grid of the library's launch for this plan: tokens rounded to 8 x splits
  if ((s_q + 7) / 8 * 8 * ns != G) { printf("grid mismatch\n"); return 1; }

  const char* kinds[3] = {"write-flushed", "write+read-flushed", "warm"};
  const char* phase[8] = {"indices compacted", "stage 0 in LDS", "stage 1", "stage 2", "stage 3",
                          "QK rest", "softmax", "PV + stores"};
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  for (int rep = 0; rep < 9; ++rep) {
    const int kind = rep % 3;
    if (kind < 2) CK(hipMemsetAsync(flush, rep, flush_bytes));
    if (kind == 1)
      hipLaunchKernelGGL(read_all, dim3(4096), dim3(256), 0, 0, (const smla::i32x4*)flush, flush_bytes / 16, sink);
    CK(hipMemsetAsync(dbg, 0, (size_t)G * 16 * 8));
    CK(hipEventRecord(e0));
    hipLaunchKernelGGL((smla::probe_short_kernel<4, true, true, 2>), dim3(G), dim3(256), 0, 0, a, dbg);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    CK(hipGetLastError());
    float ms;
    CK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<unsigned long long> d((size_t)G * 16);
    CK(hipMemcpy(d.data(), dbg, d.size() * 8, hipMemcpyDeviceToHost));
    double ph[9] = {0}, cyc = 0, rt = 0;
    unsigned long long r0 = ~0ull, r1 = 0;
    for (int g = 0; g < G; ++g) {
      const unsigned long long* x = &d[(size_t)g * 16];
      for (int k = 1; k <= 8; ++k) ph[k] += (double)(x[k] - x[k - 1]) / G;
      cyc += (double)(x[8] - x[0]);
      rt += (double)(x[14] - x[15]) / 100.0;
      r0 = std::min(r0, x[15]);
      r1 = std::max(r1, x[14]);
    }
    printf("rep %d, %s: event %.2f us, workgroups span %.2f us, shader clock %.0f MHz\n", rep, kinds[kind],
           ms * 1e3, (r1 - r0) / 100.0, cyc / rt);
    for (int k = 1; k <= 8; ++k) printf("   %-20s %8.0f cycles\n", phase[k - 1], ph[k]);
  }
  printf("done\n");
  return 0;
}
