// Issue-rate measurements behind the forward kernels' design: how fast one
// wave per SIMD issues v_mfma_f32_16x16x32_bf16
//   1. from registers, with 1..16 independent accumulator chains;
//   2. with independent fp32 FMAs between the MFMAs (one and two waves per SIMD);
//   3. with its A operand read from LDS (ds_read_b128, 1 KB per wave) a fixed
//      number of MFMAs ahead, as the QK loop of the kernels does.
// One workgroup of 4 (or 8) waves per CU, 256 workgroups.  Each wave's loop is
// timed with the shader cycle counter (s_memtime), the launch with HIP events.
// Register-only work apart from one store per thread and the LDS reads of 3,
// which stay inside a 64 KB dynamic LDS buffer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <type_traits>

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kWorkgroups = 256;
constexpr int kLdsBytes = 65536;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// CH accumulator chains, VALU independent FMAs after each MFMA.
template <int CH, int VALU>
__global__ void mfma_chains(float* out, unsigned long long* cyc, int iters, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed + i);
    b[i] = (__bf16)(seed - i);
  }
  f32x4 acc[CH];
  for (int k = 0; k < CH; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float v[16];
  for (int k = 0; k < 16; ++k) v[k] = seed * (k + 1);
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < VALU; ++j) v[(VALU * k + j) & 15] = v[(VALU * k + j) & 15] * 1.0001f + 0.5f;
    }
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  float s = 0.f;
  for (int k = 0; k < CH; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  for (int k = 0; k < 16; ++k) s += v[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
}

// 8 chains; MFMA i takes the A operand read PF MFMAs earlier from LDS (lane l
// reads 16 bytes at 1 KB·slot + 16·l: conflict-free, offsets below 48 KB).
template <int PF>
__global__ void mfma_lds_operand(float* out, unsigned long long* cyc, int iters) {
  constexpr int N = 24, CH = 8;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kLdsBytes / 4; i += blockDim.x) ((float*)lds)[i] = 0.001f * (i & 255);
  __syncthreads();
  const LDS_AS char* base = (const LDS_AS char*)(LDS_AS void*)lds + lane * 16;
  bf16x8 b;
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(0.5f + i);
  f32x4 acc[CH];
  for (int k = 0; k < CH; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 abuf[PF];
  static_for<0, PF>([&](auto I) {
    abuf[decltype(I)::value] = *(const LDS_AS bf16x8*)(base + decltype(I)::value * 1024);
  });
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N>([&](auto I) {
      constexpr int i = decltype(I)::value;
      acc[i % CH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], b, acc[i % CH], 0, 0, 0);
      abuf[i % PF] = *(const LDS_AS bf16x8*)(base + ((i + PF) % 48) * 1024);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  float s = 0.f;
  for (int k = 0; k < CH; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  for (int k = 0; k < PF; ++k) s += (float)abuf[k][0];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

struct Buffers {
  float* out;
  unsigned long long* cyc;
};

// Runs the kernel three times; prints counter cycles per MFMA of one wave
// (mean over workgroups of wave 0's loop) and the last launch's time per MFMA
// per SIMD (4 waves per workgroup: one per SIMD; 8: two).
template <typename K, typename... Args>
void run(const char* name, K kernel, int threads, int lds, double mfmas_per_wave, const Buffers& b,
         Args... args) {
  check(hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds),
        "hipFuncSetAttribute");
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "hipEventCreate");
  check(hipEventCreate(&e1), "hipEventCreate");
  float ms = 0.f;
  for (int r = 0; r < 3; ++r) {
    check(hipEventRecord(e0, 0), "hipEventRecord");
    hipLaunchKernelGGL(kernel, dim3(kWorkgroups), dim3(threads), lds, 0, b.out, b.cyc, args...);
    check(hipGetLastError(), "launch");
    check(hipEventRecord(e1, 0), "hipEventRecord");
    check(hipDeviceSynchronize(), "hipDeviceSynchronize");
    check(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
  }
  unsigned long long host[kWorkgroups];
  check(hipMemcpy(host, b.cyc, sizeof(host), hipMemcpyDeviceToHost), "hipMemcpy");
  double sum = 0;
  for (int i = 0; i < kWorkgroups; ++i) sum += (double)host[i];
  const double waves_per_simd = threads / 256.0;
  std::printf("| %s | %.2f | %.2f |\n", name, sum / kWorkgroups / mfmas_per_wave,
              ms * 1e6 / (mfmas_per_wave * waves_per_simd));
  check(hipEventDestroy(e0), "hipEventDestroy");
  check(hipEventDestroy(e1), "hipEventDestroy");
}

}  // namespace

int main() {
  Buffers b;
  check(hipMalloc(&b.out, kWorkgroups * 512 * sizeof(float)), "hipMalloc");
  check(hipMalloc(&b.cyc, kWorkgroups * sizeof(unsigned long long)), "hipMalloc");
  const int it = 2048;
  std::printf("| case | counter cycles per MFMA of one wave | ns per MFMA per SIMD (launch) |\n|---|---|---|\n");
  run("1 chain", mfma_chains<1, 0>, 256, 0, it * 1.0, b, it, 1.0f);
  run("2 chains", mfma_chains<2, 0>, 256, 0, it * 2.0, b, it, 1.0f);
  run("4 chains", mfma_chains<4, 0>, 256, 0, it * 4.0, b, it, 1.0f);
  run("8 chains", mfma_chains<8, 0>, 256, 0, it * 8.0, b, it, 1.0f);
  run("16 chains", mfma_chains<16, 0>, 256, 0, it * 16.0, b, it, 1.0f);
  run("8 chains + 4 FMAs per MFMA", mfma_chains<8, 4>, 256, 0, it * 8.0, b, it, 1.0f);
  run("16 chains + 2 FMAs per MFMA", mfma_chains<16, 2>, 256, 0, it * 16.0, b, it, 1.0f);
  run("two waves per SIMD, 8 chains", mfma_chains<8, 0>, 512, 0, it * 8.0, b, it, 1.0f);
  run("two waves per SIMD, 8 chains + 4 FMAs per MFMA", mfma_chains<8, 4>, 512, 0, it * 8.0, b, it, 1.0f);
  const int itl = 1024;
  run("A from LDS, 4 reads in flight", mfma_lds_operand<4>, 256, kLdsBytes, itl * 24.0, b, itl);
  run("A from LDS, 8 reads in flight", mfma_lds_operand<8>, 256, kLdsBytes, itl * 24.0, b, itl);
  run("A from LDS, 12 reads in flight", mfma_lds_operand<12>, 256, kLdsBytes, itl * 24.0, b, itl);
  check(hipFree(b.out), "hipFree");
  check(hipFree(b.cyc), "hipFree");
  return 0;
}
