// LDS operand-read patterns of the forward kernels, timed alone: the transposed
// V reads (ds_read_b64_tr_b16) and the K reads (ds_read_b128) of the shared
// stage layout (units of 8 rows x 8 chunks, slot = chunk·8 + row), against a
// layout of 4-row blocks (4 rows x 16 chunks per 1 KB, slot = chunk·4 + row,
// with three choices of an XOR of the chunk by the block index) that a gather
// of 256 contiguous bytes per row would fill.  One 256-thread workgroup per
// CU; each wave issues ITER x 8 reads of one pattern on a 64 KB LDS buffer
// (every address below 32 KB + 8 bytes).  Printed: ns per read per wave (HIP
// events); LDS bank conflicts come from rocprofv3 --pmc SQ_LDS_BANK_CONFLICT.
//
// Build: python bench/micro/build.py; run ./bench/micro/lds_patterns.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
#define LDS_AS __attribute__((address_space(3)))
constexpr int ITER = 2048;

// Byte offset of lane (g = lane/16, n = lane%16) of wave w for read jj of pattern P.
__device__ int offset_of(int P, int lane, int w, int jj) {
  const int g = lane >> 4, n = lane & 15, e = (n >> 1) & 1;
  if (P == 0) {            // V, unit layout: rows 4g + n/4, chunks 16w + 8(jj/4) + 2(jj%4) + e
    const int rb = g >> 1, r8 = 4 * (g & 1) + (n >> 2), c8 = 2 * (jj & 3) + e;
    return 8192 * w + (jj >> 2) * 4096 + (rb * 64 + c8 * 8 + r8) * 16 + (n & 1) * 8;
  }
  if (P <= 3) {            // V, 4-row blocks (block = rows 4g..4g+3 of chunk group w)
    const int x = P == 1 ? 0 : P == 2 ? g : (g & 1);
    const int lo = (2 * (jj & 1) + e) ^ x;
    return 8192 * w + g * 1024 + ((lo << 2) + (n >> 2)) * 16 + (n & 1) * 8 + 256 * ((jj >> 1) & 1) +
           512 * (jj >> 2);
  }
  if (P == 4) {            // K, unit layout: rows n, chunk 4jj + g
    return ((n >> 3) * 64 + (4 * (jj & 1) + g) * 8 + (n & 7)) * 16 + (jj >> 1) * 4096;
  }
  const int q = n >> 2, x = P == 5 ? 0 : P == 6 ? q : (q & 1);   // K, 4-row blocks
  return q * 1024 + (((g ^ x) << 2) + (n & 3)) * 16 + 256 * (jj & 3) + (jj >> 2) * 8192;
}

template <int P>
__global__ __launch_bounds__(256) void lds_kernel(int* out) {
  __shared__ __attribute__((aligned(1024))) char buf[65536];
  for (int i = threadIdx.x; i < 65536 / 4; i += 256) ((int*)buf)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int offs[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) offs[jj] = offset_of(P, lane, w, jj);
  int acc = 0;
  for (int it = 0; it < ITER; ++it) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if constexpr (P <= 3) {
        const i16x4 v =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)((LDS_AS char*)(LDS_AS void*)buf + offs[jj]));
        acc ^= v[0] ^ v[3];
      } else {
        const i32x4 v = *(const LDS_AS i32x4*)((LDS_AS char*)(LDS_AS void*)buf + offs[jj]);
        acc ^= v[0] ^ v[3];
      }
    }
    asm volatile("" ::: "memory");   // re-read every iteration
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

int main() {
  int* d = nullptr;
  CHECK(hipMalloc(&d, 256 * 256 * 4));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const char* names[8] = {"V (tr16), 8-row units", "V (tr16), 4-row blocks, no XOR", "V (tr16), 4-row blocks, XOR q",
                          "V (tr16), 4-row blocks, XOR q%2", "K (b128), 8-row units", "K (b128), 4-row blocks, no XOR",
                          "K (b128), 4-row blocks, XOR q", "K (b128), 4-row blocks, XOR q%2"};
  void (*ks[8])(int*) = {lds_kernel<0>, lds_kernel<1>, lds_kernel<2>, lds_kernel<3>,
                         lds_kernel<4>, lds_kernel<5>, lds_kernel<6>, lds_kernel<7>};
  for (int p = 0; p < 8; ++p) hipLaunchKernelGGL(ks[p], dim3(256), dim3(256), 0, 0, d);   // warm-up
  CHECK(hipDeviceSynchronize());
  for (int p = 0; p < 8; ++p) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(ks[p], dim3(256), dim3(256), 0, 0, d);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("| %s | %.2f |\n", names[p], ms * 1e6 / (ITER * 8.0));
    std::fflush(stdout);
  }
  CHECK(hipFree(d));
  return 0;
}
