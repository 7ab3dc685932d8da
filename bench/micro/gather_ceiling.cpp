// Gather ceiling of the memory system: throughput of random-row gathers with
// the access patterns of the forward kernels, measured for the row sizes and
// table sizes of the sparse MLA workloads.
//
//   rows of 1152 bytes (bf16 KV) from 64 slices of 37.7 MB (decode: each
//     workgroup reads rows of one sequence), from one 75.5 MB table (prefill:
//     the KV is small enough for the 256 MB MALL) and from one 2.4 MB table
//     (small enough for each XCD's 4 MB L2: the load path's own limit)
//   rows of 640 bytes (packed fp8 KV) from 128 slices of 10.5 MB
//
// Access shapes of one wave instruction (64 lanes x 16 bytes):
//   lines:  eight random rows x one 128-byte line (the bf16 kernels' shape);
//   rows:   64 consecutive 16-byte chunks of the wave's eight rows laid end to
//           end, i.e. 1 KB of one or two rows (the raw-row shape of the
//           quantised kernels);
//   quads:  four rows x 256 bytes, and pairs: two rows x 512 bytes (1152-byte
//           rows only: eight such instructions cover the first 1 KB of the
//           group's eight rows, a ninth the last line of all eight).
// Loads: direct-to-LDS (what the kernels use) with D instructions in flight
// per wave, 4/8/16 waves per workgroup, one or two workgroups per CU; and
// plain loads into registers.  Every address lies inside the buffer: row =
// hash % rows_per_slice, byte offset inside the row < row_bytes.
//
// Build: python bench/micro/build.py; run ./bench/micro/gather_ceiling (no
// arguments).
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

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// s_waitcnt vmcnt(N) (other counters not waited on)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// MODE 0: direct-to-LDS 16-byte loads, at most D in flight per wave, lines shape.
// MODE 1: 16-byte loads into registers in batches of D, lines shape.
// MODE 2: direct-to-LDS 16-byte loads, at most D in flight per wave, rows shape.
// MODE 3 / 4: as MODE 0 in the quads / pairs shape.
template <int MODE, int D>
__global__ void gather_kernel(const char* __restrict__ kv, uint32_t rows_per_slice, uint32_t nslices,
                              int row_bytes, int groups_per_wave, uint32_t* sink) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lines = row_bytes / 128;
  const uint32_t slice = blockIdx.x % nslices;
  const char* base = kv + (uint64_t)slice * rows_per_slice * row_bytes;
  uint32_t acc = 0;
  if constexpr (MODE == 2) {
    // the group's eight rows end to end: instruction j covers chunks
    // 64j .. 64j + 63 of the 8 x row_bytes / 16 chunks
    const int chunks = row_bytes / 16;
    int issued = 0;
    for (int grp = 0; grp < groups_per_wave; ++grp) {
      for (int j = 0; j < lines; ++j) {
        const int c = j * 64 + lane;
        const int r = c / chunks, ch = c - r * chunks;
        const uint32_t row = mix32((blockIdx.x * 4096u + w * 512u + grp) * 8u + r) % rows_per_slice;
        __builtin_amdgcn_global_load_lds((const void*)(base + (uint64_t)row * row_bytes + ch * 16),
                                         (__attribute__((address_space(3))) void*)(lds + ((w * 8 + (issued & 7)) & 63) * 1024),
                                         16, 0, 0);
        wait_vmcnt<D>();
        ++issued;
      }
    }
  } else if constexpr (MODE == 3 || MODE == 4) {
    constexpr int R = MODE == 3 ? 4 : 2, L = 8 / R;   // rows and 128-byte lines per instruction
    int issued = 0;
    for (int grp = 0; grp < groups_per_wave; ++grp) {
      for (int j = 0; j < 8; ++j) {
        // rows (j % (8/R))·R .. +R of the group, lines (j / (8/R))·L .. +L
        const int r = (j % (8 / R)) * R + lane % R, ch = (j / (8 / R)) * L * 8 + lane / R;
        const uint32_t row = mix32((blockIdx.x * 4096u + w * 512u + grp) * 8u + r) % rows_per_slice;
        __builtin_amdgcn_global_load_lds((const void*)(base + (uint64_t)row * row_bytes + ch * 16),
                                         (__attribute__((address_space(3))) void*)(lds + ((w * 8 + (issued & 7)) & 63) * 1024),
                                         16, 0, 0);
        wait_vmcnt<D>();
        ++issued;
      }
      const uint32_t row = mix32((blockIdx.x * 4096u + w * 512u + grp) * 8u + (lane & 7)) % rows_per_slice;
      __builtin_amdgcn_global_load_lds((const void*)(base + (uint64_t)row * row_bytes + 1024 + ((lane >> 3) << 4)),
                                       (__attribute__((address_space(3))) void*)(lds + ((w * 8 + (issued & 7)) & 63) * 1024),
                                       16, 0, 0);
      wait_vmcnt<D>();
      ++issued;
    }
  } else if constexpr (MODE == 0) {
    int issued = 0;
    for (int grp = 0; grp < groups_per_wave; ++grp) {
      const uint32_t row = mix32((blockIdx.x * 4096u + w * 512u + grp) * 8u + (lane & 7)) % rows_per_slice;
      const char* rp = base + (uint64_t)row * row_bytes + ((lane >> 3) << 4);
      for (int j = 0; j < lines; ++j) {
        // 1 KB per instruction into one of 64 LDS slots (contents unused)
        __builtin_amdgcn_global_load_lds((const void*)(rp + 128 * j),
                                         (__attribute__((address_space(3))) void*)(lds + ((w * 8 + (issued & 7)) & 63) * 1024),
                                         16, 0, 0);
        wait_vmcnt<D>();
        ++issued;
      }
    }
  } else {
    const int nins = groups_per_wave * lines;
    for (int f = 0; f + D <= nins; f += D) {
      i32x4 r[D];
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const int grp = (f + k) / lines, j = (f + k) - grp * lines;
        const uint32_t row = mix32((blockIdx.x * 4096u + w * 512u + grp) * 8u + (lane & 7)) % rows_per_slice;
        r[k] = *(const i32x4*)(base + (uint64_t)row * row_bytes + ((lane >> 3) << 4) + 128 * j);
      }
#pragma unroll
      for (int k = 0; k < D; ++k) acc ^= (uint32_t)(r[k][0] ^ r[k][3]);
    }
  }
  wait_vmcnt<0>();
  if (acc == 0x12345678u) sink[0] = acc;   // keeps the register loads alive
}

struct Regime {
  int row_bytes;
  uint32_t rows_per_slice, nslices;
  const char* name;
};

}  // namespace

int main() {
  const uint64_t total = 64ull * 32768ull * 1152ull;   // 2.25 GiB: the largest regime
  char* kv = nullptr;
  uint32_t* sink = nullptr;
  CHECK(hipMalloc(&kv, total));
  CHECK(hipMemset(kv, 1, total));
  CHECK(hipMalloc(&sink, 4));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const Regime regimes[] = {
      {1152, 32768, 64, "bf16 rows, 64 slices of 37.7 MB (HBM)"},
      {640, 16384, 128, "fp8 rows, 128 slices of 10.5 MB (HBM)"},
      {1152, 65536, 1, "bf16 rows, one 75.5 MB table (MALL)"},
      {1152, 2048, 1, "bf16 rows, one 2.4 MB table (L2)"},
  };
  auto run = [&](auto kernel, const Regime& r, int waves, int wgs, int lds_bytes, int gpw, const char* kind, int d) {
    CHECK(hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes));
    for (int it = 0; it < 4; ++it) {   // three warm-up launches, the fourth timed
      if (it == 3) CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(kernel, dim3(wgs), dim3(waves * 64), lds_bytes, 0, kv, r.rows_per_slice, r.nslices,
                         r.row_bytes, gpw, sink);
      CHECK(hipGetLastError());
      if (it == 3) CHECK(hipEventRecord(e1));
    }
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double bytes = (double)wgs * waves * gpw * 8 * r.row_bytes;
    std::printf("| %s | %s | %d | %d | %d | %d | %.1f |\n", r.name, kind, d, waves, wgs, lds_bytes / 1024,
                bytes / ms / 1e6);
    std::fflush(stdout);
  };
  std::printf("| table | loads, shape | in flight per wave | waves per WG | WGs | LDS KB per WG | GB/s |\n");
  std::printf("|---|---|---|---|---|---|---|\n");
  for (const Regime& r : regimes) {
    for (int waves : {4, 8, 16}) {
      const int gpw = 256 / waves;   // 2048 rows per workgroup
      run(gather_kernel<0, 8>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, lines", 8);
      run(gather_kernel<0, 32>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, lines", 32);
      run(gather_kernel<2, 8>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, rows", 8);
      run(gather_kernel<2, 32>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, rows", 32);
      run(gather_kernel<1, 16>, r, waves, 1024, 100 * 1024, gpw, "registers, lines", 16);
      if (r.row_bytes == 1152 && waves <= 8) {
        run(gather_kernel<3, 8>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, quads", 8);
        run(gather_kernel<3, 32>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, quads", 32);
        run(gather_kernel<4, 8>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, pairs", 8);
        run(gather_kernel<4, 32>, r, waves, 1024, 100 * 1024, gpw, "direct-to-LDS, pairs", 32);
      }
    }
    // two workgroups per CU (64 KB of LDS each)
    run(gather_kernel<0, 32>, r, 4, 2048, 64 * 1024, 64, "direct-to-LDS, lines", 32);
    run(gather_kernel<2, 32>, r, 4, 2048, 64 * 1024, 64, "direct-to-LDS, rows", 32);
  }
  CHECK(hipFree(kv));
  CHECK(hipFree(sink));
  return 0;
}
