// C-ABI layer: argument validation, planning, workspace sizing and launch.
// Declared in include/smla.h.  Everything here runs on the host (the one
// device object is the static split scratch below); nothing is enqueued
// unless every check passes.
#include "smla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "smla_internal.h"

// Split-partial scratch of smla_fwd_static_scratch: one array per device (a
// __device__ object exists once in every device's memory).  In host code the
// name stands for a host-side shadow, not a device address: the device
// address is looked up per device with hipGetSymbolAddress and only that
// pointer is handed to kernels.
static __device__ __align__(256) char scratch[SMLA_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

smla_status fail(smla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
  int32_t num_splits;
  int32_t b_topk;
  int32_t slots_per_split;
  bool persistent;          // persistent schedule
  bool block_counts;        // per-token block counts computed ahead, into the workspace
  size_t workspace_bytes;
};


// Bytes of KV reachable with 32-bit offsets from the KV base: (s_kv - 1) *
// row stride + the row length when that is at most the buffer window, else 0.
uint32_t kv_window_bytes(const smla_fwd_params* p) {
  const int64_t row_bytes = p->kv_format == SMLA_KV_BF16 ? p->kv_stride_row * 2 : p->kv_stride_row;
  const int64_t row_len = p->kv_format == SMLA_KV_BF16      ? 2 * SMLA_D_QK
                          : p->kv_format == SMLA_KV_FP8_E4M3 ? SMLA_FP8_ROW_BYTES
                                                             : SMLA_FP4_ROW_BYTES;
  const int64_t window = p->s_kv > 0 ? (p->s_kv - 1) * row_bytes + row_len : 0;
  return window > 0 && window <= (int64_t)smla::kDummyOffset ? (uint32_t)window : 0u;
}

// Decode occupancy: a token's topk range is cut so that the grid holds at least
// about two workgroups per CU, with no part smaller than 64 slots and none
// larger than the LDS index buffer.
// Workgroups a split plan aims for: one per compute unit (the forward kernels
// hold more than half of a unit's LDS, so one workgroup is resident per unit).
constexpr int kTargetWorkgroups = 256;

smla_status check_and_plan(const smla_fwd_params* p, Plan* plan) {
  if (!p) return fail(SMLA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->d_qk != SMLA_D_QK || p->d_v != SMLA_D_V)
    return fail(SMLA_ERR_UNSUPPORTED, "d_qk=%d d_v=%d: only d_qk=%d, d_v=%d are built", p->d_qk,
                p->d_v, SMLA_D_QK, SMLA_D_V);
  if (p->s_q < 0) return fail(SMLA_ERR_INVALID_ARGUMENT, "s_q=%d is negative", p->s_q);
  if (p->h_q != 16 && p->h_q != 32 && p->h_q != 64 && p->h_q != 128)
    return fail(SMLA_ERR_UNSUPPORTED, "h_q=%d: supported 16, 32, 64, 128", p->h_q);
  if (p->topk < 1) return fail(SMLA_ERR_INVALID_ARGUMENT, "topk=%d must be >= 1", p->topk);
  if (p->s_kv < 1 || p->s_kv > 2147483647LL)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "s_kv=%lld out of [1, 2^31-1]", (long long)p->s_kv);
  if (!std::isfinite(p->sm_scale)) return fail(SMLA_ERR_INVALID_ARGUMENT, "sm_scale is not finite");
  if (p->kv_format != SMLA_KV_BF16 && p->kv_format != SMLA_KV_FP8_E4M3 &&
      p->kv_format != SMLA_KV_FP4_E2M1)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "kv_format=%d unknown", p->kv_format);
  if (p->b_topk != 0 && p->b_topk != 32 && p->b_topk != 64 && p->b_topk != 128)
    return fail(SMLA_ERR_UNSUPPORTED, "b_topk=%d: supported 32, 64, 128 (0 = auto)", p->b_topk);
  if (p->num_splits < 0) return fail(SMLA_ERR_INVALID_ARGUMENT, "num_splits=%d is negative", p->num_splits);
  if (p->schedule < SMLA_SCHEDULE_AUTO || p->schedule > SMLA_SCHEDULE_PERSISTENT)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "schedule=%d unknown", p->schedule);
  if (p->persistent_workgroups < 0 || p->persistent_workgroups > 65535)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "persistent_workgroups=%d outside [0, 65535]",
                p->persistent_workgroups);

  if (p->s_q > 0) {
    if (!p->q || !p->kv || !p->indices || !p->out || !p->lse)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
    if (!aligned16(p->q) || !aligned16(p->kv) || !aligned16(p->out))
      return fail(SMLA_ERR_INVALID_ARGUMENT, "q, kv and out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(p->lse) % 4 || reinterpret_cast<uintptr_t>(p->indices) % 4)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "lse and indices must be 4-byte aligned");
    // bf16 rows: strides multiples of 8 elements keep every row 16-byte aligned.
    // Read-only Q may use any token stride (even 0, to broadcast one token).
    if (p->q_stride_head < SMLA_D_QK || p->q_stride_head % 8 || p->q_stride_token < 0 ||
        p->q_stride_token % 8)
      return fail(SMLA_ERR_INVALID_ARGUMENT,
                  "q strides (token %lld, head %lld): need head >= 576, token >= 0, both multiples "
                  "of 8", (long long)p->q_stride_token, (long long)p->q_stride_head);
    if (p->out_stride_head < SMLA_D_V || p->out_stride_head % 8 || p->out_stride_token % 8 ||
        p->out_stride_token < p->out_stride_head * p->h_q)
      return fail(SMLA_ERR_INVALID_ARGUMENT,
                  "out strides (token %lld, head %lld): need head >= 512, token >= h_q*head, both "
                  "multiples of 8", (long long)p->out_stride_token, (long long)p->out_stride_head);
    if (p->lse_stride_token < p->h_q)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "lse_stride_token=%lld < h_q",
                  (long long)p->lse_stride_token);
    if (p->indices_stride_token < 0)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "indices_stride_token=%lld is negative",
                  (long long)p->indices_stride_token);
    if (p->kv_format == SMLA_KV_BF16) {
      if (p->kv_stride_row < SMLA_D_QK || p->kv_stride_row % 8)
        return fail(SMLA_ERR_INVALID_ARGUMENT,
                    "kv_stride_row=%lld elements: need >= 576 and a multiple of 8",
                    (long long)p->kv_stride_row);
    } else {
      const int row = p->kv_format == SMLA_KV_FP8_E4M3 ? SMLA_FP8_ROW_BYTES : SMLA_FP4_ROW_BYTES;
      if (p->kv_stride_row < row || p->kv_stride_row % 16)
        return fail(SMLA_ERR_INVALID_ARGUMENT,
                    "kv_stride_row=%lld bytes: need >= %d and a multiple of 16",
                    (long long)p->kv_stride_row, row);
    }
  }

  Plan pl{};
  // The quantised-KV paths are built for B_TOPK 32 only.
  if (p->kv_format != SMLA_KV_BF16 && p->b_topk != 0 && p->b_topk != 32)
    return fail(SMLA_ERR_UNSUPPORTED, "quantised KV supports b_topk 32 only");
  const int32_t max_part = p->kv_format == SMLA_KV_FP8_E4M3 ? SMLA_MAX_SLOTS_PER_SPLIT_FP8
                                                            : SMLA_MAX_SLOTS_PER_SPLIT;
  const int32_t min_splits = (p->topk + max_part - 1) / max_part;
  int32_t ns = p->num_splits;
  if (ns == 0) {
    ns = min_splits;
    const int64_t units = (int64_t)p->s_q * (p->h_q > 64 ? p->h_q / 64 : 1);   // workgroups per split
    // (the persistent schedule runs one split per token: no occupancy splits)
    if (p->schedule != SMLA_SCHEDULE_PERSISTENT && units > 0 && units * ns < kTargetWorkgroups) {
      const int32_t want = (int32_t)((kTargetWorkgroups + units - 1) / units);
      const int32_t cap = (p->topk + 63) / 64;   // parts of at least 64 slots
      ns = want < cap ? want : cap;
      if (ns < min_splits) ns = min_splits;
    }
  }
  if (ns < min_splits)
    return fail(SMLA_ERR_UNSUPPORTED, "num_splits=%d: topk=%d needs at least %d parts of <= %d slots",
                ns, p->topk, min_splits, max_part);
  if (ns > p->topk) ns = p->topk;
  pl.num_splits = ns;
  pl.slots_per_split = (p->topk + ns - 1) / ns;
  // the parts actually used may be fewer than ns after rounding up
  pl.num_splits = (p->topk + pl.slots_per_split - 1) / pl.slots_per_split;
  // Block size: long splits (the pipelined 64-head kernel, from 1024 slots)
  // and quantised KV run B_TOPK 32; short bf16 splits of 64-head workgroups
  // run 64 (measured on the 128-head decode workload: 35.1 vs 39.5 us with
  // 2 splits, 44.0 vs 47.4 us with 4).
  pl.b_topk = p->b_topk ? p->b_topk
                        : (p->kv_format == SMLA_KV_BF16 && p->h_q >= 64 && pl.slots_per_split < 1024) ? 64
                                                                                                      : 32;
  if ((int64_t)p->s_q * pl.num_splits * (p->h_q > 64 ? 2 : 1) + 8 > 2147483647LL)
    return fail(SMLA_ERR_UNSUPPORTED, "grid of s_q*num_splits workgroups is too large");
  // Persistent schedule: bf16 KV in the 32-bit window, 64 heads, one split of
  // the pipelined kernel's length, B_TOPK 32.
  const bool can_persist = p->kv_format == SMLA_KV_BF16 && p->h_q == 64 && pl.num_splits == 1 &&
                           pl.slots_per_split >= smla::kPipeMinSlots && pl.b_topk == 32 &&
                           kv_window_bytes(p) != 0 && p->s_q <= (1 << 24);
  if (p->schedule == SMLA_SCHEDULE_PERSISTENT && !can_persist)
    return fail(SMLA_ERR_UNSUPPORTED,
                "persistent schedule: built for bf16 KV within 4 GB, h_q 64, one split, topk >= %d "
                "and b_topk 32", smla::kPipeMinSlots);
  pl.persistent = can_persist && p->schedule == SMLA_SCHEDULE_PERSISTENT;
  // One split of the pipelined kernel in the 32-bit window: each token's
  // block count is computed ahead by one pass over the index rows, so that a
  // workgroup starts its gathers without scanning its row first.
  pl.block_counts = pl.persistent || (p->kv_format == SMLA_KV_BF16 && p->h_q >= 64 && pl.num_splits == 1 &&
                                      pl.slots_per_split >= smla::kPipeMinSlots && pl.b_topk == 32 &&
                                      kv_window_bytes(p) != 0 && p->s_q <= (1 << 24));
  pl.workspace_bytes = 0;
  if (pl.num_splits > 1) {
    const size_t parts = (size_t)p->s_q * pl.num_splits * p->h_q;
    pl.workspace_bytes = parts * SMLA_D_V * sizeof(uint16_t) + ((parts * sizeof(float) + 255) & ~size_t(255));
  } else if (pl.block_counts) {
    pl.workspace_bytes = ((size_t)p->s_q * sizeof(int32_t) + 255) & ~size_t(255);
  }
  *plan = pl;
  return SMLA_OK;
}

// Compute units of the device that runs `stream`, queried once per device.
constexpr int kMaxDevicesCu = 64;
std::mutex g_cu_mutex;
int g_cu_count[kMaxDevicesCu] = {};

smla_status compute_units(hipStream_t stream, int* out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevicesCu)
    return fail(SMLA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevicesCu);
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n < 1)
      return fail(SMLA_ERR_HIP, "compute units of device %d: %s", dev, hipGetErrorString(e));
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return SMLA_OK;
}

// Fill the kernel arguments for a checked plan and launch it.  idx/idx_st:
// the (physical) indices to use; split_ws: the split-partials region.
smla_status launch_plan(const smla_fwd_params* p, const Plan& pl, const int32_t* idx, int64_t idx_st,
                        char* split_ws, hipStream_t stream) {
  smla::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(p->q);
  a.q_st = p->q_stride_token;
  a.q_sh = p->q_stride_head;
  a.kv = static_cast<const char*>(p->kv);
  a.kv_row_bytes = p->kv_format == SMLA_KV_BF16 ? p->kv_stride_row * 2 : p->kv_stride_row;
  a.idx = idx;
  a.idx_st = idx_st;
  a.out = static_cast<uint16_t*>(p->out);
  a.out_st = p->out_stride_token;
  a.out_sh = p->out_stride_head;
  a.lse = p->lse;
  a.lse_st = p->lse_stride_token;
  if (pl.num_splits > 1) {
    const size_t parts = (size_t)p->s_q * pl.num_splits * p->h_q;
    a.ws_lse = reinterpret_cast<float*>(split_ws);
    a.ws_o = reinterpret_cast<uint16_t*>(split_ws + ((parts * sizeof(float) + 255) & ~size_t(255)));
  }
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.topk = p->topk;
  a.slots_per_split = pl.slots_per_split;
  a.num_splits = pl.num_splits;
  a.head_groups = p->h_q > 64 ? p->h_q / 64 : 1;
  a.inner_groups = 1;
  if (p->kv_format == SMLA_KV_BF16 && p->h_q > 64 && pl.slots_per_split <= smla::kShortSlots) {
    // A short split is one block resident in LDS: one workgroup gathers the
    // rows once and runs both head groups over them.
    a.inner_groups = a.head_groups;
    a.head_groups = 1;
  }
  a.s_kv = p->s_kv;
  a.scale_log2 = p->sm_scale * 1.4426950408889634f;
  a.kv_window_bytes = kv_window_bytes(p);
  a.token_blocks = nullptr;
  if (pl.block_counts) {
    int32_t* nb = reinterpret_cast<int32_t*>(split_ws);
    hipError_t e = smla::launch_token_blocks(a, nb, stream);
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    a.token_blocks = nb;
    if (pl.persistent) {
      int grid = p->persistent_workgroups;
      if (grid == 0) {
        const smla_status cs = compute_units(stream, &grid);
        if (cs != SMLA_OK) return cs;
      }
      e = smla::launch_bf16_persist(a, grid, stream);
      if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
      return SMLA_OK;
    }
  }
  const hipError_t e = smla::launch_fwd(a, pl.b_topk, p->kv_format, stream);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

// Paged-KV arguments (the base parameters are already checked).
smla_status check_paged(const smla_fwd_params* p, const smla_paged_kv* pg) {
  if (!pg) return fail(SMLA_ERR_INVALID_ARGUMENT, "paged is NULL");
  if (pg->page_size < 1) return fail(SMLA_ERR_INVALID_ARGUMENT, "page_size=%d must be >= 1", pg->page_size);
  if (pg->table_width < 1)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "table_width=%d must be >= 1", pg->table_width);
  if ((int64_t)pg->table_width * pg->page_size > 2147483647LL)
    return fail(SMLA_ERR_UNSUPPORTED, "table_width*page_size exceeds the int32 logical positions");
  if (p->s_kv % pg->page_size)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "s_kv=%lld is not a whole number of pages of %d rows",
                (long long)p->s_kv, pg->page_size);
  if (pg->block_table_stride_token < 0)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "block_table_stride_token=%lld is negative",
                (long long)pg->block_table_stride_token);
  if (p->s_q > 0) {
    if (!pg->block_table) return fail(SMLA_ERR_INVALID_ARGUMENT, "block_table is NULL");
    if (reinterpret_cast<uintptr_t>(pg->block_table) % 4)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "block_table must be 4-byte aligned");
  }
  return SMLA_OK;
}

// Candidate plans for smla_fwd_tune: the planner's own plan first, then the
// split counts below with each supported block size, every valid plan once.
int tune_candidates(const smla_fwd_params* p, Plan* out, int maxn) {
  static const int32_t kSplits[] = {0, 1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
  const int32_t bts[2] = {32, 64};
  const int nbt = p->kv_format == SMLA_KV_BF16 ? 2 : 1;
  int n = 0;
  for (int32_t ns : kSplits) {
    for (int b = 0; b < nbt; ++b) {
      smla_fwd_params q = *p;
      q.num_splits = ns;
      q.b_topk = bts[b];
      Plan pl;
      if (check_and_plan(&q, &pl) != SMLA_OK) continue;
      bool seen = false;
      for (int i = 0; i < n; ++i)
        seen |= out[i].num_splits == pl.num_splits && out[i].b_topk == pl.b_topk;
      if (!seen && n < maxn) out[n++] = pl;
    }
  }
  g_last_error[0] = 0;   // rejected candidates are not a failure of the call
  return n;
}
constexpr int kMaxTuneCandidates = 32;

// Bytes of the translated-index region at the start of a paged workspace.
size_t translated_bytes(const smla_fwd_params* p) {
  return ((size_t)p->s_q * (size_t)p->topk * sizeof(int32_t) + 255) & ~size_t(255);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`, looked up once
// per device with that device current.
smla_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SMLA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(SMLA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(SMLA_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SMLA_OK;
}

}  // namespace

extern "C" {

smla_status smla_fwd_plan(const smla_fwd_params* p, int32_t* num_splits, int32_t* b_topk) {
  Plan pl;
  const smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  if (num_splits) *num_splits = pl.num_splits;
  if (b_topk) *b_topk = pl.b_topk;
  return SMLA_OK;
}

smla_status smla_fwd_schedule(const smla_fwd_params* p, int32_t* schedule) {
  if (!schedule) return fail(SMLA_ERR_INVALID_ARGUMENT, "schedule is NULL");
  Plan pl;
  const smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  *schedule = pl.persistent ? SMLA_SCHEDULE_PERSISTENT : SMLA_SCHEDULE_GRID;
  return SMLA_OK;
}

smla_status smla_fwd_workspace_size(const smla_fwd_params* p, size_t* bytes) {
  if (!bytes) return fail(SMLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan pl;
  const smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  *bytes = pl.workspace_bytes;
  return SMLA_OK;
}

smla_status smla_fwd(const smla_fwd_params* p, void* stream) {
  Plan pl;
  const smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  if (p->s_q == 0) return SMLA_OK;
  if (pl.workspace_bytes) {
    if (!p->workspace || p->workspace_bytes < pl.workspace_bytes)
      return fail(SMLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.workspace_bytes,
                  p->workspace ? p->workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(p->workspace) % 256)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  return launch_plan(p, pl, p->indices, p->indices_stride_token, static_cast<char*>(p->workspace),
                     static_cast<hipStream_t>(stream));
}

smla_status smla_fwd_static_scratch(const smla_fwd_params* p, void* stream) {
  Plan pl;
  const smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  if (p->s_q == 0) return SMLA_OK;
  if (pl.workspace_bytes > SMLA_STATIC_SCRATCH_BYTES)
    return fail(SMLA_ERR_WORKSPACE,
                "the plan's split partials need %zu bytes, more than the %u-byte static scratch "
                "(fewer splits or tokens per call fit)", pl.workspace_bytes,
                (unsigned)SMLA_STATIC_SCRATCH_BYTES);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (pl.workspace_bytes) {
    const smla_status e = scratch_address(st, &ws);
    if (e != SMLA_OK) return e;
  }
  return launch_plan(p, pl, p->indices, p->indices_stride_token, static_cast<char*>(ws), st);
}

smla_status smla_fwd_paged_workspace_size(const smla_fwd_params* p, const smla_paged_kv* pg,
                                          size_t* bytes) {
  if (!bytes) return fail(SMLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan pl;
  smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  s = check_paged(p, pg);
  if (s != SMLA_OK) return s;
  *bytes = translated_bytes(p) + pl.workspace_bytes;
  return SMLA_OK;
}

smla_status smla_fwd_paged(const smla_fwd_params* p, const smla_paged_kv* pg, void* stream) {
  Plan pl;
  smla_status s = check_and_plan(p, &pl);
  if (s != SMLA_OK) return s;
  s = check_paged(p, pg);
  if (s != SMLA_OK) return s;
  if (p->s_q == 0) return SMLA_OK;
  const size_t tb = translated_bytes(p);
  const size_t need = tb + pl.workspace_bytes;
  if (!p->workspace || p->workspace_bytes < need)
    return fail(SMLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                p->workspace ? p->workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(p->workspace) % 256)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  int32_t* phys = static_cast<int32_t*>(p->workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = smla::launch_paged_translate(
      p->indices, p->indices_stride_token, pg->block_table, pg->block_table_stride_token,
      pg->table_width, pg->page_size, p->s_kv / pg->page_size, p->s_q, p->topk, phys, st);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return launch_plan(p, pl, phys, p->topk, static_cast<char*>(p->workspace) + tb, st);
}

smla_status smla_fwd_tune_workspace_size(const smla_fwd_params* p, size_t* bytes) {
  if (!bytes) return fail(SMLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan base;
  const smla_status s = check_and_plan(p, &base);
  if (s != SMLA_OK) return s;
  Plan c[kMaxTuneCandidates];
  const int n = tune_candidates(p, c, kMaxTuneCandidates);
  size_t need = base.workspace_bytes;
  for (int i = 0; i < n; ++i) need = c[i].workspace_bytes > need ? c[i].workspace_bytes : need;
  *bytes = need;
  return SMLA_OK;
}

smla_status smla_fwd_tune(const smla_fwd_params* p, void* stream, int32_t iterations,
                          int32_t* num_splits, int32_t* b_topk, float* microseconds) {
  if (!num_splits || !b_topk)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "num_splits and b_topk outputs must not be NULL");
  if (iterations < 1 || iterations > 1000)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "iterations=%d outside [1, 1000]", iterations);
  Plan base;
  smla_status s = check_and_plan(p, &base);
  if (s != SMLA_OK) return s;
  Plan c[kMaxTuneCandidates];
  const int n = tune_candidates(p, c, kMaxTuneCandidates);
  size_t need = base.workspace_bytes;
  for (int i = 0; i < n; ++i) need = c[i].workspace_bytes > need ? c[i].workspace_bytes : need;
  if (p->s_q == 0 || n == 0) {
    *num_splits = base.num_splits;
    *b_topk = base.b_topk;
    if (microseconds) *microseconds = 0.f;
    return SMLA_OK;
  }
  if (need && (!p->workspace || p->workspace_bytes < need))
    return fail(SMLA_ERR_WORKSPACE, "workspace of %zu bytes needed for the candidates, %zu given",
                need, p->workspace ? p->workspace_bytes : (size_t)0);
  if (need && reinterpret_cast<uintptr_t>(p->workspace) % 256)
    return fail(SMLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(SMLA_ERR_HIP, "hipEventCreate failed");
  }
  float best = -1.f;
  int best_i = 0;
  for (int i = 0; i < n && s == SMLA_OK; ++i) {
    s = launch_plan(p, c[i], p->indices, p->indices_stride_token, static_cast<char*>(p->workspace), st);
    if (s != SMLA_OK) break;                                    // warm-up launch
    if (hipEventRecord(e0, st) != hipSuccess) { s = fail(SMLA_ERR_HIP, "hipEventRecord failed"); break; }
    for (int k = 0; k < iterations && s == SMLA_OK; ++k)
      s = launch_plan(p, c[i], p->indices, p->indices_stride_token, static_cast<char*>(p->workspace), st);
    if (s != SMLA_OK) break;
    float ms = 0.f;
    if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      s = fail(SMLA_ERR_HIP, "timing a candidate plan failed");
      break;
    }
    const float us = ms * 1000.f / iterations;
    if (best < 0.f || us < best) {
      best = us;
      best_i = i;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (s != SMLA_OK) return s;
  *num_splits = c[best_i].num_splits;
  *b_topk = c[best_i].b_topk;
  if (microseconds) *microseconds = best;
  return SMLA_OK;
}

smla_status smla_pack_fp8_kv_host(const uint8_t* codes, const float* scales, int64_t rows,
                                  void* packed) {
  if (rows < 0) return fail(SMLA_ERR_INVALID_ARGUMENT, "rows=%lld is negative", (long long)rows);
  if (rows > 0 && (!codes || !scales || !packed))
    return fail(SMLA_ERR_INVALID_ARGUMENT, "a pointer is NULL");
  char* dst = static_cast<char*>(packed);
  for (int64_t r = 0; r < rows; ++r) {
    char* row = dst + r * SMLA_FP8_ROW_BYTES;
    std::memcpy(row, codes + r * SMLA_D_QK, SMLA_D_QK);
    std::memcpy(row + SMLA_D_QK, scales + r * SMLA_FP8_NUM_GROUPS, SMLA_FP8_NUM_GROUPS * sizeof(float));
    std::memset(row + SMLA_D_QK + SMLA_FP8_NUM_GROUPS * sizeof(float), 0,
                SMLA_FP8_ROW_BYTES - SMLA_D_QK - SMLA_FP8_NUM_GROUPS * sizeof(float));
  }
  return SMLA_OK;
}

smla_status smla_pack_fp4_kv_host(const uint8_t* codes, const float* scales, int64_t rows,
                                  void* packed) {
  if (rows < 0) return fail(SMLA_ERR_INVALID_ARGUMENT, "rows=%lld is negative", (long long)rows);
  if (rows > 0 && (!codes || !scales || !packed))
    return fail(SMLA_ERR_INVALID_ARGUMENT, "a pointer is NULL");
  for (int64_t i = 0; i < rows * SMLA_D_QK; ++i)
    if (codes[i] > 15)
      return fail(SMLA_ERR_INVALID_ARGUMENT, "code %d at element %lld is not a 4-bit code",
                  (int)codes[i], (long long)i);
  char* dst = static_cast<char*>(packed);
  constexpr int kCodeBytes = SMLA_D_QK / 2;
  for (int64_t r = 0; r < rows; ++r) {
    unsigned char* row = reinterpret_cast<unsigned char*>(dst + r * SMLA_FP4_ROW_BYTES);
    const uint8_t* c = codes + r * SMLA_D_QK;
    for (int k = 0; k < kCodeBytes; ++k) row[k] = (unsigned char)(c[2 * k] | (c[2 * k + 1] << 4));
    std::memcpy(row + kCodeBytes, scales + r * SMLA_FP8_NUM_GROUPS, SMLA_FP8_NUM_GROUPS * sizeof(float));
    std::memset(row + kCodeBytes + SMLA_FP8_NUM_GROUPS * sizeof(float), 0,
                SMLA_FP4_ROW_BYTES - kCodeBytes - SMLA_FP8_NUM_GROUPS * sizeof(float));
  }
  return SMLA_OK;
}

const char* smla_status_string(int32_t status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SMLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* smla_last_error(void) { return g_last_error; }

int32_t smla_abi_version(void) { return SMLA_ABI_VERSION; }

}  // extern "C"
