// Internal interface between the C-ABI layer (smla_api.cpp) and the gfx950
// kernels (smla_fwd.cuh, instantiated by the smla_fwd_*.hip units; dispatch in
// smla_launch.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytesBf16 = kDqk * 2;   // 1152: nine 128-byte lines
constexpr int kFp8RowBytes = 640;         // 576 codes + 5 float32 scales + pad
constexpr int kFp4RowBytes = 320;         // 288 bytes of two codes each + 5 float32 scales + pad
constexpr int kMaxSlotsPerSplit = 2048;
// Slots per split from which the pipelined 64-head bf16 kernel runs (and the
// persistent schedule, which is built on it, may)
constexpr int kPipeMinSlots = 1024;
// Slots per split up to which a bf16 split runs as one block in the short
// kernel (four 32-row stages resident at once)
constexpr int kShortSlots = 128;
// fp8 KV: the raw-row ring and two bf16 stages leave room for 1536 indices
constexpr int kMaxSlotsPerSplitFp8 = 1536;
// Buffer-load offset past every KV window: a gather for a block past the end
// of a split loads from here, which the hardware drops (range check of the
// buffer resource), so the load costs no memory traffic.  Windows (last byte
// of the KV + 1) must not exceed it; the largest instruction offset added to
// it (1 KB) keeps the sum inside 32 bits.
constexpr uint32_t kDummyOffset = 0xFFFFF000u;

// Everything one launch of the forward kernel needs, by value.
struct FwdArgs {
  const uint16_t* q;        // bf16 bits
  int64_t q_st, q_sh;       // elements
  const char* kv;           // bf16 rows or packed fp8 rows
  int64_t kv_row_bytes;     // bytes between consecutive KV rows
  const int32_t* idx;
  int64_t idx_st;
  uint16_t* out;            // bf16 bits
  int64_t out_st, out_sh;
  float* lse;
  int64_t lse_st;
  uint16_t* ws_o;           // [s_q, num_splits, h_q, 512] bf16 bits: O/l of each part (split plans)
  float* ws_lse;            // [s_q, num_splits, h_q] fp32 (split plans)
  int32_t s_q, h_q, topk, slots_per_split, num_splits;
  int32_t head_groups;      // workgroups per (token, split): h_q / 64, at least 1
  // Groups of 64 heads that one workgroup runs in turn over the same gathered
  // blocks (1, or h_q / 64 when every block of a split fits in the stage ring
  // at once; head_groups is then 1).  bf16 KV, non-pipelined kernel only.
  int32_t inner_groups;
  int64_t s_kv;
  float scale_log2;         // sm_scale * log2(e)
  // Bytes of KV reachable with 32-bit offsets from kv: (s_kv - 1) * kv_row_bytes
  // + the row length when that is at most kDummyOffset (the gathers then use buffer
  // loads, whose hardware range check also covers every access), else 0 (the
  // gathers use 64-bit global addresses).
  uint32_t kv_window_bytes;
  // Blocks of each token up to its last valid slot (at least 1), computed by
  // a pass over the index rows before the forward kernel (single-split plans
  // in the 32-bit window; else null and each workgroup scans its own slots).
  const int32_t* token_blocks;
};

// KV row formats (the values of smla_kv_format).
enum KvFormat { kKvBf16 = 0, kKvFp8 = 1, kKvFp4 = 2 };

// Launch the forward pass (and the split combine when num_splits > 1) for a
// KV row format.  Returns the HIP error of the launches.
hipError_t launch_fwd(const FwdArgs& a, int b_topk, int kv_format, hipStream_t stream);

// Paged KV: logical index -> physical row through each token's block table
// (-1 when masked), written contiguously to phys [s_q, topk].
hipError_t launch_paged_translate(const int32_t* idx, int64_t idx_st, const int32_t* block_table,
                                  int64_t bt_st, int32_t table_width, int32_t page_size,
                                  int64_t num_pages, int32_t s_q, int32_t topk, int32_t* phys,
                                  hipStream_t stream);

// Per-token block counts (blocks up to the token's last valid slot, at least
// 1) into nb [s_q] (device scratch).
hipError_t launch_token_blocks(const FwdArgs& a, int32_t* nb, hipStream_t stream);

// Persistent schedule (bf16 KV, 64 heads, one split per token, KV within the
// 32-bit window; a.token_blocks set): `grid` persistent workgroups, each on a
// contiguous run of tokens of about equal block weight.
hipError_t launch_bf16_persist(const FwdArgs& a, int grid, hipStream_t stream);

// Forward kernel launchers per configuration (NW = waves per workgroup =
// heads per workgroup / 16; BT = B_TOPK), each instantiated in its own
// translation unit.
template <int NW, int BT>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t stream);
template <int NW>
hipError_t launch_bf16_b128(const FwdArgs& a, hipStream_t stream);
template <int NW>
hipError_t launch_fp8(const FwdArgs& a, hipStream_t stream);
template <int NW>
hipError_t launch_fp4(const FwdArgs& a, hipStream_t stream);

}  // namespace smla
