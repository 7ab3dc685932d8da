/*
 * smla.h -- C ABI of the sparse MLA attention forward library for AMD MI355X
 * (gfx950).
 *
 * The operation is defined on the page "Ascend Sparse Attention Forward
 * 算法与优化技术简析", section 数学建模 (mathematical model).  For every query
 * token t, independently:
 *
 *   gathered_kv = KV.index_select(indices[t])        [topk, d_qk]
 *   P   = Q[t] @ gathered_kv^T                       [h_q, topk]
 *   S   = softmax(P * sm_scale, dim=-1)              [h_q, topk]
 *   out = S @ gathered_kv[:, :d_v]                   [h_q, d_v]
 *   lse = log(sum_j exp(P * sm_scale))               [h_q]   (natural log)
 *
 * computed block by block with the online softmax and "skip scale" rule of
 * the same page, section 计算流程 (computation flow): running maxima and sums in
 * float32, S cast to bf16 before the product with V, a rescale of the output
 * accumulator only when some row's running maximum has grown by more than
 * RESCALE_THRES = 6 since the last rescale.
 *
 * Slots: an index outside [0, s_kv) (for example -1) masks its slot: weight
 * zero, row never read.  Repeated indices are separate slots.  A token (or a
 * split) with no valid slot yields out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises device memory.
 *  - Strides are in elements of the tensor's own type unless stated otherwise;
 *    the innermost dimension is always contiguous.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 *    default stream).
 *  - Every argument is validated on the host before anything is enqueued.  On
 *    any failure the call returns a non-zero smla_status, enqueues nothing,
 *    and smla_last_error() describes the cause.  No C++ exception crosses this
 *    interface; the device code has no error path (bad indices are masked).
 *  - The library keeps no state between calls; calls on different streams
 *    with separate outputs and workspaces may run concurrently.
 */
#ifndef SMLA_H_
#define SMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 6

/* The MLA shapes the kernels are built for: the query/key width d_qk is the
 * 512-wide latent plus the 64-wide rotary part, and V is the first 512 KV
 * columns. */
#define SMLA_D_QK 576
#define SMLA_D_V 512

/* fp8 KV cache: one float32 scale per group of 128 consecutive columns
 * (576 columns -> 5 groups, the last 64 wide).  Each token's codes and scales
 * sit in one 640-byte row, data next to scale (page section
 * "Decoding KV Cache Layout 优化"): bytes [0, 576) are the E4M3 codes, bytes
 * [576, 596) the five little-endian float32 scales, bytes [596, 640) padding.
 * Element value = e4m3(code) * scale[column / 128]. */
#define SMLA_FP8_GROUP 128
#define SMLA_FP8_NUM_GROUPS 5
#define SMLA_FP8_ROW_BYTES 640

/* fp4 KV cache: page "Ascend Sparse Attention Forward 算法与优化技术简析",
 * section 讨论 (item "Dequantize bound"), has decode read an FP8 or an FP4 KV
 * cache and dequantise it to bf16 before the matrix products, and its section
 * "Decoding KV Cache Layout 优化" keeps each token's data next to its scales.
 * Neither fixes the 4-bit format; here: OCP MX E2M1 codes (1 sign, 2
 * exponent, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives), two per byte, with the same five float32 group scales.  A 320-byte row: bytes [0, 288)
 * hold column 2k in the low nibble and column 2k+1 in the high nibble of byte
 * k, bytes [288, 308) the five scales, bytes [308, 320) padding.
 * Element value = e2m1(code) * scale[column / 128]. */
#define SMLA_FP4_ROW_BYTES 320

/* Largest number of slots one workgroup handles; the planner splits the topk
 * range of a token into parts no larger than this (bf16 and fp4 KV / fp8 KV). */
#define SMLA_MAX_SLOTS_PER_SPLIT 2048
#define SMLA_MAX_SLOTS_PER_SPLIT_FP8 1536

typedef enum smla_status {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride or alignment */
  SMLA_ERR_UNSUPPORTED = 2,      /* valid request outside the built kernels */
  SMLA_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  SMLA_ERR_HIP = 4               /* a HIP runtime call failed */
} smla_status;

typedef enum smla_schedule {
  SMLA_SCHEDULE_AUTO = 0,
  SMLA_SCHEDULE_GRID = 1,
  SMLA_SCHEDULE_PERSISTENT = 2
} smla_schedule;

typedef enum smla_kv_format {
  SMLA_KV_BF16 = 0,     /* kv: bf16 [s_kv, 576], kv_stride_row in elements */
  SMLA_KV_FP8_E4M3 = 1, /* kv: packed 640-byte rows, kv_stride_row in BYTES */
  SMLA_KV_FP4_E2M1 = 2  /* kv: packed 320-byte rows, kv_stride_row in BYTES */
} smla_kv_format;

typedef struct smla_fwd_params {
  /* sizes */
  int32_t s_q;      /* query tokens, >= 0 */
  int32_t h_q;      /* query heads: 16, 32, 64 or 128 */
  int32_t d_qk;     /* must be SMLA_D_QK */
  int32_t d_v;      /* must be SMLA_D_V */
  int32_t topk;     /* slots per token, >= 1 */
  int64_t s_kv;     /* KV rows, 1 .. 2^31-1 */
  float sm_scale;   /* softmax scale applied to P; finite */

  /* Q: bf16 [s_q, h_q, d_qk]; rows 16-byte aligned */
  const void* q;
  int64_t q_stride_token, q_stride_head;

  /* KV: see smla_kv_format; rows 16-byte aligned */
  const void* kv;
  int64_t kv_stride_row;
  int32_t kv_format;

  /* indices: int32 [s_q, topk]; any token stride >= 0 */
  const int32_t* indices;
  int64_t indices_stride_token;

  /* out: bf16 [s_q, h_q, d_v] (written); rows 16-byte aligned */
  void* out;
  int64_t out_stride_token, out_stride_head;

  /* lse: float32 [s_q, h_q] (written), heads contiguous */
  float* lse;
  int64_t lse_stride_token;

  /* tuning: 0 lets the planner choose.
   *   num_splits: parts of each token's topk range, each run by its own
   *               workgroup and merged by log-sum-exp (decode occupancy).
   *   b_topk:     slots per block of the online softmax: 32, 64 or 128
   *               (bf16 KV), 32 (fp8 and fp4 KV).  With bf16 KV a split of
   *               at most 128 slots always runs as one block of 128 (all its
   *               rows resident at once), whatever b_topk says. */
  int32_t num_splits;
  int32_t b_topk;

  /* Work schedule (page "Flash Attention Infer算子性能优化", section
   * 优化多核负载均衡: with causal or sparse masks tokens carry different
   * numbers of valid blocks, so tokens are dealt to the cores by valid-block
   * weight, not by count).
   *   schedule: SMLA_SCHEDULE_AUTO (0) lets the planner choose (the grid:
   *             on prefill and causal prefill the hardware's own dispatch of
   *             one workgroup per token balances as well as the weighted
   *             runs, and pays no token-switch cost);
   *             SMLA_SCHEDULE_GRID (1): one workgroup per (token, split, group
   *             of 64 heads);
   *             SMLA_SCHEDULE_PERSISTENT (2): a fixed number of workgroups,
   *             each on a contiguous run of tokens of about equal weight
   *             (blocks up to the token's last valid slot, plus the cost of a
   *             token switch), with the pipeline running through token
   *             boundaries.  Built for bf16 KV within a 4 GB byte window,
   *             h_q = 64, one split and topk >= 1024; SMLA_ERR_UNSUPPORTED
   *             otherwise.
   *   persistent_workgroups: workgroups of the persistent schedule; 0 = one
   *             per compute unit of the device. */
  int32_t schedule;
  int32_t persistent_workgroups;

  /* Device scratch, needed when the plan has more than one split (fp32 lse
   * and bf16 normalised output of every part) or runs one split of the
   * pipelined 64-head kernel in a 4 GB byte window (int32 block count of
   * every token, computed ahead); size from smla_fwd_workspace_size.
   * Caller-owned; it may be reused by later calls on the same stream. */
  void* workspace;
  size_t workspace_bytes;
} smla_fwd_params;

/* The plan the library would run for these parameters (argument checks
 * included): number of splits and block size.  (Whether the persistent
 * schedule runs: smla_fwd_schedule.) */
smla_status smla_fwd_plan(const smla_fwd_params* p, int32_t* num_splits, int32_t* b_topk);

/* The schedule the library would run for these parameters: SMLA_SCHEDULE_GRID
 * or SMLA_SCHEDULE_PERSISTENT. */
smla_status smla_fwd_schedule(const smla_fwd_params* p, int32_t* schedule);

/* Bytes of device workspace smla_fwd needs for these parameters (0 when the
 * plan needs none). */
smla_status smla_fwd_workspace_size(const smla_fwd_params* p, size_t* bytes);

/* Enqueue the forward pass: writes out and lse.  Asynchronous on `stream`. */
smla_status smla_fwd(const smla_fwd_params* p, void* stream);

/* ---- Forward pass without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).
 *
 * smla_fwd with the split partials kept in a scratch array the library holds
 * in each device's memory (SMLA_STATIC_SCRATCH_BYTES, resident on a device
 * from the first call there until the process ends) instead of
 * p->workspace, which is ignored.  The call allocates nothing: no hipMalloc,
 * no hipFree.  A plan whose split partials need more than the scratch holds
 * (smla_fwd_workspace_size > SMLA_STATIC_SCRATCH_BYTES) returns
 * SMLA_ERR_WORKSPACE and enqueues nothing; so does a device the library
 * cannot reach (SMLA_ERR_HIP).  The scratch of a device belongs to the
 * device of `stream` (the current device for the NULL stream).
 *
 * Every call on one device shares that device's scratch.  Calls ordered on
 * one stream are safe; calls that may overlap in time on one device (other
 * streams, other host threads) race on it and give wrong results.  Each part
 * writes all of its partial results before the merge reads them, so nothing
 * from an earlier call is ever read. */
#define SMLA_STATIC_SCRATCH_BYTES (64u << 20)
smla_status smla_fwd_static_scratch(const smla_fwd_params* p, void* stream);

/* ---- Paged KV cache.
 *
 * Page "Flash Attention Infer算子性能优化" (catlass), section
 * 优化Paged Attention路径: the KV cache lives in fixed-size pages whose rows are
 * contiguous, and a block table names, in order, the physical page holding
 * each logical block of a sequence.  Here every query token has its own block
 * table row, and its indices name LOGICAL positions:
 *
 *   logical position j of token t  ->  physical KV row
 *       block_table[t][j / page_size] * page_size + j % page_size
 *
 * of the KV tensor described by smla_fwd_params (kv, kv_stride_row,
 * kv_format), whose s_kv is the physical row count num_pages * page_size.
 * A slot is masked (weight zero, row never read) when its position is outside
 * [0, table_width * page_size) or its block's table entry is outside
 * [0, num_pages) (for example -1 for an unallocated block).  Everything else
 * is smla_fwd: same outputs, plans, splits and formats. */
typedef struct smla_paged_kv {
  const int32_t* block_table;       /* DEVICE int32 [s_q, table_width], caller-owned */
  int64_t block_table_stride_token; /* elements between consecutive tokens' rows, >= 0 */
  int32_t table_width;              /* logical blocks per token, >= 1 */
  int32_t page_size;                /* KV rows per page, >= 1; s_kv % page_size == 0 */
} smla_paged_kv;

/* Bytes of device workspace smla_fwd_paged needs: the translated indices
 * (s_q * topk int32, rounded up to 256 bytes) followed by the split partials
 * smla_fwd_workspace_size reports for the same parameters.  Never 0 when
 * s_q > 0. */
smla_status smla_fwd_paged_workspace_size(const smla_fwd_params* p, const smla_paged_kv* paged,
                                          size_t* bytes);

/* Enqueue the forward pass over a paged KV cache: one pass translates every
 * token's logical indices to physical rows (into the workspace), then the
 * forward pass of smla_fwd runs on them.  p->indices holds logical positions;
 * p->workspace must hold smla_fwd_paged_workspace_size bytes (256-byte
 * aligned).  Validation and error behaviour as smla_fwd, plus the block table
 * (non-NULL when s_q > 0, 4-byte aligned) and the page geometry. */
smla_status smla_fwd_paged(const smla_fwd_params* p, const smla_paged_kv* paged, void* stream);

/* ---- Shape-dependent plan selection.
 *
 * Page "FlashMLA算子Ascend 950移植：从tiling到访存优化全解读", section 6
 * (后续优化方向, dynamic tiling): the best tile depends on the request's
 * shape, so prepared tiling configurations are chosen per shape at run time.
 * The planner's choice (num_splits = b_topk = 0) follows measured behaviour
 * on the named workloads; for other shapes a caller can time the candidate
 * plans on its own inputs once and pass the winner explicitly (the library
 * keeps no state).  Candidates: the planner's plan, then num_splits in
 * {1, 2, 3, 4, 6, 8, 12, 16, 24, 32} with b_topk 32 and 64 (bf16 KV) or 32
 * (fp8/fp4 KV), each valid distinct plan once. */

/* Bytes of workspace smla_fwd_tune needs: the largest over the candidates. */
smla_status smla_fwd_tune_workspace_size(const smla_fwd_params* p, size_t* bytes);

/* Run every candidate plan (one warm-up launch, then `iterations` timed
 * launches between two HIP events on `stream`) and return the fastest plan's
 * num_splits and b_topk and its time per launch in microseconds (may be
 * NULL).  The call BLOCKS until the timed work is done; it creates and
 * destroys two HIP events and allocates no device memory.  Writes out and
 * lse (the result of the last candidate, a correct forward pass) and uses
 * p->workspace (smla_fwd_tune_workspace_size bytes, 256-byte aligned).
 * iterations in [1, 1000].  p->num_splits and p->b_topk are ignored.  Flat
 * KV only (for a paged cache, tune on the translated layout). */
smla_status smla_fwd_tune(const smla_fwd_params* p, void* stream, int32_t iterations,
                          int32_t* num_splits, int32_t* b_topk, float* microseconds);

/* Host helper: pack E4M3 codes [rows, 576] and float32 scales [rows, 5]
 * (host memory, row-major, contiguous) into 640-byte fp8 KV rows at `packed`
 * (host memory, rows * 640 bytes, caller-owned).  Padding bytes are zeroed. */
smla_status smla_pack_fp8_kv_host(const uint8_t* codes, const float* scales, int64_t rows,
                                  void* packed);

/* Host helper: pack E2M1 codes [rows, 576] (one 4-bit code per byte, values
 * 0..15) and float32 scales [rows, 5] (host memory, row-major, contiguous)
 * into 320-byte fp4 KV rows at `packed` (host memory, rows * 320 bytes,
 * caller-owned).  A code above 15 is an invalid argument (nothing written
 * past the check).  Padding bytes are zeroed. */
smla_status smla_pack_fp4_kv_host(const uint8_t* codes, const float* scales, int64_t rows,
                                  void* packed);

/* Static text for a status code. */
const char* smla_status_string(int32_t status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* smla_last_error(void);

/* SMLA_ABI_VERSION of the loaded library. */
int32_t smla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H_ */
