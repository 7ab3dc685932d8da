// Software-pipelined forward kernel for 64 heads per workgroup, B_TOPK 32 and
// bf16 KV (prefill, causal and bf16 decode with h_q 64 or 128).
//
// Same method as the kernels in smla_fwd.cuh (page "Ascend Sparse Attention
// Forward 算法与优化技术简析", sections 数学建模 and 计算流程: gathered rows,
// P = Q·Gᵀ, block-wise online softmax with the skip-scale rule, S cast to bf16
// before S·V), scheduled differently:
//
//  * d_v split of the PV product.  Wave w computes the QKᵀ scores and the
//    softmax of its 16 heads, then publishes its block's bf16 S operand and
//    rescale factors through LDS; every wave multiplies the S of all 64 heads
//    with its own 128 columns of V.  A V fragment is thus read from LDS once
//    per workgroup and feeds four MFMAs (instead of every wave reading all of
//    V for its 16 heads), which cuts the LDS read traffic of a block by 35%.
//  * One barrier per block, and the block pipeline is skewed by one: in
//    iteration i a wave runs QKᵀ of block i+1 first (its MFMAs hide the LDS
//    latency of fetching the published S of block i), then the PV products of
//    block i with the softmax of block i+1 interleaved between its MFMAs.
//  * No index compaction in LDS (that room holds the S exchange): the row
//    indices of a block come five blocks ahead, by a direct-to-LDS load per
//    wave, into a ring of four small LDS slots, and are read and tested when
//    the block's gather is prepared two iterations later.  Memory wait counts
//    are in order, so the load is issued early enough that the wait for an
//    older gather already covers it; holding the indices in LDS (each slot
//    its own object) rather than in registers keeps the compiler from
//    placing waits of its own for them.
//    Invalid slots gather the split's first valid row and are masked through
//    a per-block array of score biases (0 or -inf, added in the same fma that
//    scales the score); blocks past the split's last valid slot are skipped.
//  * Every iteration issues the same memory instructions: the gathers of a
//    block past the split are dummies (buffer loads outside the KV window,
//    which the hardware drops; with 64-bit addresses, loads of the padding
//    row).  All wait counts are then compile-time constants, and the
//    compiler, whose own waits assume the fewest instructions any path could
//    have issued, never has to wait for more than the schedule does.
#pragma once

#include <climits>

#include "smla_fwd.cuh"

namespace smla {
namespace {

// Scan of one split's slots [lo, hi) by the whole workgroup: blocks up to the
// last valid slot, the first valid row (the padding row) and the valid count.
struct SplitScan {
  int nblk, pad_row, nvalid;
};

template <int BT, int NT>
__device__ SplitScan scan_split(const int32_t* __restrict__ irow, int lo, int hi, int64_t s_kv,
                                int* sred, int tid) {
  if (tid == 0) {
    sred[0] = -1;
    sred[1] = INT_MAX;
    sred[2] = 0;
  }
  // all loads first (a split holds at most kMaxSlotsPerSplit slots)
  constexpr int PER = kMaxSlotsPerSplit / NT;
  int v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = lo + k * NT + tid;
    v[k] = j < hi ? irow[j] : -1;
  }
  __syncthreads();
  int last = -1, first = INT_MAX, cnt = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = lo + k * NT + tid;
    if (v[k] >= 0 && (int64_t)v[k] < s_kv) {
      last = j;
      first = min(first, j);
      ++cnt;
    }
  }
  if (cnt) {
    atomicMax(&sred[0], last);
    atomicMin(&sred[1], first);
    atomicAdd(&sred[2], cnt);
  }
  __syncthreads();
  SplitScan s;
  s.nvalid = sred[2];
  s.nblk = s.nvalid ? (sred[0] - lo) / BT + 1 : 0;
  s.pad_row = s.nvalid ? irow[sred[1]] : 0;
  return s;
}

// Gather of one row block of one block: the lane's row (row 8w + lane%8 of the
// block, its 16-byte chunk lane/8 of each 128-byte line) and the nine
// direct-to-LDS instructions that fill units (k, w), k < 9, of the stage.
template <bool BUF>
struct RowGather {
  uint32_t voff;
  const char* base;
  // raw: the slot's index (or -1); exists: the block lies in the split (else
  // the loads are dummies).  An invalid slot loads the padding row, or with
  // DUMMY_INVALID (32-bit window only) nothing.  Returns whether the slot is
  // valid.
  template <bool DUMMY_INVALID = false>
  __device__ __forceinline__ bool prepare(const KvSource<BUF>& src, int64_t row_bytes, int raw,
                                          int pad_row, int64_t s_kv, int lane, bool exists) {
    const bool valid = raw >= 0 && (int64_t)raw < s_kv;
    const int row = valid ? raw : pad_row;
    const int c = lane >> 3;
    if constexpr (BUF)
      voff = exists && (!DUMMY_INVALID || valid) ? (uint32_t)row * (uint32_t)row_bytes + (uint32_t)(c << 4)
                                                 : kDummyOffset;
    else
      base = src.kv + (int64_t)row * row_bytes + (c << 4);
    return valid;
  }
  __device__ __forceinline__ void issue(const KvSource<BUF>& src, char* stage, int w, int k) const {
    src.load16((LDS_AS void*)(stage + (k * 4 + w) * 1024), voff, base, 128 * k);
  }
};

// Register state of a wave: the output tiles of all 64 heads for this wave's
// 128 columns, and the online-softmax state of its own 16 heads.
struct PipeState {
  f32x4 o[32];      // tile ht·8 + j = Oᵀ[dv 16(8w + j) + 4g + r][head 16ht + n]
  float running_max;
  float running_max_for_softmax;
  float sumexp;     // this lane's partial running_sumexp of head n (own tile)
};

// PRE: one split per token, 32-bit window, and a.token_blocks holds each
// token's block count: no scan of the index row, and the first gathers wait
// for the ring indices only (issued ahead of Q), not for Q or a scan.
template <bool SPLIT, bool BUF, bool PRE = false>
__global__ __launch_bounds__(256) void smla_fwd_bf16_pipe_kernel(FwdArgs a) {
  debug_poison_lds();
  static_assert(!PRE || (BUF && !SPLIT), "precomputed block counts: one split, 32-bit window");
  constexpr int NW = 4, BT = 32, KT = 2;
  constexpr int NQ = 36;                      // QK MFMAs per block
  constexpr int NPV = 32;                     // PV MFMAs per block (8 V fragments x 4 head tiles)
  constexpr int LPB = 9;                      // gather instructions per wave per block
  constexpr int TILE = BT * kRowBytesBf16;
  constexpr int UG = (BT / 8) * 1024;         // bytes between chunk groups of a stage
  constexpr int PF = 12;                      // K operand reads in flight
  constexpr int PFV = 4;                      // V fragments (two reads each) in flight
  constexpr int XS = NW * 64 * 16;            // published S operands of one block
  // Statically distinct LDS objects: the compiler tracks direct-to-LDS writes
  // per object, so reading one stage never waits for gathers into another.
  __shared__ __attribute__((aligned(1024))) char st0[TILE];
  __shared__ __attribute__((aligned(1024))) char st1[TILE];
  __shared__ __attribute__((aligned(1024))) char st2[TILE];
  __shared__ __attribute__((aligned(1024))) char st3[TILE];
  __shared__ __attribute__((aligned(16))) char xs0[XS];
  __shared__ __attribute__((aligned(16))) char xs1[XS];
  __shared__ __attribute__((aligned(16))) float xa0[NW * 16];
  __shared__ __attribute__((aligned(16))) float xa1[NW * 16];
  // index ring: slot r, lane l of wave w at [r][w·64 + l] holds the index of
  // its block's row 8w + l%8
  __shared__ __attribute__((aligned(16))) int ring[4][NW * 64];
  __shared__ __attribute__((aligned(16))) float vbias[4][BT];   // per stage: 0 (valid slot) or -inf
  __shared__ float lsh[NW * 16];
  __shared__ int sred[4];
  char* const stages[4] = {st0, st1, st2, st3};
  char* const xss[2] = {xs0, xs1};
  float* const xas[2] = {xa0, xa1};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int lo = wi.split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);
  const int32_t* __restrict__ irow = a.idx + (int64_t)wi.token * a.idx_st;
  const int head = wi.head0 + w * 16 + n;
  bf16x8 qf[18];
  SplitScan sc;
  if constexpr (PRE) {
    sc.nblk = __builtin_amdgcn_readfirstlane(a.token_blocks[wi.token]);   // >= 1
    sc.pad_row = 0;                           // unused: invalid slots load nothing
    sc.nvalid = 1;                            // an empty token shows as l = 0 instead
  } else {
    load_q(a, wi.token, head, g, qf);
    sc = scan_split<BT, NW * 64>(irow, lo, hi, a.s_kv, sred, tid);
  }
  const int nblk = sc.nblk;
  PipeState st;
#pragma unroll
  for (int t = 0; t < 32; ++t) st.o[t] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  st.running_max = kNegInf;
  st.running_max_for_softmax = kNegInf;
  st.sumexp = 0.f;
  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);
  const int wbase = 2 * UG * w;               // this wave's 128 dv columns: chunk groups 2w, 2w+1

  // Index of this lane's gather slot in block b (row 8w + lane%8) into ring
  // slot r: a buffer load over the split's index row, so slots past the split
  // read 0 without a memory access (they are tested against hi when used).
  // Issued in every iteration, so the wait counts below are exact.
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc((void*)irow, 0, hi * 4, 0x00020000);
  auto load_idx = [&](int b, auto R) __attribute__((always_inline)) {
    const int j = lo + b * BT + 8 * w + (lane & 7);
    debug_poison_dma<4>((LDS_AS void*)(&ring[decltype(R)::value][w * 64]));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, (LDS_AS void*)(&ring[decltype(R)::value][w * 64]), 4,
                                             (uint32_t)j * 4u, 0, 0, 0);
  };
  const char* const ring_lane = (const char*)&ring[0][w * 64 + (lane & 7)];
  auto read_idx = [&](auto R) __attribute__((always_inline)) {
    return lds_read_opaque<decltype(R)::value * NW * 64 * 4>(ring_lane);
  };
  // Prepare the gather of block b into stage s from the loaded index raw
  // (slots past the split are invalid), publishing the score biases.
  auto prepare_gather = [&](RowGather<BUF>& rg, int s, int b, int raw) __attribute__((always_inline)) {
    const int j = lo + b * BT + 8 * w + (lane & 7);
    const bool valid =
        rg.template prepare<PRE>(src, a.kv_row_bytes, j < hi ? raw : -1, sc.pad_row, a.s_kv, lane, b < nblk);
    if (lane < 8) vbias[s][8 * w + lane] = valid ? 0.f : kNegInf;   // lanes 0..7: rows 8w..8w+7
  };
  // biases of keys 16kt + 4g + r of stage s
  auto load_bias = [&](int s, f32x4 (&bias)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) bias[kt] = lds_load<f32x4>((const char*)&vbias[s][0], (16 * kt + 4 * g) * 4);
  };

  auto qk_off = [&](int i) __attribute__((always_inline)) {
    const int s = i / KT, kt = i % KT;
    return lofs.qk[s & 1] + (s >> 1) * UG + kt * 2048;
  };
  auto tr_off = [&](int jj) __attribute__((always_inline)) {
    return wbase + lofs.tr[jj & 3] + (jj >> 2) * UG;
  };
  auto tr_load = [&](const char* tile, int off) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)((LDS_AS char*)(LDS_AS void*)tile + off));
  };

  // ---- Pᵀ = G·Qᵀ of one block (bf16 MFMA 16x16x32; even and odd d_qk steps
  // accumulate separately).  hook(i) runs after MFMA i.
  auto qk = [&](const char* tile, f32x4 (&pacc)[2][KT], auto&& hook) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) pacc[c][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 abuf[PF];
    static_for<0, PF>([&](auto I) __attribute__((always_inline)) {
      abuf[decltype(I)::value] = lds_load<bf16x8>(tile, qk_off(decltype(I)::value));
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NQ>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      constexpr int s = i / KT, kt = i % KT;
      pacc[s & 1][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], qf[s], pacc[s & 1][kt], 0, 0, 0);
      if constexpr (i + PF < NQ) abuf[i % PF] = lds_load<bf16x8>(tile, qk_off(i + PF));
      hook(I);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- Online softmax of one block in steps (interleaved with PV MFMAs).
  // Lane (g, n) holds the scores of keys 16kt + 4g + r of head n.
  struct Soft {
    float x[KT][4];
    float cur, alpha;
    bool any;
    bf16x8 s;
  };
  auto soft_step = [&](auto K, Soft& sm, const f32x4 (&pacc)[2][KT], const f32x4 (&bias)[KT])
      __attribute__((always_inline)) {
    // no contraction across the steps: every schedule rounds the running
    // state the same way, wherever the compiler places the steps
#pragma clang fp contract(off)
    constexpr int k = decltype(K)::value;
    if constexpr (k == 0) {
      // scaled logits in log2 units; an invalid slot's bias of -inf masks it
      // (a valid slot's bias of 0 leaves the product as it is)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.x[kt][r] = __builtin_fmaf(pacc[0][kt][r] + pacc[1][kt][r], a.scale_log2, bias[kt][r]);
      float c = sm.x[0][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) c = fmaxf(c, sm.x[kt][r]);
      sm.cur = c;
    } else if constexpr (k == 1) {
      sm.cur = wave_max16x4(sm.cur);
    } else if constexpr (k == 2) {
      // skip scale: move running_max_for_softmax (and rescale) only when some
      // head of this wave has run more than RESCALE_THRES past it
      const float rmax = fmaxf(st.running_max, sm.cur);
      st.running_max = rmax;
      const bool trig = rmax - st.running_max_for_softmax > kRescaleThresLog2;
      sm.any = __ballot(trig) != 0ull;
      // While a head has seen no valid slot its accumulators and sum are still
      // zero, so its factor is 1 (not exp2(-inf) = 0): the first block never
      // takes the rescale branch.
      const float al = __builtin_amdgcn_exp2f(st.running_max_for_softmax - rmax);
      sm.alpha = sm.any && st.running_max_for_softmax != kNegInf ? al : 1.0f;
      st.running_max_for_softmax = sm.any ? rmax : st.running_max_for_softmax;
      st.sumexp *= sm.alpha;
    } else if constexpr (k == 3 || k == 4) {
      // exponentials: a masked slot weighs exp2(-inf) = 0.  While the running
      // max is still -inf every score of the head is -inf, so any finite
      // offset gives the same zeros (and -inf - -inf would be NaN).
      constexpr int kt = k - 3;
      const float m = st.running_max_for_softmax == kNegInf ? 0.f : st.running_max_for_softmax;
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.x[kt][r] = __builtin_amdgcn_exp2f(sm.x[kt][r] - m);
    } else if constexpr (k == 5) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.sumexp += sm.x[kt][r];
      union { uint32_t u[4]; bf16x8 v; } t;
      t.u[0] = pack2_bf16(sm.x[0][0], sm.x[0][1]);
      t.u[1] = pack2_bf16(sm.x[0][2], sm.x[0][3]);
      t.u[2] = pack2_bf16(sm.x[1][0], sm.x[1][1]);
      t.u[3] = pack2_bf16(sm.x[1][2], sm.x[1][3]);
      sm.s = t.v;
    }
  };
  constexpr int NSOFT = 6;
  // publish S operand and rescale factor of this wave's heads for block b
  auto publish = [&](const Soft& sm, int p) __attribute__((always_inline)) {
    *(LDS_AS bf16x8*)((LDS_AS char*)(LDS_AS void*)xss[p] + (w * 64 + lane) * 16) = sm.s;
    *(LDS_AS float*)((LDS_AS char*)(LDS_AS void*)xas[p] + (w * 16 + n) * 4) = sm.alpha;   // same in all g
  };

  // ---- prologue: row indices of blocks 0..3, gathers of blocks 0..2, then
  // the index of block 4.  Ring slot b % 4 holds the indices of block b from
  // its load until its gather is prepared.  (With PRE every token has a block.)
  if (PRE || nblk > 0) {
    static_for<0, 4>([&](auto B) __attribute__((always_inline)) { load_idx(decltype(B)::value, B); });
    if constexpr (PRE) {
      // Q after the ring indices: loads complete in order, so the gathers
      // below wait for the indices only while Q is still in flight
      load_q(a, wi.token, head, g, qf);
      wait_vm_lgkm0<18>();
    } else {
      wait_vm_lgkm0<0>();   // the ring reads below are opaque to the compiler's waits
    }
    static_for<0, 3>([&](auto B) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::value;
      RowGather<BUF> rg;
      prepare_gather(rg, b, b, read_idx(B));
#pragma unroll
      for (int k = 0; k < LPB; ++k) rg.issue(src, stages[b], w, k);
    });
    load_idx(4, std::integral_constant<int, 0>{});
    // block 0: QKᵀ and softmax, published for iteration 0
    wait_vm_lgkm0<2 * LPB + 1>();
    barrier_no_vm_drain();
    f32x4 pacc[2][KT];
    qk(st0, pacc, [&](auto) {});
    f32x4 bias[KT];
    load_bias(0, bias);
    Soft sm;
    static_for<0, NSOFT>([&](auto K) __attribute__((always_inline)) { soft_step(K, sm, pacc, bias); });
    publish(sm, 0);
  }

  // ---- iteration i: consume S(i); QKᵀ(i+1); PV(i) with softmax(i+1); refill
  // the stage of block i-1 with block i+3; load the row index of block i+5.
  // DYN: whether block i+1 exists is checked at run time.
  auto iteration = [&](auto S, int i, auto DYN_) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;     // stage of block i
    constexpr int p = s & 1;                  // exchange buffer of block i
    constexpr bool DYN = decltype(DYN_)::value;
    const bool next = DYN ? i + 1 < nblk : true;
    // Every wave: gather(i+1) landed and S(i) written.  Younger than
    // gather(i+1) (issued in iteration i-2, or in the prologue) are the memory
    // instructions of iteration i-1: an index load and the gathers of block
    // i+2 (for i = 0 the prologue's gathers of block 2 and index load of
    // block 4; for i = 1 that index load as well, which this count makes
    // iteration 1 wait for too: stricter, so also correct).
    wait_vm_lgkm0<LPB + 1>();
    barrier_no_vm_drain();

    // the indices of block i+5 go to the ring slot of block i+1 (prepared in
    // iteration i-2); block i+3's were loaded in iteration i-2
    load_idx(i + 5, std::integral_constant<int, (s + 1) & 3>{});
    RowGather<BUF> rg;
    prepare_gather(rg, (s + 3) & 3, i + 3, read_idx(std::integral_constant<int, (s + 3) & 3>{}));
    char* const rstage = stages[(s + 3) & 3];
    // the LPB gathers are spread over the iteration's last NG MFMAs (the
    // tail of QKᵀ and all of PV): gathers [ceil(c·LPB/NG), ceil((c+1)·LPB/NG))
    // follow MFMA kGatherFrom + c.  The QKᵀ operand reads of the head of the
    // iteration then see no direct-to-LDS write younger than the barrier's
    // wait, so the compiler places no wait before them.  Measured against
    // gathers in PV only and gathers from QKᵀ MFMA 18: within 0.5% on
    // prefill, 3.5% ahead of PV-only on causal prefill.
    auto dma_at = [&](auto C) __attribute__((always_inline)) {
      constexpr int kGatherFrom = 30, c = decltype(C)::value - kGatherFrom, NG = NQ + NPV - kGatherFrom;
      if constexpr (c >= 0)
        static_for<(c * LPB + NG - 1) / NG, ((c + 1) * LPB + NG - 1) / NG>([&](auto K) __attribute__((always_inline)) {
          rg.issue(src, rstage, w, decltype(K)::value);
        });
    };

    bf16x8 sop[NW];
    float alph[NW];
    f32x4 bias[KT];
    auto consume_reads = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ht = 0; ht < NW; ++ht) {
        sop[ht] = lds_load<bf16x8>(xss[p], (ht * 64 + lane) * 16);
        alph[ht] = lds_load<float>((const char*)xas[p], (ht * 16 + n) * 4);
      }
    };
    const char* const tile = stages[s];
    i16x4 va[PFV], vb[PFV];
    auto fetch_v = [&](int jj) __attribute__((always_inline)) {
      va[jj % PFV] = tr_load(tile, tr_off(jj));
      vb[jj % PFV] = tr_load(tile, tr_off(jj) + 2048);
    };

    f32x4 pacc[2][KT];
    if (next) {
      qk(stages[(s + 1) & 3], pacc, [&](auto I) __attribute__((always_inline)) {
        constexpr int q = decltype(I)::value;
        if constexpr (q == 0) consume_reads();
        // score biases of block i+1, shortly before its softmax needs them
        if constexpr (q == NQ - 4) load_bias((s + 1) & 3, bias);
        // first V fragments of PV(i), once few K reads remain in flight
        if constexpr (q >= NQ - PF && q < NQ - PF + 2 * PFV && (q - (NQ - PF)) % 2 == 0)
          fetch_v((q - (NQ - PF)) / 2);
        dma_at(I);
      });
    } else {
      consume_reads();
#pragma unroll
      for (int jj = 0; jj < PFV; ++jj) fetch_v(jj);
      // the gathers the QKᵀ MFMAs would have carried (both paths issue the same
      // memory instructions)
      static_for<0, NQ>([&](auto I) __attribute__((always_inline)) { dma_at(I); });
    }

    // rescale this wave's columns of the head tiles whose owner rescaled: one
    // rarely taken branch for all tiles, and inside it one per tile (a factor
    // of 1 leaves a tile as is; a rescale usually comes from one owner wave)
    if (__ballot(alph[0] != 1.0f || alph[1] != 1.0f || alph[2] != 1.0f || alph[3] != 1.0f) != 0ull) {
      static_for<0, NW>([&](auto H) __attribute__((always_inline)) {
        constexpr int ht = decltype(H)::value;
        if (__ballot(alph[ht] != 1.0f) != 0ull) {
          static_for<0, 8>([&](auto J) __attribute__((always_inline)) {
            constexpr int t = ht * 8 + decltype(J)::value;
            st.o[t] = pin_agpr(pin_agpr(st.o[t]) * alph[ht]);
          });
        }
      });
    }

    // ---- Oᵀ += Vᵀ·Sᵀ for this wave's columns: MFMA c uses V fragment c/4
    // (dv tile 8w + c/4) and the S of head tile c%4; the softmax of block i+1
    // runs between the MFMAs.
    Soft sm;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NPV>([&](auto I) __attribute__((always_inline)) {
      constexpr int c = decltype(I)::value;
      constexpr int jj = c / NW, ht = c % NW;
      union { i16x4 h[2]; bf16x8 v; } av;
      av.h[0] = va[jj % PFV];
      av.h[1] = vb[jj % PFV];
      st.o[ht * 8 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, sop[ht], st.o[ht * 8 + jj], 0, 0, 0);
      if constexpr (ht == NW - 1 && jj + PFV < 8) fetch_v(jj + PFV);
      if constexpr (c % 4 == 1 && c / 4 < NSOFT) {
        if (next) soft_step(std::integral_constant<int, c / 4>{}, sm, pacc, bias);
      }
      dma_at(std::integral_constant<int, NQ + c>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if (next) publish(sm, p ^ 1);
  };

  using T = std::integral_constant<bool, true>;
  using F = std::integral_constant<bool, false>;
  if (PRE || nblk > 0) {
    iteration(std::integral_constant<int, 0>{}, 0, T{});
    int i0 = 1;
    // steady state: every iteration has a next block
    for (; i0 + 4 < nblk; i0 += 4) {
      iteration(std::integral_constant<int, 1>{}, i0, F{});
      iteration(std::integral_constant<int, 2>{}, i0 + 1, F{});
      iteration(std::integral_constant<int, 3>{}, i0 + 2, F{});
      iteration(std::integral_constant<int, 0>{}, i0 + 3, F{});
    }
    // the last blocks (at most four), nested so that an iteration is only
    // reached from the one before it
    if (i0 < nblk) {
      iteration(std::integral_constant<int, 1>{}, i0, T{});
      if (i0 + 1 < nblk) {
        iteration(std::integral_constant<int, 2>{}, i0 + 1, T{});
        if (i0 + 2 < nblk) {
          iteration(std::integral_constant<int, 3>{}, i0 + 2, T{});
          if (i0 + 3 < nblk) iteration(std::integral_constant<int, 0>{}, i0 + 3, T{});
        }
      }
    }
    wait_vm_lgkm0<0>();   // dummy and index loads still in flight
  }

  // ---- epilogue: every head's running_sumexp from its owner wave; this wave
  // writes its 128 columns of all 64 heads.
  const float l = wave_sum16x4(st.sumexp);
  // no valid slot: every weight is 0 (with PRE an empty token ran one fully
  // masked block; otherwise its scan found nothing)
  const bool empty = PRE ? !(l > 0.f) : sc.nvalid == 0;
  const float lse = empty ? kNegInf : (st.running_max_for_softmax + __builtin_amdgcn_logf(l)) * kLn2;
  if (g == 0) {
    lsh[w * 16 + n] = l;
    if constexpr (!SPLIT)
      a.lse[(int64_t)wi.token * a.lse_st + head] = lse;
    else
      a.ws_lse[((int64_t)wi.token * a.num_splits + wi.split) * a.h_q + head] = lse;
  }
  __syncthreads();
  float inv[NW];
#pragma unroll
  for (int ht = 0; ht < NW; ++ht) {
    const float lh = lsh[ht * 16 + n];
    inv[ht] = (PRE ? !(lh > 0.f) : empty) ? 0.f : 1.0f / lh;
  }
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int ht = t / 8, dt = 8 * w + t % 8;
    const int hd = wi.head0 + ht * 16 + n;
    const f32x4 o = pin_agpr(st.o[t]) * inv[ht];
    i32x2 v;
    v[0] = (int)pack2_bf16(o[0], o[1]);
    v[1] = (int)pack2_bf16(o[2], o[3]);
    if constexpr (!SPLIT) {
      *(i32x2*)(a.out + (int64_t)wi.token * a.out_st + (int64_t)hd * a.out_sh + 16 * dt + 4 * g) = v;
    } else {
      const int64_t part = ((int64_t)wi.token * a.num_splits + wi.split) * a.h_q + hd;
      *(i32x2*)(a.ws_o + part * kDv + 16 * dt + 4 * g) = v;
    }
  }
}

}  // namespace
}  // namespace smla
