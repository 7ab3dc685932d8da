// Sparse MLA attention forward for AMD MI355X (gfx950, CDNA4).
//
// Method: page "Ascend Sparse Attention Forward 算法与优化技术简析".
//   Section 数学建模 (mathematical model): per query token, gather the KV rows
//   named by the token's indices, P = Q·Gᵀ, S = softmax(P·sm_scale),
//   out = S·G[:, :d_v].
//   Section 计算流程 (computation flow): walk the slots in blocks of B_TOPK,
//   keep running_max, running_max_for_softmax and running_sumexp in fp32,
//   rescale the output accumulator only when some row's running max exceeds
//   the max used for the exponentials by more than RESCALE_THRES = 6 ("skip
//   scale"), cast S to bf16 before the product with V.
//
// MI355X design (the page's Ascend Cube/Vector pipeline is prior art only):
//   * One workgroup per (query token, split of its topk range).  Each wave owns
//     16 query heads; h_q/16 waves per workgroup.
//   * Prologue: the split's indices are read once, invalid ones dropped and the
//     valid ones compacted in order into LDS (masked slots carry zero weight,
//     so dropping them is exact); only ceil(valid / B_TOPK) blocks run.
//   * Gather: 16-byte direct-to-LDS loads (global_load_lds_dwordx4), several
//     blocks in flight in a ring of statically distinct LDS stage buffers.
//     Rows are stored with a 16-byte-chunk XOR swizzle so that both operand
//     reads below are free of LDS bank conflicts.
//   * QKᵀ on MFMA 16x16x32 bf16 as Pᵀ = G·Qᵀ: the key tile is the A operand
//     read from LDS, Q stays in registers for the whole loop as the B operand.
//     The result puts one head per lane column and four keys per lane, so row
//     maxima are in-lane work plus two cross-lane steps.
//   * Skip-scale decision per wave (its 16 heads), a wave-uniform branch.
//   * PV as Oᵀ = Vᵀ·Sᵀ: S feeds the B operand straight from registers; the
//     transposed V operand comes from ds_read_b64_tr_b16 on the same LDS tile;
//     Oᵀ (fp32, 128 registers per lane) keeps the one-head-per-lane layout, so
//     a rescale is a per-lane scalar multiply.
//   * Decode: split-topk partials (normalised output + lse) merged by a
//     log-sum-exp combine kernel.
//
// This header holds the kernels as templates; the smla_fwd_*.hip units each
// instantiate a subset of the launch configurations (compiled in parallel).
#pragma once

#include "smla_common.cuh"

namespace smla {
namespace {

// Compact the valid slots of [lo, hi) of one token's index row into sidx,
// in order.  Returns the number of valid slots.  All threads participate.
template <int NW>
__device__ int compact_slots(const int32_t* __restrict__ irow, int lo, int hi, int64_t s_kv,
                             int* sidx, int* swcnt, int tid) {
  constexpr int NT = NW * 64;
  const int lane = tid & 63, w = tid >> 6;
  int nvalid = 0;
  for (int c0 = lo; c0 < hi; c0 += NT) {
    const int j = c0 + tid;
    int v = -1;
    if (j < hi) v = irow[j];
    const bool ok = (j < hi) && v >= 0 && (int64_t)v < s_kv;
    const uint64_t m = __ballot(ok);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) swcnt[w] = __popcll(m);
    __syncthreads();
    int base = nvalid, tot = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int cnt = swcnt[u];
      if (u < w) base += cnt;
      tot += cnt;
    }
    if (ok) sidx[base + pre] = v;
    nvalid += tot;
    __syncthreads();
  }
  return nvalid;
}

// Source of the gathers.  With BUF the whole KV lies in a 32-bit window:
// buffer loads (MUBUF) from one uniform resource, each lane adding its 32-bit
// row offset (the hardware also range-checks every access against the
// window).  Otherwise 64-bit global addresses (FLAT-encoded global loads).
// The buffer form is preferred: the compiler's wait-count tracking treats a
// FLAT direct-to-LDS load as a possible LDS access and then drains every
// pending LDS read (lgkmcnt(0)) after it, which breaks the operand prefetch
// of the products.
template <bool BUF>
struct KvSource {
  const char* kv;
  __amdgpu_buffer_rsrc_t rsrc;
  KvSource() = default;
  __device__ __forceinline__ KvSource(const char* p, uint32_t window) : kv(p) {
    if constexpr (BUF)
      // word 3 = 0x00020000: 32-bit data format, no swizzle, no index stride
      rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)window, 0x00020000);
  }
  // One 16-byte direct-to-LDS load of byte row_off + add (add: wave-uniform)
  // into lds + 16·lane.
  __device__ __forceinline__ void load16(LDS_AS void* lds, uint32_t voff, const char* vaddr,
                                         int add) const {
    debug_poison_dma(lds);
    if constexpr (BUF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, voff, add, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(vaddr + add), lds, 16, 0, 0);
  }
};

// Gather of one block (BT compacted slots) into an LDS stage.  Unit
// u = m·(BT/8) + rb is filled by one wave instruction; waves take units
// u = w, w + NW, ... so that each wave keeps a fixed set of row blocks.  Lane
// l fills slot l of the unit: row 8rb + l%8, chunk 8m + l/8; its
// address is one row base plus 128·m.  Padding slots past the valid count
// hold the token's first valid row: it is finite and the softmax gives those
// slots weight exactly 0.
//
// The instructions of one block are spread through the MFMA stream of the
// previous block (a burst of them back-pressures the issuing wave); GatherPlan
// holds the per-lane row bases, GatherPlan::issue(k) sends the k-th
// instruction of this wave.
template <int NW, int BT, bool BUF>
struct GatherPlan {
  static constexpr int R = BT / 8;                    // row blocks
  static constexpr int UNITS = 9 * R;                 // instructions per block
  static constexpr int PER_WAVE = (UNITS + NW - 1) / NW;
  static constexpr int NRB = NW >= R ? 1 : R / NW;    // row blocks per wave
  uint32_t voff[NRB];                                 // BUF: byte offsets in the window
  const char* base[NRB];                              // !BUF: addresses
  KvSource<BUF> src;
  char* stage;
  int w;

  __device__ __forceinline__ void prepare(char* stg, const KvSource<BUF>& src, int64_t row_bytes,
                                          const int* sidx_blk, int tid) {
    const int l = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    stage = stg;
    this->src = src;
#pragma unroll
    for (int j = 0; j < NRB; ++j) {
      const int rb = (w + j * NW) % R;
      const int c = l >> 3;
      const int row = sidx_blk[8 * rb + (l & 7)];
      if constexpr (BUF)
        voff[j] = (uint32_t)row * (uint32_t)row_bytes + (uint32_t)(c << 4);
      else
        base[j] = src.kv + (int64_t)row * row_bytes + (c << 4);
    }
  }

  // k-th instruction of this wave: unit u = k·NW + w.
  __device__ __forceinline__ void issue(int k) {
    const int u = k * NW + w;                          // wave-uniform
    if (UNITS % NW == 0 || u < UNITS) {
      const int m = u / R;
      const int j = NW >= R ? 0 : k % NRB;             // which of this wave's row blocks
      src.load16((LDS_AS void*)(stage + u * 1024), voff[j], base[j], 128 * m);
    }
  }
  __device__ __forceinline__ void issue_all() {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) issue(k);
  }
};

template <int NW, int BT>
constexpr int loads_per_block() {
  return GatherPlan<NW, BT, true>::PER_WAVE;
}

// Wait until at most `pend` later blocks' gathers are outstanding, plus all
// LDS traffic.  pend is in [0, NST-2].
template <int LPB, int NST>
__device__ __forceinline__ void wait_block(int pend) {
  if constexpr (NST > 3) {
    if (pend >= 2) { wait_vm_lgkm0<2 * LPB>(); return; }
  }
  if constexpr (NST > 2) {
    if (pend >= 1) { wait_vm_lgkm0<LPB>(); return; }
  }
  wait_vm_lgkm0<0>();
}

// Per-wave online-softmax state for 16 heads (one per lane column).
struct State {
  f32x4 o[32];      // Oᵀ[dv = 16·dt + 4·g + r][head n]
  float running_max;
  float running_max_for_softmax;
  float sumexp;     // this lane's partial running_sumexp (keys 4g..4g+3 of each tile)
};

// Per-lane LDS byte offsets of the two operand reads (see the stage layout).
// Every step of the unrolled loops adds a compile-time immediate to one of a
// few per-lane bases.
template <int BT>
struct LaneOffsets {
  int qk[2];   // K operand: row n (+16kt), chunk 4s + g; by s & 1
  int tr[4];   // V operand: rows 4g + i/4 (+32ks), chunk 2dt + ((i&3)>>1); by dt & 3
};

template <int BT>
__device__ __forceinline__ LaneOffsets<BT> lane_offsets(int lane) {
  const int g = lane >> 4, n = lane & 15;
  LaneOffsets<BT> o;
  // QK: row block 2kt + n/8, row-in-block n%8, chunk-in-group 4(s&1) + g
#pragma unroll
  for (int v = 0; v < 2; ++v)
    o.qk[v] = ((n >> 3) * 64 + unit_slot(4 * v + g, n & 7)) * 16;
  // V: row 4g + n/4 -> row block g/2 (+4ks), row-in-block 4(g&1) + n/4;
  //    chunk 2dt + ((n&3)>>1) -> group dt/4, chunk-in-group 2(dt&3) + ((n&3)>>1)
  const int rb = g >> 1, r8 = 4 * (g & 1) + (n >> 2);
#pragma unroll
  for (int v = 0; v < 4; ++v)
    o.tr[v] = (rb * 64 + unit_slot(2 * v + ((n & 3) >> 1), r8)) * 16 + (n & 1) * 8;
  return o;
}

// One block: QKᵀ, skip-scale online softmax, PV.  The LDS operands of both
// products are fetched ahead through small rotating register buffers
// (scheduling fences keep the order).  With REFILL the gather instructions of
// a later block are interleaved with the PV MFMAs; with SIDE the side work
// (the fp8 dequantisation of the next block) is interleaved with the QK MFMAs.
// No side work in the QK loop (bf16 KV).
struct NoSideWork {
  static constexpr int PER_THREAD = 0;
  __device__ __forceinline__ void run(int) {}
};

template <int NW, int BT, bool REFILL, bool SIDE, bool FP8, class Gather, class Side>
__device__ __forceinline__ void compute_block(const char* tile, const LaneOffsets<BT>& lo,
                                              const bf16x8 (&qf)[18], State& st,
                                              int blk, int nvalid, float scale_log2, int lane,
                                              Gather& next, Side& side,
                                              const float* stile = nullptr) {
  constexpr int KT = BT / 16;
  constexpr int UNIT_GROUP = (BT / 8) * 1024;   // bytes between chunk groups
  constexpr int NQ = 18 * KT;                   // QK MFMAs
  // K operand reads in flight (LDS latency under load is ~10 MFMAs; at most
  // 15 LDS operations can be outstanding per wave)
  constexpr int PF = FP8 ? 8 : 12;
  const int g = lane >> 4;

  // ---- Pᵀ = G·Qᵀ over d_qk = 576 = 18 steps of 32.  MFMA i: step s = i / KT,
  // key tile kt = i % KT.  bf16 KV: even and odd steps accumulate separately so
  // that 2·KT independent chains are in flight.  fp8 KV: the tile holds the
  // E4M3 codes (exact in bf16) and each 128-column scale group accumulates on
  // its own; the per-row group scales are applied below in fp32.
  auto qk_off = [&](int i) __attribute__((always_inline)) {
    const int s = i / KT, kt = i % KT;
    return lo.qk[s & 1] + (s >> 1) * UNIT_GROUP + kt * 2048;
  };
  // Gather instructions of the refill: spread evenly over the MFMAs of both
  // products (bf16) or of the PV product (fp8, whose QK loop carries the
  // dequantisation): gathers [ceil(c·NDMA/N), ceil((c+1)·NDMA/N)) follow MFMA
  // c of the N that carry them.  Issuing them in a burst stalls the wave on a
  // full vector-memory queue.
  constexpr int NDMA = Gather::PER_WAVE;
  constexpr int NPVT = 32 * (BT / 32);          // PV MFMAs
  constexpr int NQD = SIDE ? 0 : NQ;            // QK MFMAs that carry gathers
  constexpr int NDT = NQD + NPVT;
  auto refill_at = [&](auto C) __attribute__((always_inline)) {
    constexpr int c = decltype(C)::value;
    if constexpr (REFILL)
      static_for<(c * NDMA + NDT - 1) / NDT, ((c + 1) * NDMA + NDT - 1) / NDT>(
          [&](auto K) __attribute__((always_inline)) { next.issue(decltype(K)::value); });
  };
  constexpr int NACC = FP8 ? 5 : 2;
  auto acc_of = [](int s) constexpr { return FP8 ? s / 4 : (s & 1); };
  f32x4 pacc[NACC][KT];
#pragma unroll
  for (int c = 0; c < NACC; ++c)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) pacc[c][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 abuf[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) abuf[i] = lds_load<bf16x8>(tile, qk_off(i));
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, NQ>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    constexpr int s = i / KT, kt = i % KT;
    pacc[acc_of(s)][kt] =
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], qf[s], pacc[acc_of(s)][kt], 0, 0, 0);
    if constexpr (i + PF < NQ) abuf[i % PF] = lds_load<bf16x8>(tile, qk_off(i + PF));
    if constexpr (!SIDE) refill_at(I);
    if constexpr (SIDE) {
      // side tasks [ceil(i·NS/NQ), ceil((i+1)·NS/NQ)) go after MFMA i
      constexpr int NS = Side::PER_THREAD;
      static_for<(i * NS + NQ - 1) / NQ, ((i + 1) * NS + NQ - 1) / NQ>(
          [&](auto K) __attribute__((always_inline)) { side.run(decltype(K)::value); });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  f32x4 p[KT];
  // fp8: group scales of this lane's keys 16kt + 4g + r, from the block's
  // group-major scale tile [5][BT]
  float ksc[KT][4][5];
  if constexpr (FP8) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        const f32x4 a4 = lds_load<f32x4>((const char*)stile, (c * BT + 16 * kt + 4 * g) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) ksc[kt][r][c] = a4[r];
      }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
#pragma unroll
        for (int c = 0; c < 5; ++c) v = fmaf(ksc[kt][r][c], pacc[c][kt][r], v);
        p[kt][r] = v;
      }
  } else {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) p[kt] = pacc[0][kt] + pacc[1][kt];
  }

  // ---- scaled logits in log2 units; slots past the compacted count are masked
  float x[KT][4];
  float cur = kNegInf;
  const int j0 = blk * BT + 4 * g;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = p[kt][r] * scale_log2;
      x[kt][r] = (j0 + 16 * kt + r < nvalid) ? v : kNegInf;
      cur = fmaxf(cur, x[kt][r]);
    }
  }
  cur = wave_max16x4(cur);
  // Every block holds at least one valid slot, so the new running max is finite.
  const float rmax = fmaxf(st.running_max, cur);
  st.running_max = rmax;
  const bool trig = rmax - st.running_max_for_softmax > kRescaleThresLog2;
  if (__ballot(trig) != 0ull) {
    // On the first block (running_max_for_softmax still -inf in every lane,
    // as every block holds a valid slot) the accumulators and sums are zero
    // and stay zero: only the max moves.
    if (st.running_max_for_softmax != kNegInf) {
      const float alpha = __builtin_amdgcn_exp2f(st.running_max_for_softmax - rmax);
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        // The accumulators live in AGPRs (MFMA C/D); pinning the rescaled values
        // back there keeps the register allocator from moving all 128 of them to
        // VGPRs around the loop for this rarely taken branch.
        st.o[dt] = pin_agpr(pin_agpr(st.o[dt]) * alpha);
      }
      st.sumexp *= alpha;
    }
    st.running_max_for_softmax = rmax;
  }
  const float m = st.running_max_for_softmax;
  float sv[KT][4];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[kt][r] = __builtin_amdgcn_exp2f(x[kt][r] - m);
      st.sumexp += sv[kt][r];
    }
  }

  // ---- Oᵀ += Vᵀ·Sᵀ, 32 keys per MFMA step.  Lane (g, n) holds S for head n
  // and keys {32ks + 4g + e, 32ks + 16 + 4g + e}, e < 4; the transposed reads
  // give the V operand the same key order.
  constexpr int KS = BT / 32;                   // key steps of 32
  // S as the bf16 B operand; fp8 KV: one operand per 128-column V group with
  // that row's group scale folded in, so that the V operand stays the exact code.
  constexpr int NSB = FP8 ? 4 : 1;
  bf16x8 sb[NSB][KS];
#pragma unroll
  for (int gv = 0; gv < NSB; ++gv) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float w[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          w[h][r] = FP8 ? sv[2 * ks + h][r] * ksc[2 * ks + h][r][gv] : sv[2 * ks + h][r];
      union { uint32_t u[4]; bf16x8 v; } t;
      t.u[0] = pack2_bf16(w[0][0], w[0][1]);
      t.u[1] = pack2_bf16(w[0][2], w[0][3]);
      t.u[2] = pack2_bf16(w[1][0], w[1][1]);
      t.u[3] = pack2_bf16(w[1][2], w[1][3]);
      sb[gv][ks] = t.v;
    }
  }
  auto tr_load = [&](int off) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS i16x4*)((LDS_AS char*)(LDS_AS void*)tile + off));
  };
  // Every wave multiplies its own 16 heads with the whole V tile.
  // MFMA i: ks = i / 32, dv tile dt = i % 32.
  constexpr int NPV = 32 * KS;
  constexpr int PFV = 6;                      // V fragments (2 reads each) in flight
  auto tr_off = [&](int i) __attribute__((always_inline)) {
    const int ks = i / 32, dt = i % 32;
    return lo.tr[dt & 3] + (dt >> 2) * UNIT_GROUP + ks * 4096;
  };
  i16x4 va[PFV], vb[PFV];
#pragma unroll
  for (int i = 0; i < PFV; ++i) {
    va[i] = tr_load(tr_off(i));
    vb[i] = tr_load(tr_off(i) + 2048);
  }
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, NPV>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    union { i16x4 h[2]; bf16x8 v; } a;
    a.h[0] = va[i % PFV];
    a.h[1] = vb[i % PFV];
    constexpr int dt = i % 32;
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, sb[FP8 ? dt / 8 : 0][i / 32], st.o[dt], 0, 0, 0);
    if constexpr (i + PFV < NPV) {
      va[i % PFV] = tr_load(tr_off(i + PFV));
      vb[i % PFV] = tr_load(tr_off(i + PFV) + 2048);
    }
    refill_at(std::integral_constant<int, NQD + decltype(I)::value>{});
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Work item of this workgroup: (token, split of its slots, group of 64 heads).
// With several head groups (h_q = 128) the groups of one item get workgroup
// ids 8 apart: ids are dealt round-robin to the 8 XCDs, so both land on the
// same XCD at nearly the same time and the second gather of the item's rows
// mostly hits that XCD's L2.  Returns false for padding workgroups.
struct WorkItem {
  int token, split, head0;
};
__device__ __forceinline__ bool work_item(const FwdArgs& a, WorkItem& wi) {
  // The workgroups of one token (head groups x splits) share the token's Q
  // and, across head groups, its gathered rows.  Workgroup b runs on XCD b % 8
  // (the dispatcher deals workgroups to the XCDs in turn), so a token's
  // workgroups take consecutive rounds b / 8 on one XCD: the later ones find
  // Q and the rows in that XCD's L2.  (A placement hint only: correctness
  // does not depend on it.)
  const int per = a.head_groups * a.num_splits;
  const int b = blockIdx.x, r = b >> 3;
  const int group = r / per, local = r - group * per;
  const int token = group * 8 + (b & 7);
  if (token >= a.s_q) return false;
  wi.token = token;
  wi.split = local % a.num_splits;
  wi.head0 = (local / a.num_splits) * 64;
  return true;
}

// Load Q for this wave's 16 heads: B operand of Pᵀ = G·Qᵀ, lane (g, n) holds
// Q[head n][32s + 8g .. 32s + 8g + 7].
__device__ __forceinline__ void load_q(const FwdArgs& a, int token, int head, int g, bf16x8 (&qf)[18]) {
  const uint16_t* qrow = a.q + (int64_t)token * a.q_st + (int64_t)head * a.q_sh + 8 * g;
#pragma unroll
  for (int s = 0; s < 18; ++s) qf[s] = *(const bf16x8*)(qrow + 32 * s);
}

__device__ __forceinline__ void init_state(State& st) {
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) st.o[dt] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  st.running_max = kNegInf;
  st.running_max_for_softmax = kNegInf;
  st.sumexp = 0.f;
}

// Epilogue: total running_sumexp per head, normalise, write the output (or
// the split partial: normalised output, rounded to bf16, and lse of this part).
template <bool SPLIT>
__device__ __forceinline__ void write_output(const FwdArgs& a, State& st, int token, int split,
                                             int head, int g, int nvalid) {
  const float l = wave_sum16x4(st.sumexp);
  const bool empty = nvalid == 0;
  const float inv = empty ? 0.f : 1.0f / l;
  const float lse = empty ? kNegInf : (st.running_max_for_softmax + __builtin_amdgcn_logf(l)) * kLn2;
  if constexpr (!SPLIT) {
    uint16_t* orow = a.out + (int64_t)token * a.out_st + (int64_t)head * a.out_sh + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const f32x4 o = pin_agpr(st.o[dt]);
      i32x2 v;
      v[0] = (int)pack2_bf16(o[0] * inv, o[1] * inv);
      v[1] = (int)pack2_bf16(o[2] * inv, o[3] * inv);
      *(i32x2*)(orow + 16 * dt) = v;
    }
    if (g == 0) a.lse[(int64_t)token * a.lse_st + head] = lse;
  } else {
    const int64_t part = ((int64_t)token * a.num_splits + split) * a.h_q + head;
    uint16_t* orow = a.ws_o + part * kDv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const f32x4 o = pin_agpr(st.o[dt]);
      i32x2 v;
      v[0] = (int)pack2_bf16(o[0] * inv, o[1] * inv);
      v[1] = (int)pack2_bf16(o[2] * inv, o[3] * inv);
      *(i32x2*)(orow + 16 * dt) = v;
    }
    if (g == 0) a.ws_lse[part] = lse;
  }
}

// Compaction of index values already loaded (C per thread: slot
// lo + c·NT + tid, -1 past the split), as compact_slots.
template <int NW, int C>
__device__ int compact_values(const int (&v)[C], int64_t s_kv, int* sidx, int* swcnt, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  int nvalid = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool ok = v[c] >= 0 && (int64_t)v[c] < s_kv;
    const uint64_t m = __ballot(ok);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) swcnt[w] = __popcll(m);
    __syncthreads();
    int base = nvalid, tot = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int cnt = swcnt[u];
      if (u < w) base += cnt;
      tot += cnt;
    }
    if (ok) sidx[base + pre] = v[c];
    nvalid += tot;
    __syncthreads();
  }
  return nvalid;
}

// Output row of a head (the output, or the split partial) and its lse slot.
template <bool SPLIT>
__device__ __forceinline__ uint16_t* out_row(const FwdArgs& a, int token, int split, int head, float*& lse) {
  if constexpr (!SPLIT) {
    lse = a.lse + (int64_t)token * a.lse_st + head;
    return a.out + (int64_t)token * a.out_st + (int64_t)head * a.out_sh;
  } else {
    const int64_t part = ((int64_t)token * a.num_splits + split) * a.h_q + head;
    lse = a.ws_lse + part;
    return a.ws_o + part * kDv;
  }
}

// Short splits (at most 128 slots: decode with the topk range cut into
// parts) as ONE block of B_TOPK = 128 (page "Ascend Sparse Attention Forward
// 算法与优化技术简析", section 计算流程: the block loop of the online softmax
// with a single block, so running_max_for_softmax is the block's max and no
// rescale can occur).  The 128 rows fill four 32-row stages of LDS at once.
//   * The split's indices are loaded first, then Q: compaction waits only
//     for the indices.  Every slot past the valid count repeats the first
//     valid row (finite, weight 0), so all four stages hold real rows.
//   * QKᵀ runs stage by stage, each stage after its own rows have arrived;
//     the logits of all 128 slots stay in registers, then one softmax pass.
//   * With NG = 2 (h_q = 128) a wave owns 16 heads of each 64-head group:
//     every K and V operand read from LDS feeds the MFMAs of both groups,
//     which halves the LDS operand traffic (the products' bound with one
//     wave per SIMD).  Both groups' Q (registers) are live in QKᵀ only, both
//     output accumulators (AGPRs) in PV only.
template <int NW, bool SPLIT, bool BUF, int NG>
__global__ __launch_bounds__(NW * 64) void smla_fwd_bf16_short_kernel(FwdArgs a) {
  debug_poison_lds();
  constexpr int BT = 32, NST = 4, MAXS = BT * NST;
  constexpr int LPB = loads_per_block<NW, BT>();
  constexpr int TILE = BT * kRowBytesBf16;
  constexpr int NT = NW * 64;
  constexpr int C = (MAXS + NT - 1) / NT;
  constexpr int KT = MAXS / 16;                 // key tiles of 16 slots
  constexpr int UNIT_GROUP = (BT / 8) * 1024;   // bytes between chunk groups of a stage
  __shared__ __attribute__((aligned(1024))) char st0[TILE];
  __shared__ __attribute__((aligned(1024))) char st1[TILE];
  __shared__ __attribute__((aligned(1024))) char st2[TILE];
  __shared__ __attribute__((aligned(1024))) char st3[TILE];
  __shared__ int sidx[MAXS];
  __shared__ int swcnt[NW];
  char* const stages[4] = {st0, st1, st2, st3};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int token = wi.token, split = wi.split;
  const int lo = split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);

  const int32_t* irow = a.idx + (int64_t)token * a.idx_st;
  int v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = lo + c * NT + tid;
    v[c] = j < hi ? irow[j] : -1;
  }
  const int head = wi.head0 + w * 16 + n;
  const int nvalid = compact_values<NW, C>(v, a.s_kv, sidx, swcnt, tid);

  if (nvalid == 0) {
    // no valid slot: out = 0, lse = −∞ (every group)
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
      float* lse;
      uint16_t* row = out_row<SPLIT>(a, token, split, head + 64 * gr, lse);
#pragma unroll
      for (int k = 0; k < 16; ++k) *(i32x4*)(row + 32 * k + 8 * g) = i32x4{0, 0, 0, 0};
      if (g == 0) *lse = kNegInf;
    }
    return;
  }
  for (int j = nvalid + tid; j < MAXS; j += NT) sidx[j] = sidx[0];
  __syncthreads();

  // Stage 0's gathers, then Q, then stages 1..3 (loads complete in issue
  // order, so the wait for stage b covers Q from b = 0 on).  Q is not loaded
  // before the indices: the whole chip issues these bursts at once, and Q
  // traffic ahead of the index loads delays every workgroup's indices.
  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);
  bf16x8 q0[18], q1[18];
  static_for<0, NST>([&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    GatherPlan<NW, BT, BUF> gp;
    gp.prepare(stages[b], src, a.kv_row_bytes, sidx + b * BT, tid);
    gp.issue_all();
    if constexpr (b == 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      load_q(a, token, head, g, q0);
      if constexpr (NG == 2) load_q(a, token, head + 64, g, q1);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  });

  // ---- Pᵀ = G·Qᵀ, stage by stage.  Key tile 2b + kt of stage b; even and
  // odd steps of a stage accumulate separately (more independent chains).
  constexpr int PF = 12;                        // K operand reads in flight
  f32x4 p[NG][KT];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) p[gr][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto qk_off = [&](int i) __attribute__((always_inline)) {
    const int s = i / 2, kt = i % 2;
    return lofs.qk[s & 1] + (s >> 1) * UNIT_GROUP + kt * 2048;
  };
  static_for<0, NST>([&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const char* tile = stages[b];
    wait_vm_lgkm0<(NST - 1 - b) * LPB>();
    barrier_no_vm_drain();
    f32x4 odd[NG][2];
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) odd[gr][0] = odd[gr][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 abuf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) abuf[i] = lds_load<bf16x8>(tile, qk_off(i));
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 36>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, s = i / 2, kt = i % 2;
      if constexpr (s % 2 == 0) {
        p[0][2 * b + kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], q0[s], p[0][2 * b + kt], 0, 0, 0);
        if constexpr (NG == 2)
          p[1][2 * b + kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], q1[s], p[1][2 * b + kt], 0, 0, 0);
      } else {
        odd[0][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], q0[s], odd[0][kt], 0, 0, 0);
        if constexpr (NG == 2)
          odd[1][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], q1[s], odd[1][kt], 0, 0, 0);
      }
      if constexpr (i + PF < 36) abuf[i % PF] = lds_load<bf16x8>(tile, qk_off(i + PF));
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int gr = 0; gr < NG; ++gr)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) p[gr][2 * b + kt] += odd[gr][kt];
  });

  // ---- softmax over the block: scaled logits in log2 units, slots past the
  // valid count masked; running_max_for_softmax = the block's max (finite:
  // slot 0 is valid), S = exp2(x - max), running_sumexp = Σ S (fp32, before
  // the bf16 cast of S).
  bf16x8 sb[NG][NST];
  float msoft[NG], lsum[NG];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    float x[KT][4];
    float cur = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float val = p[gr][kt][r] * a.scale_log2;
        x[kt][r] = (16 * kt + 4 * g + r < nvalid) ? val : kNegInf;
        cur = fmaxf(cur, x[kt][r]);
      }
    const float m = wave_max16x4(cur);
    float sum = 0.f;
    float sv[KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[kt][r] = __builtin_amdgcn_exp2f(x[kt][r] - m);
        sum += sv[kt][r];
      }
    msoft[gr] = m;
    lsum[gr] = wave_sum16x4(sum);
    // B operand of key step b (stage b): keys 32b + 4g + e and 32b + 16 + 4g + e
#pragma unroll
    for (int b = 0; b < NST; ++b) {
      union { uint32_t u[4]; bf16x8 v; } t;
      t.u[0] = pack2_bf16(sv[2 * b][0], sv[2 * b][1]);
      t.u[1] = pack2_bf16(sv[2 * b][2], sv[2 * b][3]);
      t.u[2] = pack2_bf16(sv[2 * b + 1][0], sv[2 * b + 1][1]);
      t.u[3] = pack2_bf16(sv[2 * b + 1][2], sv[2 * b + 1][3]);
      sb[gr][b] = t.v;
    }
  }

  // ---- Oᵀ = Vᵀ·Sᵀ in chunks of four d_v tiles: a chunk accumulates over the
  // four stages (key steps), then its tiles are final: normalised, packed and
  // stored while the next chunks' products run, so the output stores are
  // spread over PV instead of one burst at the end.  Each V fragment feeds
  // both groups.
  float* lsep[NG];
  uint16_t* rowp[NG];
  float inv[NG];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    rowp[gr] = out_row<SPLIT>(a, token, split, head + 64 * gr, lsep[gr]);
    rowp[gr] += (g & 1) ? 16 + 4 * (g - 1) : 4 * g;
    inv[gr] = 1.0f / lsum[gr];
    if (g == 0) *lsep[gr] = (msoft[gr] + __builtin_amdgcn_logf(lsum[gr])) * kLn2;
  }
  constexpr int PFV = 6;                        // V fragments (two reads each) in flight
  auto tr_load = [&](int b, int off) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS i16x4*)((LDS_AS char*)(LDS_AS void*)stages[b] + off));
  };
  // fragment f: chunk f / 16, stage (f / 4) % 4, tile dt = 4·chunk + f % 4
  auto frag_off = [&](int f) __attribute__((always_inline)) {
    const int dt = 4 * (f / 16) + f % 4;
    return lofs.tr[dt & 3] + (dt >> 2) * UNIT_GROUP;
  };
  i16x4 va[PFV], vb[PFV];
  static_for<0, PFV>([&](auto F) __attribute__((always_inline)) {
    constexpr int f = decltype(F)::value;
    va[f] = tr_load((f / 4) % 4, frag_off(f));
    vb[f] = tr_load((f / 4) % 4, frag_off(f) + 2048);
  });
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, 8>([&](auto Q) __attribute__((always_inline)) {
    constexpr int ch = decltype(Q)::value;
    f32x4 o[NG][4];
#pragma unroll
    for (int gr = 0; gr < NG; ++gr)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[gr][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, 16>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, f = 16 * ch + i, b = i / 4, j = i % 4;
      union { i16x4 h[2]; bf16x8 v; } av;
      av.h[0] = va[f % PFV];
      av.h[1] = vb[f % PFV];
      o[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, sb[0][b], o[0][j], 0, 0, 0);
      if constexpr (NG == 2)
        o[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, sb[1][b], o[1][j], 0, 0, 0);
      if constexpr (f + PFV < 128) {
        va[f % PFV] = tr_load(((f + PFV) / 4) % 4, frag_off(f + PFV));
        vb[f % PFV] = tr_load(((f + PFV) / 4) % 4, frag_off(f + PFV) + 2048);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // tiles 4ch .. 4ch+3 are final: pairs (4ch, 4ch+1) and (4ch+2, 4ch+3)
    // give stores 2ch and 2ch+1 (16 bytes per lane, 64 contiguous bytes per
    // head: rows 0<->1 and 2<->3 of the pair swapped)
#pragma unroll
    for (int gr = 0; gr < NG; ++gr)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x4 oe = o[gr][2 * k], oo = o[gr][2 * k + 1];
        const float iv = inv[gr];
        const uint32_t e0 = pack2_bf16(oe[0] * iv, oe[1] * iv), e1 = pack2_bf16(oe[2] * iv, oe[3] * iv);
        const uint32_t o0 = pack2_bf16(oo[0] * iv, oo[1] * iv), o1 = pack2_bf16(oo[2] * iv, oo[3] * iv);
        const auto s0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
        *(i32x4*)(rowp[gr] + 32 * (2 * ch + k)) = i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// B_TOPK = 128 over a split of any length (page "Ascend Sparse Attention
// Forward 算法与优化技术简析", section 计算流程 step 1 names 64 or 96 slots per
// block; its section 讨论 argues for larger blocks when the per-block vector
// work dominates): the block loop of the online softmax with blocks of 128
// slots, one block resident in LDS as four 32-row stages.  QKᵀ runs stage by
// stage as the rows arrive; one softmax step per 128 slots (running_max,
// skip-scale rescale at RESCALE_THRES, running_sumexp); PV stage by stage,
// and once every wave is done with a stage it is refilled with the next
// block's rows (a barrier per stage), so the next block's gathers overlap the
// rest of this block's PV.  One wave per 16 heads (h_q/16 waves, at most 64
// heads per workgroup).
template <int NW, bool SPLIT, bool BUF>
__global__ __launch_bounds__(NW * 64) void smla_fwd_bf16_b128_kernel(FwdArgs a) {
  debug_poison_lds();
  constexpr int BT = 32, NST = 4, BB = BT * NST;
  constexpr int LPB = loads_per_block<NW, BT>();
  constexpr int TILE = BT * kRowBytesBf16;
  constexpr int NT = NW * 64;
  constexpr int KT = BB / 16;                   // key tiles of 16 slots per block
  constexpr int UNIT_GROUP = (BT / 8) * 1024;
  __shared__ __attribute__((aligned(1024))) char st0[TILE];
  __shared__ __attribute__((aligned(1024))) char st1[TILE];
  __shared__ __attribute__((aligned(1024))) char st2[TILE];
  __shared__ __attribute__((aligned(1024))) char st3[TILE];
  __shared__ int sidx[kMaxSlotsPerSplit + BB];
  __shared__ int swcnt[NW];
  char* const stages[4] = {st0, st1, st2, st3};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int token = wi.token, split = wi.split;
  const int lo = split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);
  const int head = wi.head0 + w * 16 + n;
  const int nvalid = compact_slots<NW>(a.idx + (int64_t)token * a.idx_st, lo, hi, a.s_kv, sidx, swcnt, tid);
  float* lsep;
  uint16_t* row = out_row<SPLIT>(a, token, split, head, lsep);
  if (nvalid == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) *(i32x4*)(row + 32 * k + 8 * g) = i32x4{0, 0, 0, 0};
    if (g == 0) *lsep = kNegInf;
    return;
  }
  const int nblk = (nvalid + BB - 1) / BB;
  // padding slots of the last block repeat the first valid row (weight 0)
  for (int j = nvalid + tid; j < nblk * BB; j += NT) sidx[j] = sidx[0];
  __syncthreads();

  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);
  bf16x8 qf[18];
  // block 0: stage 0's gathers, Q, stages 1..3 (loads complete in order)
  static_for<0, NST>([&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    GatherPlan<NW, BT, BUF> gp;
    gp.prepare(stages[b], src, a.kv_row_bytes, sidx + b * BT, tid);
    gp.issue_all();
    if constexpr (b == 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      load_q(a, token, head, g, qf);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  });

  f32x4 o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  float running_max = kNegInf, running_max_for_softmax = kNegInf, sumexp = 0.f;
  constexpr int PF = 12;
  auto qk_off = [&](int i) __attribute__((always_inline)) {
    const int s = i / 2, kt = i % 2;
    return lofs.qk[s & 1] + (s >> 1) * UNIT_GROUP + kt * 2048;
  };
  auto tr_load = [&](const char* tile, int off) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS i16x4*)((LDS_AS char*)(LDS_AS void*)tile + off));
  };
  auto tr_off = [&](int dt) __attribute__((always_inline)) {
    return lofs.tr[dt & 3] + (dt >> 2) * UNIT_GROUP;
  };

  for (int j = 0; j < nblk; ++j) {
    // ---- Pᵀ = G·Qᵀ stage by stage (stage b: key tiles 2b, 2b+1)
    f32x4 p[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) p[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, NST>([&](auto B) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::value;
      const char* tile = stages[b];
      wait_vm_lgkm0<(NST - 1 - b) * LPB>();
      barrier_no_vm_drain();
      f32x4 odd[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 abuf[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) abuf[i] = lds_load<bf16x8>(tile, qk_off(i));
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, 36>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value, s = i / 2, kt = i % 2;
        if constexpr (s % 2 == 0)
          p[2 * b + kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], qf[s], p[2 * b + kt], 0, 0, 0);
        else
          odd[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[i % PF], qf[s], odd[kt], 0, 0, 0);
        if constexpr (i + PF < 36) abuf[i % PF] = lds_load<bf16x8>(tile, qk_off(i + PF));
        __builtin_amdgcn_sched_barrier(0);
      });
      p[2 * b] += odd[0];
      p[2 * b + 1] += odd[1];
    });

    // ---- online softmax step over the block's 128 slots
    float x[KT][4];
    float cur = kNegInf;
    const int j0 = j * BB + 4 * g;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float val = p[kt][r] * a.scale_log2;
        x[kt][r] = (j0 + 16 * kt + r < nvalid) ? val : kNegInf;
        cur = fmaxf(cur, x[kt][r]);
      }
    cur = wave_max16x4(cur);
    // every block holds a valid slot, so the new running max is finite
    const float rmax = fmaxf(running_max, cur);
    running_max = rmax;
    if (__ballot(rmax - running_max_for_softmax > kRescaleThresLog2) != 0ull) {
      if (running_max_for_softmax != kNegInf) {
        const float alpha = __builtin_amdgcn_exp2f(running_max_for_softmax - rmax);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) o[dt] = pin_agpr(pin_agpr(o[dt]) * alpha);
        sumexp *= alpha;
      }
      running_max_for_softmax = rmax;
    }
    const float m = running_max_for_softmax;
    bf16x8 sb[NST];
#pragma unroll
    for (int b = 0; b < NST; ++b) {
      float sv[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[h][r] = __builtin_amdgcn_exp2f(x[2 * b + h][r] - m);
          sumexp += sv[h][r];
        }
      union { uint32_t u[4]; bf16x8 v; } t;
      t.u[0] = pack2_bf16(sv[0][0], sv[0][1]);
      t.u[1] = pack2_bf16(sv[0][2], sv[0][3]);
      t.u[2] = pack2_bf16(sv[1][0], sv[1][1]);
      t.u[3] = pack2_bf16(sv[1][2], sv[1][3]);
      sb[b] = t.v;
    }

    // ---- Oᵀ += Vᵀ·Sᵀ stage by stage; a stage is refilled with block j+1
    // once every wave is past its products
    const bool more = j + 1 < nblk;
    static_for<0, NST>([&](auto B) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::value;
      const char* tile = stages[b];
      constexpr int PFV = 6;
      i16x4 va[PFV], vb[PFV];
#pragma unroll
      for (int i = 0; i < PFV; ++i) {
        va[i] = tr_load(tile, tr_off(i));
        vb[i] = tr_load(tile, tr_off(i) + 2048);
      }
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, 32>([&](auto I) __attribute__((always_inline)) {
        constexpr int dt = decltype(I)::value;
        union { i16x4 h[2]; bf16x8 v; } av;
        av.h[0] = va[dt % PFV];
        av.h[1] = vb[dt % PFV];
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, sb[b], o[dt], 0, 0, 0);
        if constexpr (dt + PFV < 32) {
          va[dt % PFV] = tr_load(tile, tr_off(dt + PFV));
          vb[dt % PFV] = tr_load(tile, tr_off(dt + PFV) + 2048);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (more) {
        // every wave's reads of this stage have returned (its last products
        // consumed them) before the barrier; then the refill may land
        wait_vm_lgkm0<63>();
        barrier_no_vm_drain();
        GatherPlan<NW, BT, BUF> gp;
        gp.prepare(stages[b], src, a.kv_row_bytes, sidx + (j + 1) * BB + b * BT, tid);
        gp.issue_all();
      }
    });
  }

  // ---- epilogue: O / running_sumexp, 16-byte stores (rows 0<->1, 2<->3 of
  // each tile pair swapped: 64 contiguous bytes per head)
  const float l = wave_sum16x4(sumexp);
  const float inv = 1.0f / l;
  if (g == 0) *lsep = (running_max_for_softmax + __builtin_amdgcn_logf(l)) * kLn2;
  uint16_t* base = row + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const f32x4 oe = pin_agpr(o[2 * k]), oo = pin_agpr(o[2 * k + 1]);
    const uint32_t e0 = pack2_bf16(oe[0] * inv, oe[1] * inv), e1 = pack2_bf16(oe[2] * inv, oe[3] * inv);
    const uint32_t o0 = pack2_bf16(oo[0] * inv, oo[1] * inv), o1 = pack2_bf16(oo[2] * inv, oo[3] * inv);
    const auto s0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
    *(i32x4*)(base + 32 * k) = i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
  }
}

template <int NW, int BT, int NST, bool SPLIT, bool BUF>
__global__ __launch_bounds__(NW * 64) void smla_fwd_bf16_kernel(FwdArgs a) {
  debug_poison_lds();
  constexpr int LPB = loads_per_block<NW, BT>();
  constexpr int TILE = BT * kRowBytesBf16;
  // Statically distinct stage buffers: the compiler tracks direct-to-LDS
  // writes per LDS object, so reading one stage never waits for the gathers
  // still in flight into the others.
  __shared__ __attribute__((aligned(1024))) char st0[TILE];
  __shared__ __attribute__((aligned(1024))) char st1[TILE];
  __shared__ __attribute__((aligned(16))) char st2[NST > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(16))) char st3[NST > 3 ? TILE : 16];
  __shared__ int sidx[kMaxSlotsPerSplit + BT];
  __shared__ int swcnt[NW];
  char* const stages[4] = {st0, st1, st2, st3};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int token = wi.token, split = wi.split;
  const int lo = split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);

  // Q first: its loads are in flight while the indices are compacted.
  const int head = wi.head0 + w * 16 + n;
  bf16x8 qf[18];
  load_q(a, token, head, g, qf);
  const int nvalid = compact_slots<NW>(a.idx + (int64_t)token * a.idx_st, lo, hi, a.s_kv, sidx,
                                       swcnt, tid);
  const int nblk = (nvalid + BT - 1) / BT;
  // Padding slots of the last block repeat the first valid row (weight 0).
  for (int j = nvalid + tid; j < nblk * BT; j += NW * 64) sidx[j] = sidx[0];
  __syncthreads();

  State st;
  init_state(st);

  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  NoSideWork nside;
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);

  // Prologue: NST-1 blocks in flight.
#pragma unroll
  for (int b = 0; b < NST - 1; ++b) {
    if (b < nblk) {
      GatherPlan<NW, BT, BUF> gp;
      gp.prepare(stages[b], src, a.kv_row_bytes, sidx + b * BT, tid);
      gp.issue_all();
    }
  }

  // Steady state: every block i refills the stage freed by block i-1 with
  // block i+NST-1 (the refill is interleaved with block i's PV products).
  // Groups of NST blocks keep every stage index a compile-time constant.
  int i0 = 0;
  for (; i0 + 2 * NST - 2 < nblk; i0 += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int i = i0 + s;
      wait_block<LPB, NST>(NST - 2);
      barrier_no_vm_drain();
      GatherPlan<NW, BT, BUF> gp;
      gp.prepare(stages[(s + NST - 1) % NST], src, a.kv_row_bytes, sidx + (i + NST - 1) * BT, tid);
      compute_block<NW, BT, true, false, false>(stages[s], lofs, qf, st, i, nvalid, a.scale_log2, lane, gp, nside);
    }
  }
  // Tail: the last blocks, refilling while blocks remain.
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int i = i0 + s;
    if (i < nblk) {
      wait_block<LPB, NST>(min(nblk - 1, i + NST - 2) - i);
      barrier_no_vm_drain();
      GatherPlan<NW, BT, BUF> gp;
      if (i + NST - 1 < nblk) {
        gp.prepare(stages[(s + NST - 1) % NST], src, a.kv_row_bytes, sidx + (i + NST - 1) * BT, tid);
        compute_block<NW, BT, true, false, false>(stages[s], lofs, qf, st, i, nvalid, a.scale_log2, lane, gp, nside);
      } else {
        compute_block<NW, BT, false, false, false>(stages[s], lofs, qf, st, i, nvalid, a.scale_log2, lane, gp, nside);
      }
    }
  }
  // The tail loop runs at most NST blocks: i0 + 2·NST - 2 >= nblk there.
  for (i0 += NST; i0 < nblk; i0 += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int i = i0 + s;
      if (i < nblk) {
        wait_block<LPB, NST>(min(nblk - 1, i + NST - 2) - i);
        barrier_no_vm_drain();
        GatherPlan<NW, BT, BUF> gp;
        compute_block<NW, BT, false, false, false>(stages[s], lofs, qf, st, i, nvalid, a.scale_log2, lane, gp, nside);
      }
    }
  }

  // Further head groups over the same blocks (inner_groups > 1 only when the
  // split has at most NST blocks: each sits in stage i, complete and visible
  // since its wait and barrier above, and no refill overwrote it).  The next
  // group's Q loads are issued before this group's output stores.
  for (int hg = 1; hg < a.inner_groups; ++hg) {
    const int prev = head + (hg - 1) * 64;
    load_q(a, token, head + hg * 64, g, qf);
    write_output<SPLIT>(a, st, token, split, prev, g, nvalid);
    init_state(st);
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      if (s < nblk) {
        GatherPlan<NW, BT, BUF> gp;
        compute_block<NW, BT, false, false, false>(stages[s], lofs, qf, st, s, nvalid, a.scale_log2, lane, gp, nside);
      }
    }
  }
  write_output<SPLIT>(a, st, token, split, head + (a.inner_groups - 1) * 64, g, nvalid);
}

// ---------------------------------------------------------------------------
// Quantised KV caches: a packed row holds a token's 576 codes followed by five
// float32 scales (one per 128 columns) and padding, data next to scale as the
// page's section "Decoding KV Cache Layout 优化" recommends, so one gather
// brings both.  Two code formats:
//   fp8: OCP E4M3, one code per byte, 640-byte rows;
//   fp4: OCP E2M1, two codes per byte (column 2k in the low nibble of byte k,
//        column 2k+1 in the high nibble), 320-byte rows (the pages name an FP4
//        KV cache for decode beside the FP8 one).
// Raw rows land in an LDS ring by direct-to-LDS loads; the workgroup converts
// the codes of block i+1 to bf16 (exactly: every E4M3 and every E2M1 value is
// a bf16 value) in the stage layout above while computing block i, so the
// MFMA code is shared, and folds the scales in fp32 (dequantisation without
// any rounding of K or V).
struct KvFp8Format {
  static constexpr int ROW = kFp8RowBytes;        // 640
  static constexpr int CODE_BYTES = kDqk;         // 576
  static constexpr int MAX_SLOTS = kMaxSlotsPerSplitFp8;
  // 16 codes of row r, columns 16cc .. 16cc+15 -> eight packed bf16 pairs
  __device__ __forceinline__ static void convert16(const char* raw, int r, int cc, uint32_t (&o)[8]) {
    const i32x4 codes = lds_load<i32x4>(raw, r * ROW + cc * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // two codes -> two exact fp32 values -> two exact bf16 values
      const auto f = (j & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(codes[j >> 1], true)
                             : __builtin_amdgcn_cvt_pk_f32_fp8(codes[j >> 1], false);
      o[j] = pack2_bf16(f[0], f[1]);
    }
  }
};
struct KvFp4Format {
  static constexpr int ROW = kFp4RowBytes;        // 320
  static constexpr int CODE_BYTES = kDqk / 2;     // 288
  static constexpr int MAX_SLOTS = kMaxSlotsPerSplit;
  __device__ __forceinline__ static void convert16(const char* raw, int r, int cc, uint32_t (&o)[8]) {
    const i32x2 codes = lds_load<i32x2>(raw, r * ROW + cc * 8);
    static_for<0, 8>([&](auto J) __attribute__((always_inline)) {
      // byte j%4 of word j/4: columns 2j (low nibble) and 2j+1 (high nibble),
      // converted with scale 1 (exact)
      constexpr int j = decltype(J)::value;
      const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)codes[j >> 2], 1.0f, j & 3);
      o[j] = __builtin_bit_cast(uint32_t, b);
    });
  }
};

// Gather of one block of packed rows into a raw LDS slot, row-major; wave
// instruction k fills 64 consecutive 16-byte chunks (whole lines of several
// rows).  When the block's units do not divide evenly among the waves, a wave
// past the last unit repeats its own previous unit (the same bytes to the
// same LDS slot), so that every wave issues PER_WAVE instructions per block:
// the waits count them.
// SWZ: chunk c of row r sits at chunk c ^ swizzle(r) of the row's LDS span
// (raw_swizzle below), so that reads of one chunk of eight consecutive rows
// fall on distinct LDS banks; each row stays contiguous, so every instruction
// still loads the same global bytes as without it.
template <class Fmt>
__device__ __forceinline__ int raw_swizzle(int row) {
  // fp8: 640-byte rows, two rows apart share a bank offset -> XOR (r/2)%4;
  // fp4: 320-byte rows, four rows apart do -> XOR (r/4)%2
  return Fmt::ROW == 640 ? (row >> 1) & 3 : (row >> 2) & 1;
}
template <int NW, bool BUF, class Fmt, bool SWZ = false>
struct RawGather {
  static constexpr int BT = 32;
  static constexpr int CHUNKS = Fmt::ROW / 16;                 // 16-byte chunks per row
  static constexpr int UNITS = BT * CHUNKS / 64;              // fp8 20, fp4 10 instructions per block
  static_assert(BT * CHUNKS % 64 == 0, "whole units per block");
  static constexpr int PER_WAVE = (UNITS + NW - 1) / NW;
  static constexpr bool EARLY = false;
  KvSource<BUF> src;
  int64_t row_bytes;
  const int* sidx_blk;
  char* slot;
  int tid;
  bool dummy = false;   // a block past the split: the same instructions, nothing useful loaded

  __device__ __forceinline__ void prepare(char* raw, const KvSource<BUF>& s, int64_t rb,
                                          const int* sb, int t) {
    slot = raw;
    src = s;
    row_bytes = rb;
    sidx_blk = sb;
    tid = t;
  }
  // Loads past the end of the split: buffer loads at the out-of-window offset
  // (dropped by the range check), 64-bit loads of row 0 (inside the KV).
  __device__ __forceinline__ void prepare_dummy(char* raw, const KvSource<BUF>& s, int t) {
    slot = raw;
    src = s;
    row_bytes = 0;
    sidx_blk = nullptr;
    tid = t;
    dummy = true;
  }
  __device__ __forceinline__ void issue(int k) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    int u = k * NW + w;                                    // wave-uniform
    if (UNITS % NW != 0 && u >= UNITS) u -= NW;            // repeat this wave's previous unit
    const int c = u * 64 + l;
    const int row = c / CHUNKS, pc = c - row * CHUNKS;
    const int ch = SWZ ? pc ^ raw_swizzle<Fmt>(row) : pc;
    const int kvrow = dummy ? 0 : sidx_blk[row];
    if constexpr (BUF)
      src.load16((LDS_AS void*)(slot + u * 1024),
                 dummy ? kDummyOffset : (uint32_t)kvrow * (uint32_t)row_bytes + (ch << 4), nullptr, 0);
    else
      src.load16((LDS_AS void*)(slot + u * 1024), 0, src.kv + (int64_t)kvrow * row_bytes + (ch << 4), 0);
  }
  __device__ __forceinline__ void issue_all() {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) issue(k);
  }
};

// Conversion of one raw block into a bf16 stage: task c converts 16 codes of
// row c/36 (columns 16·(c%36) .. +15).  The stage holds the codes without
// rounding; the row's group scales are applied in fp32 by the block
// computation (to the QK partial sums of each group, and to S for each V
// group).  The scales are copied to a separate small tile: once converted,
// the raw slot may be refilled by any wave while others still compute on the
// block.
template <int NW, class Fmt>
struct DequantRaw {
  static constexpr int BT = 32;
  static constexpr int TASKS = BT * (kDqk / 16);            // 1152
  static constexpr int NT = NW * 64;
  static constexpr int PER_THREAD = (TASKS + NT - 1) / NT;
  const char* raw;
  char* tile;
  float* stile;   // [5][BT] group-major copy of the block's scales
  int tid;

  __device__ __forceinline__ void run(int k, int t) {
    // Threads past the last task redo it: the same bytes written twice.
    const int c = min(k * NT + t, TASKS - 1);
    const int r = c / 36, cc = c - r * 36;
    // every task also copies one scale of its row (groups repeat: same value)
    const int gs = cc % 5;
    *(LDS_AS float*)((LDS_AS char*)(LDS_AS void*)stile + (gs * BT + r) * 4) =
        lds_load<float>(raw, r * Fmt::ROW + Fmt::CODE_BYTES + gs * 4);
    uint32_t o[8];
    Fmt::convert16(raw, r, cc, o);
    // bf16 chunks 2cc and 2cc+1 of row r in the unit layout
    const int rb = r >> 3, r8 = r & 7;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 2 * cc + h;
      const int off = ((ch >> 3) * (BT / 8) + rb) * 1024 + unit_slot(ch & 7, r8) * 16;
      *(LDS_AS i32x4*)((LDS_AS char*)(LDS_AS void*)tile + off) =
          i32x4{(int)o[4 * h], (int)o[4 * h + 1], (int)o[4 * h + 2], (int)o[4 * h + 3]};
    }
  }
  // Task k's addresses depend only on the thread and k, so left visible the
  // compiler hoists every task's addresses out of the block loop; with one
  // or two waves (18 or 9 tasks per thread) they no longer fit in registers.
  // An opaque copy of the thread index keeps them local to each pass.
  __device__ __forceinline__ int opaque_tid() const {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  }
  __device__ __forceinline__ void run(int k) { run(k, opaque_tid()); }
  __device__ __forceinline__ void run_all() {
    const int t = opaque_tid();
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) run(k, t);
  }
};

template <int NW, bool SPLIT, bool BUF, class Fmt = KvFp8Format>
__global__ __launch_bounds__(NW * 64) void smla_fwd_fp8_kernel(FwdArgs a) {
  debug_poison_lds();
  constexpr int BT = 32;
  constexpr int NSTR = 4;                                  // raw ring depth
  constexpr int LPB = RawGather<NW, BUF, Fmt>::PER_WAVE;
  constexpr int RAW = BT * Fmt::ROW;
  constexpr int TILE = BT * kRowBytesBf16;
  __shared__ __attribute__((aligned(1024))) char rw0[RAW];
  __shared__ __attribute__((aligned(1024))) char rw1[RAW];
  __shared__ __attribute__((aligned(1024))) char rw2[RAW];
  __shared__ __attribute__((aligned(1024))) char rw3[RAW];
  __shared__ __attribute__((aligned(1024))) char tl0[TILE];
  __shared__ __attribute__((aligned(1024))) char tl1[TILE];
  __shared__ __attribute__((aligned(16))) float sc0[5 * BT];
  __shared__ __attribute__((aligned(16))) float sc1[5 * BT];
  __shared__ int sidx[Fmt::MAX_SLOTS + BT];
  __shared__ int swcnt[NW];
  char* const raws[4] = {rw0, rw1, rw2, rw3};
  char* const tiles[2] = {tl0, tl1};
  float* const stiles[2] = {sc0, sc1};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int token = wi.token, split = wi.split;
  const int lo = split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);

  const int head = wi.head0 + w * 16 + n;
  bf16x8 qf[18];
  load_q(a, token, head, g, qf);
  const int nvalid = compact_slots<NW>(a.idx + (int64_t)token * a.idx_st, lo, hi, a.s_kv, sidx,
                                       swcnt, tid);
  const int nblk = (nvalid + BT - 1) / BT;
  for (int j = nvalid + tid; j < nblk * BT; j += NW * 64) sidx[j] = sidx[0];
  __syncthreads();

  State st;
  init_state(st);
  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);

  // Prologue: raw blocks 0..NSTR-1 in flight, block 0 dequantised.
#pragma unroll
  for (int b = 0; b < NSTR; ++b) {
    if (b < nblk) {
      RawGather<NW, BUF, Fmt> rg;
      rg.prepare(raws[b], src, a.kv_row_bytes, sidx + b * BT, tid);
      rg.issue_all();
    }
  }
  if (nblk > 0) {
    wait_block<LPB, NSTR>(min(nblk - 1, NSTR - 1));
    barrier_no_vm_drain();
    DequantRaw<NW, Fmt> dq{raws[0], tiles[0], stiles[0], tid};
    dq.run_all();
  }

  // Block i: wait for raw block i+1, then (after the barrier) refill the raw
  // slot of block i with block i+NSTR during the PV products and dequantise
  // block i+1 into the other bf16 tile during the QK products.
  // (always inlined: the state captured by reference must stay in registers)
  auto step = [&](auto S, int i, auto REFILL, auto DEQ) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    if constexpr (decltype(DEQ)::value)
      wait_block<LPB, NSTR>(min(nblk - 1, i + NSTR - 1) - (i + 1));
    else
      wait_block<LPB, NSTR>(0);
    barrier_no_vm_drain();
    RawGather<NW, BUF, Fmt> rg;
    if constexpr (decltype(REFILL)::value)
      rg.prepare(raws[s], src, a.kv_row_bytes, sidx + (i + NSTR) * BT, tid);
    DequantRaw<NW, Fmt> dq{raws[(s + 1) % NSTR], tiles[(s + 1) & 1], stiles[(s + 1) & 1], tid};
    compute_block<NW, BT, decltype(REFILL)::value, decltype(DEQ)::value, true>(
        tiles[s & 1], lofs, qf, st, i, nvalid, a.scale_log2, lane, rg, dq, stiles[s & 1]);
  };
  using T = std::integral_constant<bool, true>;
  using F = std::integral_constant<bool, false>;
  int i0 = 0;
  for (; i0 + 2 * NSTR - 1 < nblk; i0 += NSTR) {
    step(std::integral_constant<int, 0>{}, i0 + 0, T{}, T{});
    step(std::integral_constant<int, 1>{}, i0 + 1, T{}, T{});
    step(std::integral_constant<int, 2>{}, i0 + 2, T{}, T{});
    step(std::integral_constant<int, 3>{}, i0 + 3, T{}, T{});
  }
  for (; i0 < nblk; i0 += NSTR) {
    auto tail = [&](auto S) __attribute__((always_inline)) {
      const int i = i0 + decltype(S)::value;
      if (i >= nblk) return;
      if (i + NSTR < nblk) step(S, i, T{}, T{});
      else if (i + 1 < nblk) step(S, i, F{}, T{});
      else step(S, i, F{}, F{});
    };
    tail(std::integral_constant<int, 0>{});
    tail(std::integral_constant<int, 1>{});
    tail(std::integral_constant<int, 2>{});
    tail(std::integral_constant<int, 3>{});
  }

  write_output<SPLIT>(a, st, token, split, head, g, nvalid);
}

unsigned grid_size(const FwdArgs& a) {
  return (unsigned)(((int64_t)a.s_q + 7) / 8 * 8 * a.head_groups * a.num_splits);
}

// Short split (at most kShortSlots slots): one block of up to 128 slots, two
// head groups per wave when inner_groups is 2.
template <int NW, bool SPLIT, bool BUF>
void launch_bf16_short(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid(grid_size(a)), block(NW * 64);
  if constexpr (NW == 4) {
    if (a.inner_groups == 2) {
      hipLaunchKernelGGL((smla_fwd_bf16_short_kernel<NW, SPLIT, BUF, 2>), grid, block, 0, stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((smla_fwd_bf16_short_kernel<NW, SPLIT, BUF, 1>), grid, block, 0, stream, a);
}

template <int NW, int BT, bool SPLIT, bool BUF>
void launch_bf16_variant(const FwdArgs& a, hipStream_t stream) {
  constexpr int NST = BT == 32 ? 4 : 2;
  if (a.slots_per_split <= kShortSlots)
    launch_bf16_short<NW, SPLIT, BUF>(a, stream);
  else
    hipLaunchKernelGGL((smla_fwd_bf16_kernel<NW, BT, NST, SPLIT, BUF>), dim3(grid_size(a)), dim3(NW * 64), 0,
                       stream, a);
}

template <int NW, bool SPLIT, bool BUF, class Fmt = KvFp8Format>
void launch_fp8_variant(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((smla_fwd_fp8_kernel<NW, SPLIT, BUF, Fmt>), dim3(grid_size(a)), dim3(NW * 64), 0,
                     stream, a);
}

}  // namespace

}  // namespace smla
