// Software-pipelined forward kernel for an fp8 (E4M3) KV cache, 64 heads per
// workgroup, B_TOPK 32 (fp8 decode with h_q 64 or 128).
//
// Method as in smla_fwd.cuh (page "Ascend Sparse Attention Forward
// 算法与优化技术简析", sections 数学建模 and 计算流程); the KV rows are the
// packed fp8 rows of section "Decoding KV Cache Layout 优化" (576 E4M3 codes,
// five float32 scales, one per 128 columns, padding to 640 bytes).
// Dequantisation is exact: every E4M3 value is a bf16 value, so the codes feed
// the bf16 MFMAs unchanged and the scales are applied in fp32 (QKᵀ: one
// accumulator per 128-column group, combined with the row's scales; PV: the
// row's scale of the V group is folded into the bf16 S operand).
//
// Schedule as in smla_fwd_pipe.cuh (d_v split of PV, one barrier per block,
// QKᵀ of block i+1 before PV of block i, softmax of block i+1 between the PV
// MFMAs), with these differences:
//  * The stages hold the raw 640-byte rows (20 KB per block), so six fit:
//    four blocks are in flight while two are in use.
//  * No dequantisation pass: the MFMA operands are converted from the codes in
//    registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact).  A K read is
//    16 codes (two MFMA steps: the d_qk order inside each 64-column window is
//    permuted, and Q is loaded in the same order); a V fragment is one
//    transposed byte read (ds_read_b64_tr_b8) of 8 codes.
//  * Each wave's 128 d_v columns are exactly one scale group, so the published
//    S operands are per V group: bf16(S · scale_group(row)).
#pragma once

#include "smla_fwd_pipe.cuh"

namespace smla {
namespace {

// 16 E4M3 codes -> two bf16 MFMA operands (codes 0..7, 8..15), exact.
__device__ __forceinline__ void fp8x16_to_bf16(const i32x4 c, bf16x8& lo, bf16x8& hi) {
  union { bf16x2 p[4]; bf16x8 v; } a, b;
  a.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], 1.0f, false);
  a.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], 1.0f, true);
  a.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], 1.0f, false);
  a.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], 1.0f, true);
  b.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[2], 1.0f, false);
  b.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[2], 1.0f, true);
  b.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[3], 1.0f, false);
  b.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[3], 1.0f, true);
  lo = a.v;
  hi = b.v;
}

// 8 E4M3 codes -> one bf16 MFMA operand, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(const i32x2 c) {
  union { bf16x2 p[4]; bf16x8 v; } a;
  a.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], 1.0f, false);
  a.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], 1.0f, true);
  a.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], 1.0f, false);
  a.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], 1.0f, true);
  return a.v;
}

// Raw stage layout: 1 KB units of 8 rows x 8 16-byte chunks, chunk-major
// (slot = (c%8)·8 + r%8); unit (m, rb) -- chunk group m = c/8 (0..4), row
// block rb = r/8 -- at (4m + gray(rb))·1 KB.  The Gray order puts the row
// blocks a K read pairs (rb 2kt, 2kt+1) and those a V read pairs (rb, rb+2)
// on opposite halves of the LDS bank row (address bit 10).
__device__ __forceinline__ constexpr int fp8_unit(int m, int rb) {
  return 4 * m + (rb ^ (rb >> 1));
}

template <bool SPLIT, bool BUF, int NST>
__global__ __launch_bounds__(256) void smla_fwd_fp8_pipe_kernel(FwdArgs a) {
  constexpr int NW = 4, BT = 32, KT = 2;
  constexpr int NP = 9;                       // 64-column windows of d_qk (pairs of MFMA steps)
  constexpr int NQ = NP * 2 * KT;             // QK MFMAs per block
  constexpr int NPV = 32;                     // PV MFMAs per block
  constexpr int LPB = 5;                      // gather instructions per wave per block
  static_assert(NST % 2 == 0 && NST >= 4 && NST <= 6, "an even number of raw stages, 4..6");
  constexpr int RAW = BT * kFp8RowBytes;      // 20 KB
  constexpr int PF = 4;                       // K reads (16 codes each) in flight
  constexpr int PFV = 4;                      // V fragments in flight
  constexpr int XS = NW * NW * 64 * 16;       // S operands of one block: [V group][head tile][lane]
  __shared__ __attribute__((aligned(1024))) char st0[RAW];
  __shared__ __attribute__((aligned(1024))) char st1[RAW];
  __shared__ __attribute__((aligned(1024))) char st2[RAW];
  __shared__ __attribute__((aligned(1024))) char st3[RAW];
  __shared__ __attribute__((aligned(1024))) char st4[NST > 4 ? RAW : 16];
  __shared__ __attribute__((aligned(1024))) char st5[NST > 5 ? RAW : 16];
  __shared__ __attribute__((aligned(16))) char xs0[XS];
  __shared__ __attribute__((aligned(16))) char xs1[XS];
  __shared__ __attribute__((aligned(16))) float xa0[NW * 16];
  __shared__ __attribute__((aligned(16))) float xa1[NW * 16];
  __shared__ __attribute__((aligned(16))) int ring[NST][NW * 64];   // index ring (as in the bf16 kernel)
  __shared__ __attribute__((aligned(16))) float vbias[NST][BT];   // per stage: 0 (valid slot) or -inf
  __shared__ float lsh[NW * 16];
  __shared__ int sred[4];
  char* const stages[6] = {st0, st1, st2, st3, st4, st5};
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

  // Q in the permuted d_qk order: window t, lane (g, n): columns 64t + 16g ..
  // +15 of head n; the first 8 are the B operand of MFMA step 2t, the last 8
  // of step 2t+1 (the K reads below use the same order).
  bf16x8 qf[NP][2];
  {
    const uint16_t* qrow = a.q + (int64_t)wi.token * a.q_st + (int64_t)head * a.q_sh + 16 * g;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      qf[t][0] = *(const bf16x8*)(qrow + 64 * t);
      qf[t][1] = *(const bf16x8*)(qrow + 64 * t + 8);
    }
  }
  const SplitScan sc = scan_split<BT, NW * 64>(irow, lo, hi, a.s_kv, sred, tid);
  const int nblk = sc.nblk;
  PipeState st;
#pragma unroll
  for (int t = 0; t < 32; ++t) st.o[t] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  st.running_max = kNegInf;
  st.running_max_for_softmax = kNegInf;
  st.sumexp = 0.f;
  const KvSource<BUF> src(a.kv, a.kv_window_bytes);

  // Per-lane LDS offsets.  K read (window t, key tile kt): row 16kt + n, chunk
  // 4t + g.  V read (fragment jj = dv tile 8w + jj): lane (j, 2k + h) points at
  // row R_j(k) = k < 4 ? 4j + k : 16 + 4j + k - 4, bytes 8h..8h+7 of chunk 8w + jj;
  // the transposed read hands lane (j, i) the codes of dv column i for keys
  // R_j(0..7), which is the key order of the S operand (the QKᵀ output layout).
  int kbase[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
    kbase[kt] = fp8_unit(0, 2 * kt + (n >> 3)) * 1024 + g * 128 + (n & 7) * 16;
  auto k_off = [&](int t, int kt) __attribute__((always_inline)) {
    return kbase[kt] + (t >> 1) * 4096 + (t & 1) * 512;
  };
  int vbase;
  {
    const int j = lane >> 4, k = (lane & 15) >> 1, h = lane & 1;
    const int R = k < 4 ? 4 * j + k : 16 + 4 * j + (k - 4);
    vbase = w * 4096 + fp8_unit(0, R >> 3) * 1024 + (R & 7) * 16 + 8 * h;
  }
  // Scales of this lane's keys 16kt + 4g + r: group 0..3 (one 16-byte slot of
  // chunk 36) and group 4 (first word of chunk 37).
  auto scale_off = [&](int kt, int r) __attribute__((always_inline)) {
    const int R = 16 * kt + 4 * g + r;
    return fp8_unit(4, R >> 3) * 1024 + (4 * 8 + (R & 7)) * 16;
  };

  // Row index of this lane's gather slot in block b (row 8w + lane%8) into
  // ring slot r by a direct-to-LDS buffer load over the split's index row
  // (slots past the split read 0 without a memory access); issued in every
  // iteration, read and tested when the gather is prepared, NST-2 iterations
  // later.
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc((void*)irow, 0, hi * 4, 0x00020000);
  auto load_idx = [&](int b, auto R) __attribute__((always_inline)) {
    const int j = lo + b * BT + 8 * w + (lane & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, (LDS_AS void*)(&ring[decltype(R)::value][w * 64]), 4,
                                             (uint32_t)j * 4u, 0, 0, 0);
  };
  const char* const ring_lane = (const char*)&ring[0][w * 64 + (lane & 7)];
  auto read_idx = [&](auto R) __attribute__((always_inline)) {
    return lds_read_opaque<decltype(R)::value * NW * 64 * 4>(ring_lane);
  };
  // Gather of block b's row block w: 5 instructions, chunk group m of rows
  // 8w + lane%8 (chunk lane/8 of each 128-byte line).
  struct Gather {
    uint32_t voff;
    const char* base;
  };
  auto prepare_gather = [&](Gather& gt, int s, int b, int raw) __attribute__((always_inline)) {
    const int j = lo + b * BT + 8 * w + (lane & 7);
    const bool valid = j < hi && raw >= 0 && (int64_t)raw < a.s_kv;
    const int row = valid ? raw : sc.pad_row;
    const int c = lane >> 3;
    if constexpr (BUF)   // blocks past the split: dummy loads, dropped by the range check
      gt.voff = b < nblk ? (uint32_t)row * (uint32_t)a.kv_row_bytes + (uint32_t)(c << 4) : kDummyOffset;
    else
      gt.base = a.kv + (int64_t)row * a.kv_row_bytes + (c << 4);
    if (lane < 8) vbias[s][8 * w + lane] = valid ? 0.f : kNegInf;   // lanes 0..7: rows 8w..8w+7
  };
  // score biases of keys 16kt + 4g + r of stage s
  auto load_bias = [&](int s, f32x4 (&bias)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) bias[kt] = lds_load<f32x4>((const char*)&vbias[s][0], (16 * kt + 4 * g) * 4);
  };
  auto issue = [&](const Gather& gt, char* stage, int m) __attribute__((always_inline)) {
    src.load16((LDS_AS void*)(stage + fp8_unit(m, w) * 1024), gt.voff, gt.base, 128 * m);
  };

  // ---- Pᵀ = Σ_G scale_G(row) · (K_G·Q_Gᵀ) with MFMA 16x16x32 bf16 on the
  // converted codes.  MFMA i: window t = i / 4, key tile kt = (i / 2) % 2, step
  // half h = i % 2; scale group G = t / 2 owns MFMAs 8G .. 8G+7 (group 4: 32..35).
  // Groups accumulate alternately in two register sets; group G is scaled and
  // folded into P (fp32) at the end of group G+1, when its MFMAs are done and
  // before group G+2 reuses the set.  Group 4 stays in set 0 and is folded by
  // the softmax.  hook(i) runs after MFMA i.
  struct QkOut {
    f32x4 acc[KT];          // group 4 partial sums
    float p[KT][4];         // groups 0..3, scaled
    float sc4g[KT][4];      // group 4 scales of this lane's keys
  };
  auto qk = [&](const char* tile, QkOut& qo, auto&& hook) __attribute__((always_inline)) {
    constexpr int NR = NP * KT;               // K reads per block
    f32x4 acc[2][KT];
    float scg[KT][4];
    i32x4 kraw[PF];
    bf16x8 kop[2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) qo.p[kt][r] = 0.f;
    auto read_group_scales = [&](int G, float (&dst)[KT][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[kt][r] = lds_load<float>(tile, scale_off(kt, r) + (G < 4 ? 4 * G : 128));
    };
    auto fold = [&](int set) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) qo.p[kt][r] = fmaf(scg[kt][r], acc[set][kt][r], qo.p[kt][r]);
    };
    static_for<0, PF>([&](auto I) __attribute__((always_inline)) {
      constexpr int r = decltype(I)::value;
      kraw[r] = lds_load<i32x4>(tile, k_off(r / KT, r % KT));
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NQ>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      constexpr int r = i / 2, h = i % 2;     // read r: window r / KT, key tile r % KT
      constexpr int t = r / KT, kt = r % KT;
      constexpr int G = t / 2;
      if constexpr (h == 0) {
        fp8x16_to_bf16(kraw[r % PF], kop[0], kop[1]);
        if constexpr (r + PF < NR) kraw[r % PF] = lds_load<i32x4>(tile, k_off((r + PF) / KT, (r + PF) % KT));
      }
      constexpr bool first = t % 2 == 0 && h == 0;   // first MFMA of group G for this key tile
      acc[G & 1][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          kop[h], qf[t][h], first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[G & 1][kt], 0, 0, 0);
      // group Gf = i/8 - 1 is folded after MFMA 8(Gf+1)+7 (group 3: after the
      // last MFMA); its scales are read 7 (3) MFMAs earlier
      if constexpr (i >= 8 && i % 8 == 0) read_group_scales(i / 8 - 1, scg);
      if constexpr (i >= 15 && i % 8 == 7) fold(((i / 8) - 1) & 1);
      if constexpr (i == NQ - 1) {
        fold(1);                              // group 3 (scales read after MFMA 32)
        read_group_scales(4, qo.sc4g);
        qo.acc[0] = acc[0][0];
        qo.acc[1] = acc[0][1];
      }
      hook(I);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- online softmax in steps (as in the bf16 kernel) on P = Σ_G scale·acc_G;
  // the published operands are bf16(S · scale_G) for the four V groups G
  // (sc4: those scales of this lane's keys, read while the softmax runs).
  struct Soft {
    float x[KT][4];
    float cur, alpha;
    bool any;
  };
  // step 5 also publishes the block's S operands (one per V group) and
  // rescale factors into exchange buffer p, early enough for the writes to
  // land while the remaining PV MFMAs run
  auto soft_step = [&](auto K, Soft& sm, const QkOut& qo, const f32x4 (&bias)[KT], const f32x4 (&sc4)[KT][4],
                       int p) __attribute__((always_inline)) {
    // no contraction across the steps (the running state rounds the same way
    // wherever the compiler places the steps)
#pragma clang fp contract(off)
    constexpr int k = decltype(K)::value;
    if constexpr (k == 0) {
      // an invalid slot's bias of -inf masks it; a valid slot's 0 changes nothing
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.x[kt][r] = __builtin_fmaf(fmaf(qo.sc4g[kt][r], qo.acc[kt][r], qo.p[kt][r]), a.scale_log2, bias[kt][r]);
      float c = sm.x[0][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) c = fmaxf(c, sm.x[kt][r]);
      sm.cur = c;
    } else if constexpr (k == 1) {
      sm.cur = wave_max16x4(sm.cur);
    } else if constexpr (k == 2) {
      const float rmax = fmaxf(st.running_max, sm.cur);
      st.running_max = rmax;
      const bool trig = rmax - st.running_max_for_softmax > kRescaleThresLog2;
      sm.any = __ballot(trig) != 0ull;
      // factor 1 while the head's accumulators are still zero (first block)
      const float al = __builtin_amdgcn_exp2f(st.running_max_for_softmax - rmax);
      sm.alpha = sm.any && st.running_max_for_softmax != kNegInf ? al : 1.0f;
      st.running_max_for_softmax = sm.any ? rmax : st.running_max_for_softmax;
      st.sumexp *= sm.alpha;
    } else if constexpr (k == 3 || k == 4) {
      // a masked slot weighs exp2(-inf) = 0; while the running max is -inf
      // every score of the head is -inf and any finite offset gives zeros
      constexpr int kt = k - 3;
      const float m = st.running_max_for_softmax == kNegInf ? 0.f : st.running_max_for_softmax;
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.x[kt][r] = __builtin_amdgcn_exp2f(sm.x[kt][r] - m);
    } else if constexpr (k == 5) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.sumexp += sm.x[kt][r];
      // S operand of each V group G with that group's row scales
#pragma unroll
      for (int G = 0; G < NW; ++G) {
        union { uint32_t u[4]; bf16x8 v; } t;
        t.u[0] = pack2_bf16(sm.x[0][0] * sc4[0][0][G], sm.x[0][1] * sc4[0][1][G]);
        t.u[1] = pack2_bf16(sm.x[0][2] * sc4[0][2][G], sm.x[0][3] * sc4[0][3][G]);
        t.u[2] = pack2_bf16(sm.x[1][0] * sc4[1][0][G], sm.x[1][1] * sc4[1][1][G]);
        t.u[3] = pack2_bf16(sm.x[1][2] * sc4[1][2][G], sm.x[1][3] * sc4[1][3][G]);
        *(LDS_AS bf16x8*)((LDS_AS char*)(LDS_AS void*)xss[p] + ((G * NW + w) * 64 + lane) * 16) = t.v;
      }
      *(LDS_AS float*)((LDS_AS char*)(LDS_AS void*)xas[p] + (w * 16 + n) * 4) = sm.alpha;   // same in all g
    }
  };
  constexpr int NSOFT = 6;
  auto read_scales = [&](const char* tile, f32x4 (&sc4)[KT][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc4[kt][r] = lds_load<f32x4>(tile, scale_off(kt, r));
  };

  // ---- prologue: indices of blocks 0..NST-1, gathers of blocks 0..NST-2,
  // then the indices of blocks NST..2·NST-4.  Ring slot b % NST holds the
  // indices of block b from their load until its gather is prepared (in
  // iteration b-NST+1; the load is in iteration b-2·NST+3, before the gathers
  // that iteration issues, so the wait for those gathers covers it).
  constexpr int XI = NST - 3;                 // index loads after the prologue gathers
  if (nblk > 0) {
    static_for<0, NST>([&](auto B) __attribute__((always_inline)) { load_idx(decltype(B)::value, B); });
    wait_vm_lgkm0<0>();   // the ring reads below are opaque to the compiler's waits
    static_for<0, NST - 1>([&](auto B) __attribute__((always_inline)) {   // past the split: dummy loads
      constexpr int b = decltype(B)::value;
      Gather gt;
      prepare_gather(gt, b, b, read_idx(B));
#pragma unroll
      for (int m = 0; m < LPB; ++m) issue(gt, stages[b], m);
    });
    static_for<NST, NST + XI>([&](auto B) __attribute__((always_inline)) {
      load_idx(decltype(B)::value, std::integral_constant<int, decltype(B)::value % NST>{});
    });
    // block 0: wait for its gathers (the later ones stay in flight)
    wait_vm_lgkm0<(NST - 2) * LPB + XI>();
    barrier_no_vm_drain();
    QkOut qo;
    qk(st0, qo, [&](auto) {});
    f32x4 bias[KT];
    load_bias(0, bias);
    f32x4 sc4[KT][4];
    read_scales(st0, sc4);
    Soft sm;
    static_for<0, NSOFT>([&](auto K) __attribute__((always_inline)) { soft_step(K, sm, qo, bias, sc4, 0); });
  }

  // ---- iteration i: consume S(i); QKᵀ(i+1); PV(i) with softmax(i+1); refill
  // the stage of block i-1 with block i+NST-1; load the row index of block
  // i+2·NST-3.
  auto iteration = [&](auto S, int i, auto FIRST_, auto DYN_) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;     // stage of block i
    constexpr int p = s & 1;                  // exchange buffer of block i (i and s have one parity)
    constexpr bool FIRST = decltype(FIRST_)::value;   // i = s <= NST-3
    constexpr bool DYN = decltype(DYN_)::value;
    const bool next = DYN ? i + 1 < nblk : true;
    // Every iteration issues the same memory instructions (loads for blocks
    // past the split are dummies), so the wait counts are constants.
    // gather(i+1) was issued in iteration i-(NST-2), or for a first iteration
    // in the prologue; younger are, in each of the iterations i-(NST-3)..i-1,
    // an index load and a block's gathers, and for a first iteration the
    // prologue's later gathers and XI index loads: (NST-3)·(LPB+1) + i.
    wait_vm_lgkm0<(NST - 3) * (LPB + 1) + (FIRST ? s : 0)>();
    barrier_no_vm_drain();

    // block i+2·NST-3 takes the ring slot of block i+NST-3 (prepared in
    // iteration i-2); block i+NST-1's index was loaded in iteration i-NST+2
    load_idx(i + 2 * NST - 3, std::integral_constant<int, (s + NST - 3) % NST>{});
    Gather gt;
    constexpr int rs = (s + NST - 1) % NST;   // stage of block i-1 = stage of block i+NST-1
    prepare_gather(gt, rs, i + NST - 1, read_idx(std::integral_constant<int, (s + NST - 1) % NST>{}));
    auto dma_at = [&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value, N = NQ + NPV;
      static_for<(c * LPB + N - 1) / N, ((c + 1) * LPB + N - 1) / N>([&](auto K) __attribute__((always_inline)) {
        issue(gt, stages[rs], decltype(K)::value);
      });
    };

    bf16x8 sop[NW];
    float alph[NW];
    f32x4 bias[KT];
    f32x4 sc4[KT][4];
    constexpr int sn = (s + 1) % NST;         // stage of block i+1
    auto consume_reads = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ht = 0; ht < NW; ++ht) {
        sop[ht] = lds_load<bf16x8>(xss[p], ((w * NW + ht) * 64 + lane) * 16);
        alph[ht] = lds_load<float>((const char*)xas[p], (ht * 16 + n) * 4);
      }
    };
    const char* const tile = stages[s];
    i32x2 vraw[PFV];
    auto fetch_v = [&](int jj) __attribute__((always_inline)) {
      vraw[jj % PFV] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS_AS i32x2*)((LDS_AS char*)(LDS_AS void*)tile + vbase + jj * 128));
    };

    QkOut qo;
    if (next) {
      qk(stages[sn], qo, [&](auto I) __attribute__((always_inline)) {
        constexpr int q = decltype(I)::value;
        if constexpr (q == 0) consume_reads();
        if constexpr (q == NQ - 4) load_bias(sn, bias);   // shortly before the softmax of block i+1
        if constexpr (q >= NQ - 8 && (q - (NQ - 8)) % 2 == 0) fetch_v((q - (NQ - 8)) / 2);
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

    if (__ballot(alph[0] != 1.0f || alph[1] != 1.0f || alph[2] != 1.0f || alph[3] != 1.0f) != 0ull) {
      static_for<0, NW>([&](auto H) __attribute__((always_inline)) {
        constexpr int ht = decltype(H)::value;
        if (__ballot(alph[ht] != 1.0f) != 0ull) {   // only the head tiles whose owner rescaled
          static_for<0, 8>([&](auto J) __attribute__((always_inline)) {
            constexpr int t = ht * 8 + decltype(J)::value;
            st.o[t] = pin_agpr(pin_agpr(st.o[t]) * alph[ht]);
          });
        }
      });
    }

    // ---- Oᵀ += Vᵀ·Sᵀ for this wave's group: MFMA c uses V fragment c/4 and
    // the S of head tile c%4; the softmax of block i+1 between the MFMAs.
    Soft sm;
    bf16x8 vop;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NPV>([&](auto I) __attribute__((always_inline)) {
      constexpr int c = decltype(I)::value;
      constexpr int jj = c / NW, ht = c % NW;
      if constexpr (ht == 0) {
        vop = fp8x8_to_bf16(vraw[jj % PFV]);
        if constexpr (jj + PFV < 8) fetch_v(jj + PFV);
      }
      st.o[ht * 8 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, sop[ht], st.o[ht * 8 + jj], 0, 0, 0);
      if constexpr (c == 4) {
        if (next) read_scales(stages[sn], sc4);   // V-group scales for step 5
      }
      if constexpr (c % 3 == 1 && c / 3 < NSOFT) {
        if (next) soft_step(std::integral_constant<int, c / 3>{}, sm, qo, bias, sc4, p ^ 1);
      }
      dma_at(std::integral_constant<int, NQ + c>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  using T = std::integral_constant<bool, true>;
  using F = std::integral_constant<bool, false>;
  // Iterations that may not run are nested, so that each is reached only from
  // the one before it (the compiler's own waits then see every memory
  // instruction of the earlier iterations): the first NST-2 iterations, then
  // (inside the last of them) the steady groups and the last blocks.
  auto tail = [&](auto self, auto K, int i0) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    if constexpr (k < NST) {
      if (i0 + k < nblk) {
        iteration(std::integral_constant<int, (NST - 2 + k) % NST>{}, i0 + k, F{}, T{});
        self(self, std::integral_constant<int, k + 1>{}, i0);
      }
    }
  };
  auto first = [&](auto self, auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    if (k < nblk) {
      iteration(K, k, T{}, T{});
      if constexpr (k + 1 < NST - 2) {
        self(self, std::integral_constant<int, k + 1>{});
      } else {
        // steady state: groups of NST iterations keep every stage index a constant
        int i0 = NST - 2;
        for (; i0 + NST < nblk; i0 += NST) {
          static_for<0, NST>([&](auto J) __attribute__((always_inline)) {
            iteration(std::integral_constant<int, (NST - 2 + decltype(J)::value) % NST>{}, i0 + decltype(J)::value,
                      F{}, F{});
          });
        }
        tail(tail, std::integral_constant<int, 0>{}, i0);
      }
    }
  };
  first(first, std::integral_constant<int, 0>{});
  if (nblk > 0) wait_vm_lgkm0<0>();   // dummy and index loads still in flight

  // ---- epilogue (as in the bf16 kernel)
  const float l = wave_sum16x4(st.sumexp);
  const bool empty = sc.nvalid == 0;
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
  for (int ht = 0; ht < NW; ++ht) inv[ht] = empty ? 0.f : 1.0f / lsh[ht * 16 + n];
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
