// Software-pipelined forward kernel for a quantised KV cache (fp8 E4M3 rows of
// 640 bytes, fp4 E2M1 rows of 320), 64 heads per workgroup, B_TOPK 32.
//
// Method as in smla_fwd.cuh (page "Ascend Sparse Attention Forward
// 算法与优化技术简析", sections 数学建模 and 计算流程); the KV rows are the packed
// rows of section "Decoding KV Cache Layout 优化" (codes next to their five
// float32 group scales).  Dequantisation is exact: every code is a bf16 value,
// the MFMAs take the codes unchanged and the scales are applied in fp32 (QKᵀ:
// one accumulator per 128-column group, folded with the row's scales; PV: the
// V group's row scale folded into the bf16 S operand).
//
// Each block's codes are converted ONCE per workgroup, into a bf16 stage in the
// layout of the bf16 kernels, and the products then run as in the bf16
// pipelined kernel (smla_fwd_pipe.cuh: d_v split of PV, QKᵀ of block i+1 before
// PV of block i, softmax of block i+1 between the PV MFMAs).  Converting the
// codes in registers at the operand reads instead repeats the conversion of
// every K code in each of the four waves.  Raw stages: four for fp4, two for
// fp8 (what fits beside two bf16 stages and the S exchange).  Per iteration i:
//   barrier; QKᵀ(i+1) on bf16 stage (i+1)&1 and PV(i) on stage i&1, the raw
//   stage freed in the last iteration refilled with block i+1+NR by gathers
//   spread over the MFMAs;
//   barrier; convert raw block i+2 into bf16 stage i&1 (free now: every wave
//   is past PV(i)) and its scales into the stage's scale tile.
// The split's valid indices are compacted into LDS once (as in the
// non-pipelined kernels: masked slots carry zero weight, the last block's
// padding slots repeat the first valid row and are masked by count), so no
// index is loaded inside the loop, and every iteration issues the same memory
// instructions (loads for blocks past the split are dummies): the wait counts
// are compile-time constants.
#pragma once

#include "smla_fwd_pipe.cuh"

namespace smla {
namespace {

template <bool SPLIT, bool BUF, class Fmt>
__global__ __launch_bounds__(256) void smla_fwd_q_pipe_kernel(FwdArgs a) {
  debug_poison_lds();
  constexpr int NW = 4, BT = 32, KT = 2;
  constexpr bool FP4 = Fmt::ROW == 320;
  // raw stages: blocks in flight ahead of the conversion (what fits beside two
  // bf16 stages and the S exchange)
  constexpr int NR = FP4 ? 4 : 2;
  constexpr int NQ = 36;                      // QK MFMAs per block
  constexpr int NPV = 32;                     // PV MFMAs per block
  using Gather = RawGather<NW, BUF, Fmt, true>;   // swizzled rows (conflict-free conversion reads)
  constexpr int LPB = Gather::PER_WAVE;       // gather instructions per wave per block
  constexpr int RAW = BT * Fmt::ROW;
  constexpr int TILE = BT * kRowBytesBf16;
  constexpr int UG = (BT / 8) * 1024;         // bytes between chunk groups of a bf16 stage
  constexpr int PF = 12;                      // K operand reads in flight
  constexpr int PFV = 4;                      // V fragments (two reads each) in flight
  constexpr int XS = NW * NW * 64 * 16;       // S operands of one block: [V group][head tile][lane]
  static_assert(4 % NR == 0, "the iteration loop is unrolled by four");
  static_assert(NR * RAW + 2 * TILE + 2 * XS + Fmt::MAX_SLOTS * 4 < 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char rw0[RAW];
  __shared__ __attribute__((aligned(1024))) char rw1[RAW];
  __shared__ __attribute__((aligned(1024))) char rw2[NR > 2 ? RAW : 16];
  __shared__ __attribute__((aligned(1024))) char rw3[NR > 3 ? RAW : 16];
  __shared__ __attribute__((aligned(1024))) char tl0[TILE];
  __shared__ __attribute__((aligned(1024))) char tl1[TILE];
  __shared__ __attribute__((aligned(16))) float sc0[5 * BT];
  __shared__ __attribute__((aligned(16))) float sc1[5 * BT];
  __shared__ __attribute__((aligned(16))) char xs0[XS];
  __shared__ __attribute__((aligned(16))) char xs1[XS];
  __shared__ __attribute__((aligned(16))) float xa0[NW * 16];
  __shared__ __attribute__((aligned(16))) float xa1[NW * 16];
  __shared__ int sidx[Fmt::MAX_SLOTS + BT];
  __shared__ int swcnt[NW];
  __shared__ float lsh[NW * 16];
  char* const raws[4] = {rw0, rw1, rw2, rw3};
  char* const tiles[2] = {tl0, tl1};
  float* const stiles[2] = {sc0, sc1};
  char* const xss[2] = {xs0, xs1};
  float* const xas[2] = {xa0, xa1};

  WorkItem wi;
  if (!work_item(a, wi)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int lo = wi.split * a.slots_per_split;
  const int hi = min(a.topk, lo + a.slots_per_split);
  const int head = wi.head0 + w * 16 + n;

  const int nvalid = compact_slots<NW>(a.idx + (int64_t)wi.token * a.idx_st, lo, hi, a.s_kv, sidx, swcnt, tid);
  const int nblk = (nvalid + BT - 1) / BT;
  for (int j = nvalid + tid; j < nblk * BT; j += NW * 64) sidx[j] = sidx[0];
  __syncthreads();

  PipeState st;
#pragma unroll
  for (int t = 0; t < 32; ++t) st.o[t] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  st.running_max = kNegInf;
  st.running_max_for_softmax = kNegInf;
  st.sumexp = 0.f;

  if (nblk > 0) {
    const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
    const KvSource<BUF> src(a.kv, a.kv_window_bytes);
    const int wbase = 2 * UG * w;             // this wave's 128 dv columns (V group w): chunk groups 2w, 2w+1

    // gather block b into raw stage r (a dummy past the split)
    auto prepare = [&](Gather& gt, int r, int b) __attribute__((always_inline)) {
      if (b < nblk)
        gt.prepare(raws[r], src, a.kv_row_bytes, sidx + b * BT, tid);
      else
        gt.prepare_dummy(raws[r], src, tid);
    };
    // Convert raw stage R into bf16 stage / scale tile p.  Wave w converts row
    // block w: lane l takes row 8w + l%8 and the 16-byte bf16 chunks
    // 8k + l/8, k < 9 (8 codes: 4 raw bytes of E2M1 or 8 of E4M3, exact at
    // scale 1), and
    // writes chunk k to slot l of unit (k, w) of the stage: every store of the
    // wave is one contiguous 1 KB unit (no bank conflict).  Lanes 0..39 also
    // copy scale group l/8 of their row.  The raw reads are one asm block that
    // waits for its own results: the caller's wait and barrier guarantee the
    // rows have landed, and reads the compiler could see would make it wait
    // for every younger gather as well.
    static_assert(FP4 ? Fmt::CODE_BYTES == 288 : (Fmt::ROW == 640 && Fmt::CODE_BYTES == 576), "row formats");
    auto convert = [&](auto R, int p) __attribute__((always_inline)) {
      constexpr int r = decltype(R)::value;
      const int row = 8 * w + (lane & 7), gsel = min(lane >> 3, 4), x = raw_swizzle<Fmt>(row);
      const uint32_t rbase = (uint32_t)(uintptr_t)(const LDS_AS void*)raws[r] + row * Fmt::ROW;
      // 8 codes per bf16 chunk: 4 bytes (E2M1) or 8 bytes (E4M3).  Raw chunk
      // (bf16 chunk 8k + l/8) / 4 or / 2 = 2k + l/32 (E2M1) or 4k + l/16
      // (E4M3); the row's swizzle XORs its low bits, the k part rides in the
      // immediate offsets.
      const uint32_t caddr = FP4 ? rbase + ((((lane >> 5) ^ x) << 4) | (((lane >> 3) & 3) << 2))
                                 : rbase + ((((lane >> 4) ^ x) << 4) | (((lane >> 3) & 1) << 3));
      // scale g: byte 4(g%4) of raw chunk CODE_BYTES/16 + g/4 (low chunk bits free)
      const uint32_t saddr = rbase + Fmt::CODE_BYTES + ((((gsel >> 2) ^ x) << 4) | ((gsel & 3) << 2));
      float scl;
      uint32_t o[9][4];
      if constexpr (FP4) {
        uint32_t code[9];
        asm volatile(
            "ds_read_b32 %0, %10\n\tds_read_b32 %1, %10 offset:32\n\tds_read_b32 %2, %10 offset:64\n\t"
            "ds_read_b32 %3, %10 offset:96\n\tds_read_b32 %4, %10 offset:128\n\tds_read_b32 %5, %10 offset:160\n\t"
            "ds_read_b32 %6, %10 offset:192\n\tds_read_b32 %7, %10 offset:224\n\tds_read_b32 %8, %10 offset:256\n\t"
            "ds_read_b32 %9, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            // early-clobber: a read's result must not land in a register that
            // still holds an address of the block
            : "=&v"(code[0]), "=&v"(code[1]), "=&v"(code[2]), "=&v"(code[3]), "=&v"(code[4]),
              "=&v"(code[5]), "=&v"(code[6]), "=&v"(code[7]), "=&v"(code[8]), "=&v"(scl)
            : "v"(caddr), "v"(saddr)
            : "memory");
#pragma unroll
        for (int k = 0; k < 9; ++k)
          static_for<0, 4>([&](auto J) __attribute__((always_inline)) {
            // byte j: columns 8c + 2j (low nibble) and 8c + 2j + 1 (high nibble)
            constexpr int j = decltype(J)::value;
            o[k][j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code[k], 1.0f, j));
          });
      } else {
        i32x2 code[9];
        asm volatile(
            "ds_read_b64 %0, %10\n\tds_read_b64 %1, %10 offset:64\n\tds_read_b64 %2, %10 offset:128\n\t"
            "ds_read_b64 %3, %10 offset:192\n\tds_read_b64 %4, %10 offset:256\n\tds_read_b64 %5, %10 offset:320\n\t"
            "ds_read_b64 %6, %10 offset:384\n\tds_read_b64 %7, %10 offset:448\n\tds_read_b64 %8, %10 offset:512\n\t"
            "ds_read_b32 %9, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(code[0]), "=&v"(code[1]), "=&v"(code[2]), "=&v"(code[3]), "=&v"(code[4]),
              "=&v"(code[5]), "=&v"(code[6]), "=&v"(code[7]), "=&v"(code[8]), "=&v"(scl)
            : "v"(caddr), "v"(saddr)
            : "memory");
#pragma unroll
        for (int k = 0; k < 9; ++k)
          static_for<0, 4>([&](auto J) __attribute__((always_inline)) {
            // word j/2, half j%2: columns 8c + 2j and 8c + 2j + 1
            constexpr int j = decltype(J)::value;
            o[k][j] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)code[k][j >> 1], 1.0f, (j & 1) != 0));
          });
      }
      if (lane < 40) stiles[p][gsel * BT + row] = scl;
#pragma unroll
      for (int k = 0; k < 9; ++k)
        *(LDS_AS i32x4*)((LDS_AS char*)(LDS_AS void*)tiles[p] + (k * 4 + w) * 1024 + lane * 16) =
            i32x4{(int)o[k][0], (int)o[k][1], (int)o[k][2], (int)o[k][3]};
    };

    bf16x8 qf[18];
    // ---- prologue: blocks 0..NR-1 in flight, then Q; blocks 0 and 1 converted,
    // block NR into the raw stage of block 0
    static_for<0, NR>([&](auto B) __attribute__((always_inline)) {
      Gather gt;
      prepare(gt, decltype(B)::value, decltype(B)::value);
      gt.issue_all();
    });
    load_q(a, wi.token, head, g, qf);
    wait_vm_lgkm0<(NR - 2) * LPB + 18>();
    barrier_no_vm_drain();
    convert(std::integral_constant<int, 0>{}, 0);
    convert(std::integral_constant<int, 1>{}, 1);
    wait_vm_lgkm0<63>();
    barrier_no_vm_drain();
    {
      Gather gt;
      prepare(gt, 0, NR);
      gt.issue_all();
    }

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

    // ---- Pᵀ = Σ_G scale_G(row) · (K_G·Q_Gᵀ).  MFMA i: d_qk step s = i / 2 (32
    // columns), key tile kt = i % 2; scale group G = s / 4 owns MFMAs
    // 8G .. 8G+7 (group 4: 32..35).  Groups accumulate alternately in two
    // register sets; group G is folded (fp32 scale of the lane's key times its
    // partial sum) at the end of group G+1, group 3 after the last MFMA, and
    // group 4 (set 0) by the softmax.  The scales of groups 0..3 stay in qo.sc
    // for the S operands of the V groups.  hook(i) runs after MFMA i.
    struct QkOut {
      f32x4 acc[KT];          // group 4 partial sums
      float p[KT][4];         // groups 0..3, scaled
      float sc4g[KT][4];      // group 4 scales of this lane's keys
      f32x4 sc[NW][KT];       // V-group scales (groups 0..3) of this lane's keys, for S
    };
    auto qk = [&](const char* tile, const float* stile, QkOut& qo, auto&& hook) __attribute__((always_inline)) {
      f32x4 acc[2][KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) qo.p[kt][r] = 0.f;
      auto read_group_scales = [&](int G, float (&dst)[KT][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const f32x4 v = lds_load<f32x4>((const char*)stile, (G * BT + 16 * kt + 4 * g) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[kt][r] = v[r];
        }
      };
      auto fold = [&](int set, int G) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) qo.p[kt][r] = fmaf(qo.sc[G][kt][r], acc[set][kt][r], qo.p[kt][r]);
      };
      auto read_vgroup_scales = [&](int G) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          qo.sc[G][kt] = lds_load<f32x4>((const char*)stile, (G * BT + 16 * kt + 4 * g) * 4);
      };
      bf16x8 abuf[PF];
      static_for<0, PF>([&](auto I) __attribute__((always_inline)) {
        abuf[decltype(I)::value] = lds_load<bf16x8>(tile, qk_off(decltype(I)::value));
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NQ>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        constexpr int s = i / KT, kt = i % KT, G = s / 4;
        constexpr bool first = s % 4 == 0;    // first step of group G for this key tile
        acc[G & 1][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            abuf[i % PF], qf[s], first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[G & 1][kt], 0, 0, 0);
        if constexpr (i + PF < NQ) abuf[i % PF] = lds_load<bf16x8>(tile, qk_off(i + PF));
        if constexpr (i >= 8 && i % 8 == 0) read_vgroup_scales(i / 8 - 1);
        if constexpr (i >= 15 && i % 8 == 7) fold(((i / 8) - 1) & 1, (i / 8) - 1);
        if constexpr (i == NQ - 1) {
          fold(1, 3);                         // group 3 (scales read after MFMA 32)
          read_group_scales(4, qo.sc4g);
          qo.acc[0] = acc[0][0];
          qo.acc[1] = acc[0][1];
        }
        hook(I);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- online softmax in steps on P = Σ_G scale·acc_G; step 5 publishes the
    // block's S operands, one per V group G (bf16(S · scale_G(row))), and the
    // rescale factors.
    struct Soft {
      float x[KT][4];
      float cur, alpha;
      bool any;
    };
    auto soft_step = [&](auto K, Soft& sm, const QkOut& qo, int j0, const f32x4 (&sc4)[NW][KT], int p)
        __attribute__((always_inline)) {
#pragma clang fp contract(off)
      constexpr int k = decltype(K)::value;
      if constexpr (k == 0) {
        // scaled logits in log2 units; the padding slots of the last block
        // (index past the valid count) are masked
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = fmaf(qo.sc4g[kt][r], qo.acc[kt][r], qo.p[kt][r]) * a.scale_log2;
            sm.x[kt][r] = (j0 + 16 * kt + r < nvalid) ? v : kNegInf;
          }
        float c = sm.x[0][0];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) c = fmaxf(c, sm.x[kt][r]);
        sm.cur = c;
      } else if constexpr (k == 1) {
        sm.cur = wave_max16x4(sm.cur);
      } else if constexpr (k == 2) {
        // every block holds a valid slot: the new running max is finite
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
        constexpr int kt = k - 3;
        const float m = st.running_max_for_softmax;
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.x[kt][r] = __builtin_amdgcn_exp2f(sm.x[kt][r] - m);
      } else if constexpr (k == 5) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) st.sumexp += sm.x[kt][r];
#pragma unroll
        for (int G = 0; G < NW; ++G) {
          union { uint32_t u[4]; bf16x8 v; } t;
          t.u[0] = pack2_bf16(sm.x[0][0] * sc4[G][0][0], sm.x[0][1] * sc4[G][0][1]);
          t.u[1] = pack2_bf16(sm.x[0][2] * sc4[G][0][2], sm.x[0][3] * sc4[G][0][3]);
          t.u[2] = pack2_bf16(sm.x[1][0] * sc4[G][1][0], sm.x[1][1] * sc4[G][1][1]);
          t.u[3] = pack2_bf16(sm.x[1][2] * sc4[G][1][2], sm.x[1][3] * sc4[G][1][3]);
          *(LDS_AS bf16x8*)((LDS_AS char*)(LDS_AS void*)xss[p] + ((G * NW + w) * 64 + lane) * 16) = t.v;
        }
        *(LDS_AS float*)((LDS_AS char*)(LDS_AS void*)xas[p] + (w * 16 + n) * 4) = sm.alpha;   // same in all g
      }
    };
    constexpr int NSOFT = 6;

    // block 0: QKᵀ and softmax, published for iteration 0
    {
      QkOut qo;
      qk(tiles[0], stiles[0], qo, [&](auto) {});
      Soft sm;
      static_for<0, NSOFT>([&](auto K) __attribute__((always_inline)) {
        soft_step(K, sm, qo, 4 * g, qo.sc, 0);
      });
    }

    // ---- iteration i (S = i mod 4: block i in bf16 stage i&1, block i+1 in the
    // other; every LDS object an iteration touches is a compile-time choice, so
    // the compiler's tracking of the direct-to-LDS writes sees which stage each
    // gather fills)
    auto iteration = [&](auto S, int i) __attribute__((always_inline)) {
      constexpr int s4 = decltype(S)::value;
      constexpr int p = s4 & 1;               // = i & 1
      const bool next = i + 1 < nblk;
      // every wave: S(i) published, block i+1 converted
      wait_vm_lgkm0<63>();
      barrier_no_vm_drain();

      // refill the raw stage of block i+1 (converted last iteration) with
      // block i+1+NR, spread over the MFMAs of both products
      Gather gt;
      prepare(gt, (s4 + 1) % NR, i + 1 + NR);
      auto dma_at = [&](auto C) __attribute__((always_inline)) {
        constexpr int c = decltype(C)::value, N = NQ + NPV;
        static_for<(c * LPB + N - 1) / N, ((c + 1) * LPB + N - 1) / N>(
            [&](auto K) __attribute__((always_inline)) { gt.issue(decltype(K)::value); });
      };

      bf16x8 sop[NW];
      float alph[NW];
      auto consume_reads = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ht = 0; ht < NW; ++ht) {
          sop[ht] = lds_load<bf16x8>(xss[p], ((w * NW + ht) * 64 + lane) * 16);
          alph[ht] = lds_load<float>((const char*)xas[p], (ht * 16 + n) * 4);
        }
      };
      const char* const tile = tiles[p];
      i16x4 va[PFV], vb[PFV];
      auto fetch_v = [&](int jj) __attribute__((always_inline)) {
        va[jj % PFV] = tr_load(tile, tr_off(jj));
        vb[jj % PFV] = tr_load(tile, tr_off(jj) + 2048);
      };

      QkOut qo;
      if (next) {
        qk(tiles[p ^ 1], stiles[p ^ 1], qo, [&](auto I) __attribute__((always_inline)) {
          constexpr int q = decltype(I)::value;
          if constexpr (q == 0) consume_reads();
          if constexpr (q >= NQ - PF && q < NQ - PF + 2 * PFV && (q - (NQ - PF)) % 2 == 0)
            fetch_v((q - (NQ - PF)) / 2);
          dma_at(I);
        });
      } else {
        consume_reads();
#pragma unroll
        for (int jj = 0; jj < PFV; ++jj) fetch_v(jj);
        static_for<0, NQ>([&](auto I) __attribute__((always_inline)) { dma_at(I); });
      }

      // rescale this wave's columns of the head tiles whose owner rescaled
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

      // ---- Oᵀ += Vᵀ·Sᵀ for V group w: MFMA c uses V fragment c/4 and the S of
      // head tile c%4; the softmax of block i+1 between the MFMAs
      Soft sm;
      const int j1 = (i + 1) * BT + 4 * g;
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
          if (next) soft_step(std::integral_constant<int, c / 4>{}, sm, qo, j1, qo.sc, p ^ 1);
        }
        dma_at(std::integral_constant<int, NQ + c>{});
        __builtin_amdgcn_sched_barrier(0);
      });

      // ---- every wave past PV(i): convert block i+2 into stage p once its
      // gathers have landed (younger: the gathers of blocks i+3 .. i+1+NR)
      if (i + 2 < nblk) {
        wait_vm_lgkm0<(NR - 1) * LPB>();
        barrier_no_vm_drain();
        convert(std::integral_constant<int, (s4 + 2) % NR>{}, p);
      }
    };

    int i = 0;
    for (; i + 3 < nblk; i += 4) {
      iteration(std::integral_constant<int, 0>{}, i);
      iteration(std::integral_constant<int, 1>{}, i + 1);
      iteration(std::integral_constant<int, 2>{}, i + 2);
      iteration(std::integral_constant<int, 3>{}, i + 3);
    }
    if (i < nblk) {
      iteration(std::integral_constant<int, 0>{}, i);
      if (i + 1 < nblk) {
        iteration(std::integral_constant<int, 1>{}, i + 1);
        if (i + 2 < nblk) iteration(std::integral_constant<int, 2>{}, i + 2);
      }
    }
    wait_vm_lgkm0<0>();                       // dummy loads still in flight
  }

  // ---- epilogue (as in the bf16 pipelined kernel)
  const float l = wave_sum16x4(st.sumexp);
  const bool empty = nvalid == 0;
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
