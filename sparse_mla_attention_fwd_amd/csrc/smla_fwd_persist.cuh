// Persistent, load-balanced forward kernel for many query tokens of 64 heads
// with bf16 KV, B_TOPK 32, one split per token (prefill and causal prefill).
//
// Method as in smla_fwd_pipe.cuh (page "Ascend Sparse Attention Forward
// 算法与优化技术简析", sections 数学建模 and 计算流程).  Schedule: page "Flash
// Attention Infer算子性能优化", section 优化多核负载均衡 -- when tokens carry
// different numbers of valid blocks (causal or sparse masks), cutting the
// tokens evenly by count leaves a long tail; instead the tokens are dealt to
// the cores greedily by their valid-block weight.  Here:
//
//  * smla_token_blocks_kernel counts each token's blocks up to its last valid
//    slot (at least one block, so an empty token still passes through the
//    pipeline and writes its zero output and -inf lse).  A token's weight is
//    its block count plus the measured cost of a token switch in blocks.
//  * One workgroup per compute unit.  Workgroup g takes the contiguous run of
//    tokens whose running weight (at each token's midpoint) falls in
//    [g·W/G, (g+1)·W/G), W the total weight and G the grid size: every
//    workgroup gets within one token of the mean weight.  Each workgroup
//    computes its own run from the block counts (a scan of all tokens'
//    weights at start-up).
//  * Inside a workgroup the run is one stream of blocks.  The gather ring, the
//    index ring and the skewed QKᵀ/PV pipeline of the pipelined kernel run
//    through token boundaries without draining: the first gathers of the next
//    token are in flight while the current token's last blocks compute.  The
//    next token's Q is loaded right after the last QKᵀ of the current token
//    (the registers are free then), and the finished token's output is
//    normalised and written right after the next barrier, before the first
//    PV product of the new token accumulates.  A token thus costs its blocks
//    plus the epilogue, instead of a pipeline ramp-up and drain of several
//    blocks each.
//
// Positions of the stream are tracked by four cursors (blocks i, i+1, i+3,
// i+5 of iteration i: PV, QKᵀ/softmax, gather, index load), each a (token,
// block) pair that advances by one block per iteration and reads the next
// token's block count ahead of its crossing.  Only the 32-bit buffer-load
// gather form is built (a KV of at most 4 GB): invalid slots and positions
// past the run load from outside the buffer window, which returns zeros
// without a memory access, and their score bias of -inf masks them.
#pragma once

#include "smla_fwd_pipe.cuh"

namespace smla {
namespace {

// Extra weight of a token over its blocks, in blocks: its Q switch and
// epilogue.  Measured with per-iteration shader-clock stamps on the prefill
// workload: a block takes about 2,900 cycles, a token switch about 16,000 more
// (the next token's Q loads and the finished token's output stores each hold
// up one iteration's wait for about 8,000 cycles, memory latency under the
// gathers' load).
constexpr int kTokenWeight = 6;

// (token, block) position of one pipeline stage in the workgroup's stream.
struct Cursor {
  int t, b, nb, nbn;   // token, block in it, its block count, the next token's
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int DUMMY>
__global__ __launch_bounds__(256) void smla_fwd_bf16_persist_kernel(FwdArgs a, const int32_t* __restrict__ nbp) {
  debug_poison_lds();
  constexpr int NW = 4, BT = 32, KT = 2;
  constexpr int NQ = 36;                      // QK MFMAs per block
  constexpr int NPV = 32;                     // PV MFMAs per block
  constexpr int LPB = 9;                      // gather instructions per wave per block
  constexpr int TILE = BT * kRowBytesBf16;
  constexpr int UG = (BT / 8) * 1024;
  constexpr int PF = 12;
  constexpr int PFV = 4;
  constexpr int XS = NW * 64 * 16;
  __shared__ __attribute__((aligned(1024))) char st0[TILE];
  __shared__ __attribute__((aligned(1024))) char st1[TILE];
  __shared__ __attribute__((aligned(1024))) char st2[TILE];
  __shared__ __attribute__((aligned(1024))) char st3[TILE];
  __shared__ __attribute__((aligned(16))) char xs0[XS];
  __shared__ __attribute__((aligned(16))) char xs1[XS];
  __shared__ __attribute__((aligned(16))) float xa0[NW * 16];
  __shared__ __attribute__((aligned(16))) float xa1[NW * 16];
  __shared__ __attribute__((aligned(16))) int ring[4][NW * 64];
  __shared__ __attribute__((aligned(16))) float vbias[4][BT];
  __shared__ float lsh[2][NW * 16];           // running_sumexp of a finished token, by token parity
  __shared__ int sred[4];
  char* const stages[4] = {st0, st1, st2, st3};
  char* const xss[2] = {xs0, xs1};
  float* const xas[2] = {xa0, xa1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int G = gridDim.x, gid = blockIdx.x;

  // ---- this workgroup's run of tokens [T0, T1): token t goes to workgroup
  // floor((C(t) + w(t)/2) · G / W), C(t) the weight of the tokens before t.
  int T0, T1;
  {
    const int per = (a.s_q + 255) / 256;
    const int c0 = min(a.s_q, tid * per), c1 = min(a.s_q, c0 + per);
    int64_t mine = 0;
    for (int t = c0; t < c1; ++t) mine += nbp[t] + kTokenWeight;
    // exclusive scan of the 256 partial weights (wave prefix, then across waves)
    int64_t incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int64_t* wsum = reinterpret_cast<int64_t*>(&ring[0][0]);   // [0..3]: wave totals
    if (lane == 63) wsum[w] = incl;
    if (tid == 0) {
      sred[0] = a.s_q;
      sred[1] = a.s_q;
    }
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int64_t s = wsum[u];
      before += u < w ? s : 0;
      total += s;
    }
    int64_t cum = before + incl - mine;
    int first_mine = a.s_q, first_next = a.s_q;
    for (int t = c0; t < c1; ++t) {
      const int wt = nbp[t] + kTokenWeight;
      const int64_t grp = min((int64_t)G - 1, ((2 * cum + wt) * G) / (2 * total));
      if (grp >= gid && first_mine == a.s_q) first_mine = t;
      if (grp >= gid + 1 && first_next == a.s_q) first_next = t;
      cum += wt;
    }
    if (first_mine < a.s_q) atomicMin(&sred[0], first_mine);
    if (first_next < a.s_q) atomicMin(&sred[1], first_next);
    __syncthreads();
    T0 = uniform(sred[0]);
    T1 = uniform(sred[1]);
  }
  if (T0 >= T1) return;

  auto cur_init = [&](Cursor& c) __attribute__((always_inline)) {
    c.t = T0;
    c.b = 0;
    c.nb = uniform(nbp[T0]);
    c.nbn = T0 + 1 < T1 ? uniform(nbp[T0 + 1]) : 1;
  };
  auto cur_next = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.b == c.nb) {
      ++c.t;
      c.b = 0;
      c.nb = c.nbn;
      c.nbn = c.t + 1 < T1 ? uniform(nbp[c.t + 1]) : 1;
    }
  };
  Cursor cP, cQ, cG, cI;                      // blocks i, i+1, i+3, i+5 of iteration i
  cur_init(cP);
  cur_init(cQ);
  cur_next(cQ);
  cur_init(cG);
  cur_init(cI);
  // stream length: blocks of the run
  int L;
  {
    // (each thread adds the block counts of its tokens inside the run)
    __syncthreads();
    if (tid == 0) sred[2] = 0;
    __syncthreads();
    int mine = 0;
    for (int t = T0 + tid; t < T1; t += 256) mine += nbp[t];
    if (mine) atomicAdd(&sred[2], mine);
    __syncthreads();
    L = uniform(sred[2]);
  }

  const int64_t s_kv = a.s_kv;
  const int topk = a.topk;
  bf16x8 qf[18];
  load_q(a, T0, w * 16 + n, g, qf);
  PipeState st;
#pragma unroll
  for (int t = 0; t < 32; ++t) st.o[t] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
  st.running_max = kNegInf;
  st.running_max_for_softmax = kNegInf;
  st.sumexp = 0.f;
  const LaneOffsets<BT> lofs = lane_offsets<BT>(lane);
  const KvSource<true> src(a.kv, a.kv_window_bytes);
  const int wbase = 2 * UG * w;

  // Index of this lane's gather slot of the block at cursor c (row 8w + lane%8)
  // into ring slot R: a buffer load over the token's index row (a position
  // past the run loads nothing: an empty buffer window).
  auto load_idx = [&](const Cursor& c, auto R) __attribute__((always_inline)) {
    const bool in = c.t < T1;
    const int32_t* irow = a.idx + (int64_t)(in ? c.t : 0) * a.idx_st;
    const __amdgpu_buffer_rsrc_t irs =
        __builtin_amdgcn_make_buffer_rsrc((void*)irow, 0, in ? topk * 4 : 0, 0x00020000);
    const int j = c.b * BT + 8 * w + (lane & 7);
    debug_poison_dma<4>((LDS_AS void*)(&ring[decltype(R)::value][w * 64]));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, (LDS_AS void*)(&ring[decltype(R)::value][w * 64]), 4,
                                             (uint32_t)j * 4u, 0, 0, 0);
  };
  const char* const ring_lane = (const char*)&ring[0][w * 64 + (lane & 7)];
  auto read_idx = [&](auto R) __attribute__((always_inline)) {
    return lds_read_opaque<decltype(R)::value * NW * 64 * 4>(ring_lane);
  };
  // Gather of the block at cursor c into stage s: invalid slots and positions
  // past the run load from outside the window (zeros, no memory traffic).
  struct Gather {
    uint32_t voff;
  };
  auto prepare_gather = [&](Gather& rg, int s, const Cursor& c, int raw) __attribute__((always_inline)) {
    const int j = c.b * BT + 8 * w + (lane & 7);
    const bool valid = c.t < T1 && j < topk && raw >= 0 && (int64_t)raw < s_kv;
    rg.voff = valid ? (uint32_t)raw * (uint32_t)a.kv_row_bytes + (uint32_t)((lane >> 3) << 4) : kDummyOffset;
    if (lane < 8) vbias[s][8 * w + lane] = valid ? 0.f : kNegInf;
  };
  auto issue = [&](const Gather& rg, char* stage, int k) __attribute__((always_inline)) {
    src.load16((LDS_AS void*)(stage + (k * 4 + w) * 1024), rg.voff, nullptr, 128 * k);
  };
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

  // ---- Pᵀ = G·Qᵀ of one block (as in the pipelined kernel)
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
      const float rmax = fmaxf(st.running_max, sm.cur);
      st.running_max = rmax;
      const bool trig = rmax - st.running_max_for_softmax > kRescaleThresLog2;
      sm.any = __ballot(trig) != 0ull;
      const float al = __builtin_amdgcn_exp2f(st.running_max_for_softmax - rmax);
      sm.alpha = sm.any && st.running_max_for_softmax != kNegInf ? al : 1.0f;
      st.running_max_for_softmax = sm.any ? rmax : st.running_max_for_softmax;
      st.sumexp *= sm.alpha;
    } else if constexpr (k == 3 || k == 4) {
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
  auto publish = [&](const Soft& sm, int p) __attribute__((always_inline)) {
    *(LDS_AS bf16x8*)((LDS_AS char*)(LDS_AS void*)xss[p] + (w * 64 + lane) * 16) = sm.s;
    *(LDS_AS float*)((LDS_AS char*)(LDS_AS void*)xas[p] + (w * 16 + n) * 4) = sm.alpha;
  };

  // ---- token switch.  finish_state: the finished token's running_sumexp of
  // this wave's heads goes to lsh[par] (read by every wave after the next
  // barrier) and its lse is kept for the epilogue; the state restarts.
  float ep_lse = kNegInf;
  int ep_token = 0, ep_par = 0, tok_par = 0;
  auto finish_state = [&](int token) __attribute__((always_inline)) {
    const float l = wave_sum16x4(st.sumexp);
    ep_lse = l > 0.f ? (st.running_max_for_softmax + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
    if (g == 0) lsh[tok_par][w * 16 + n] = l;
    ep_token = token;
    ep_par = tok_par;
    tok_par ^= 1;
    st.running_max = kNegInf;
    st.running_max_for_softmax = kNegInf;
    st.sumexp = 0.f;
  };
  // epilogue of token ep_token: normalise this wave's 128 columns of all 64
  // heads, write them and the lse of this wave's heads, and clear the
  // accumulators for the next token
  auto epilogue = [&](bool clear) __attribute__((always_inline)) {
    float inv[NW];
#pragma unroll
    for (int ht = 0; ht < NW; ++ht) {
      const float l = lsh[ep_par][ht * 16 + n];
      inv[ht] = l > 0.f ? 1.0f / l : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int ht = t / 8, dt = 8 * w + t % 8;
      const f32x4 o = pin_agpr(st.o[t]) * inv[ht];
      i32x2 v;
      v[0] = (int)pack2_bf16(o[0], o[1]);
      v[1] = (int)pack2_bf16(o[2], o[3]);
      *(i32x2*)(a.out + (int64_t)ep_token * a.out_st + (int64_t)(ht * 16 + n) * a.out_sh + 16 * dt + 4 * g) = v;
      if (clear) st.o[t] = pin_agpr(f32x4{0.f, 0.f, 0.f, 0.f});
    }
    if (g == 0) a.lse[(int64_t)ep_token * a.lse_st + w * 16 + n] = ep_lse;
  };

  // ---- prologue: indices of blocks 0..3, gathers of blocks 0..2, index of
  // block 4; block 0: QKᵀ and softmax.  Flags of the memory instructions that
  // the next iteration's wait must allow for: q (Q loads), e (epilogue).
  bool ep_due = false;
  {
    Cursor c = cI;
    static_for<0, 4>([&](auto B) __attribute__((always_inline)) {
      load_idx(c, B);
      cur_next(c);
    });
    wait_vm_lgkm0<0>();
    static_for<0, 3>([&](auto B) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::value;
      Gather rg;
      prepare_gather(rg, b, cG, read_idx(B));
#pragma unroll
      for (int k = 0; k < LPB; ++k) issue(rg, stages[b], k);
      cur_next(cG);
    });
    load_idx(c, std::integral_constant<int, 0>{});
    cur_next(c);
    cI = c;                                   // block 5
    wait_vm_lgkm0<2 * LPB + 1>();
    barrier_no_vm_drain();
    f32x4 pacc[2][KT];
    qk(st0, pacc, [&](auto) {});
    // block 0 is its token's last: the next token's Q, now that QKᵀ(0) is
    // done (loaded and waited for here, once per workgroup at most)
    if (cP.b == cP.nb - 1 && cP.t + 1 < T1) {
      load_q(a, cP.t + 1, w * 16 + n, g, qf);
      wait_vm_lgkm0<0>();
    }
    f32x4 bias[KT];
    load_bias(0, bias);
    Soft sm;
    static_for<0, NSOFT>([&](auto K) __attribute__((always_inline)) { soft_step(K, sm, pacc, bias); });
    publish(sm, 0);
  }

  // ---- iteration i (cursors cP, cQ, cG, cI at blocks i, i+1, i+3, i+5)
  // Order of the memory instructions of an iteration: [epilogue stores] index
  // load, QKᵀ (no gathers), [Q loads of a token switch], PV with the block's
  // nine gathers spread over its MFMAs.  The gathers are the youngest, so the
  // wait at the top of the next iteration for all but the last nine
  // instructions covers both the block it needs and a switch's Q loads, on
  // every path: the compiler then sees no load pending into Q and places no
  // wait of its own in the QKᵀ products.
  auto iteration = [&](auto S, int i, auto DYN_) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;     // stage of block i
    constexpr int p = s & 1;
    constexpr bool DYN = decltype(DYN_)::value;
    const bool next = DYN ? i + 1 < L : true;
    // gather(i+1) landed (only the previous iteration's gathers, the nine
    // youngest memory instructions, may still be in flight; loads complete in
    // order, and an epilogue's stores are older and at worst waited for too)
    wait_vm_lgkm0<LPB>();
    barrier_no_vm_drain();
    // block i-1 ended its token: write that token now that every wave's sums
    // are in lsh, before PV(i) accumulates the next token
    if (ep_due) epilogue(true);
    ep_due = false;

    load_idx(cI, std::integral_constant<int, (s + 1) & 3>{});
    Gather rg;
    prepare_gather(rg, (s + 3) & 3, cG, read_idx(std::integral_constant<int, (s + 3) & 3>{}));
    char* const rstage = stages[(s + 3) & 3];
    // gathers [ceil(c·LPB/NPV), ceil((c+1)·LPB/NPV)) follow PV MFMA c
    auto dma_at = [&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value;
      static_for<(c * LPB + NPV - 1) / NPV, ((c + 1) * LPB + NPV - 1) / NPV>([&](auto K) __attribute__((always_inline)) {
        issue(rg, rstage, decltype(K)::value);
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
        if constexpr (q == NQ - 4) load_bias((s + 1) & 3, bias);
        if constexpr (q >= NQ - PF && q < NQ - PF + 2 * PFV && (q - (NQ - PF)) % 2 == 0)
          fetch_v((q - (NQ - PF)) / 2);
      });
      // block i+1 starts a token: the finished token's sums go to the epilogue
      if (cQ.b == 0) finish_state(cP.t);
      // block i+1 ends its token and another follows: that token's Q, now that
      // QKᵀ(i+1) is done with the registers
      if (cQ.b == cQ.nb - 1 && cQ.t + 1 < T1) load_q(a, cQ.t + 1, w * 16 + n, g, qf);
    } else {
      consume_reads();
#pragma unroll
      for (int jj = 0; jj < PFV; ++jj) fetch_v(jj);
    }
    ep_due = next && cQ.b == 0;

    // rescale, then Oᵀ += Vᵀ·Sᵀ with the softmax of block i+1 in between
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
      dma_at(I);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (next) publish(sm, p ^ 1);
    cur_next(cP);
    cur_next(cQ);
    cur_next(cG);
    cur_next(cI);
  };

  using T = std::integral_constant<bool, true>;
  using F = std::integral_constant<bool, false>;
  iteration(std::integral_constant<int, 0>{}, 0, T{});
  int i0 = 1;
  for (; i0 + 4 < L; i0 += 4) {
    iteration(std::integral_constant<int, 1>{}, i0, F{});
    iteration(std::integral_constant<int, 2>{}, i0 + 1, F{});
    iteration(std::integral_constant<int, 3>{}, i0 + 2, F{});
    iteration(std::integral_constant<int, 0>{}, i0 + 3, F{});
  }
  if (i0 < L) {
    iteration(std::integral_constant<int, 1>{}, i0, T{});
    if (i0 + 1 < L) {
      iteration(std::integral_constant<int, 2>{}, i0 + 1, T{});
      if (i0 + 2 < L) {
        iteration(std::integral_constant<int, 3>{}, i0 + 2, T{});
        if (i0 + 3 < L) iteration(std::integral_constant<int, 0>{}, i0 + 3, T{});
      }
    }
  }
  wait_vm_lgkm0<0>();

  // ---- the run's last token (block L-1 ended it; its sums are final)
  finish_state(T1 - 1);
  __syncthreads();
  epilogue(false);
}

}  // namespace

hipError_t launch_bf16_persist(const FwdArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((smla_fwd_bf16_persist_kernel<0>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                     a.token_blocks);
  return hipGetLastError();
}

}  // namespace smla
