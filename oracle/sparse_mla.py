"""float64 oracle of the sparse MLA attention forward pass -- test infrastructure.

Only ``tests/``, the smoke check and the CPU-baseline leg of the benchmark use
this module; the HIP library never does, and nothing here calls the library.

Source: the page "Ascend Sparse Attention Forward 算法与优化技术简析"
(a DeepSeek FlashMLA design note).  Its section 数学建模 (mathematical model)
defines the operation for one query token; tokens are independent.  Its
section 计算流程 (computation flow) gives the block-wise online-softmax
algorithm with the "skip scale" rule.

Readings taken where the page is silent or ambiguous:

* The flow never multiplies P by sm_scale, the definition does.  Both
  functions scale the logits first, x = sm_scale·P, and take every maximum and
  the rescale threshold in units of x.
* RESCALE_THRES is in natural-log units of x: the flow states the rule keeps
  exp(running_max - running_max_for_softmax) at most exp(6).
* A slot whose index is outside [0, s_kv) (the causal workload writes -1) is
  masked: weight zero, row never read.  Duplicate indices are separate slots
  (index_select keeps repeats).
* A token (or row) with no valid slot gets out = 0 and lse = -inf.
* lse is the natural log-sum-exp of the scaled logits, the quantity the
  flow's running_sumexp and running_max_for_softmax encode:
  lse = running_max_for_softmax + ln(running_sumexp).
* running_sumexp adds the S of the current block before its bf16 cast; the
  cast only feeds the product with V.
* "If some row triggers, rescale": every row the decision covers is rescaled
  and its running_max_for_softmax set to running_max.  The decision can cover
  all h_q rows (the page) or groups of rows; in exact arithmetic the result is
  the same either way.
"""
from __future__ import annotations

import numpy as np

# 计算流程, step 3.5: the rescale threshold "typically 6" in the kernel.
RESCALE_THRES = 6.0


def valid_slot_mask(indices: np.ndarray, s_kv: int) -> np.ndarray:
    """True where a slot names a real KV row: 0 <= idx < s_kv."""
    idx = np.asarray(indices)
    return (idx >= 0) & (idx < s_kv)


def _as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sparse_mla_fwd_exact(q, kv, indices, sm_scale, d_v, *, return_weights=False):
    """The definition (section 数学建模), evaluated in float64.

    For each token t (tokens are processed independently):
      gathered_kv = KV.index_select(indices[t])          [n, d_qk]
      P   = Q[t] @ gathered_kv^T                         [h_q, n]
      S   = softmax(P * sm_scale, dim=-1)                [h_q, n]
      out = S @ gathered_kv[:, :d_v]                     [h_q, d_v]
      lse = log(sum_j exp(P * sm_scale))                 [h_q]

    Args:
      q:        [s_q, h_q, d_qk] values (bf16 or other, upcast exactly).
      kv:       [s_kv, d_qk] values (for fp8 caches: already dequantised
                exactly, see ``dequant_fp8_rows``).
      indices:  [s_q, topk] integer row ids; out-of-range ids are masked.
      sm_scale: the float32 softmax scale the kernel receives; it is used as
                exactly that float32 number upcast to float64.
      d_v:      number of leading KV columns that form V.
    Returns (out [s_q, h_q, d_v], lse [s_q, h_q]) in float64, plus the
    per-token weight matrices S if ``return_weights``.
    """
    q = _as_f64(q)
    kv = _as_f64(kv)
    idx = np.asarray(indices)
    s_q, h_q, d_qk = q.shape
    s_kv = kv.shape[0]
    assert kv.shape[1] == d_qk and idx.shape[0] == s_q and 0 < d_v <= d_qk
    scale = float(np.float32(sm_scale))
    valid = valid_slot_mask(idx, s_kv)
    out = np.zeros((s_q, h_q, d_v), dtype=np.float64)
    lse = np.full((s_q, h_q), -np.inf, dtype=np.float64)
    weights = []
    for t in range(s_q):
        sel = idx[t][valid[t]]
        if sel.size == 0:
            weights.append(np.zeros((h_q, 0)))
            continue
        g = kv[sel]                      # index_select: repeats stay repeats
        x = (q[t] @ g.T) * scale         # scaled logits [h_q, n]
        m = x.max(axis=1, keepdims=True)
        w = np.exp(x - m)
        z = w.sum(axis=1, keepdims=True)
        s = w / z
        out[t] = s @ g[:, :d_v]
        lse[t] = (m + np.log(z))[:, 0]
        weights.append(s)
    if return_weights:
        return out, lse, weights
    return out, lse


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest even) -> bfloat16 (round to nearest
    even), returned as float64.  Models a kernel that forms S in float32 and
    casts it to bf16; used only by the optional numerics model below."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    b = ((b + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32).astype(np.float64)


def sparse_mla_fwd_online(q, kv, indices, sm_scale, d_v, *, b_topk=64,
                          rescale_thres=RESCALE_THRES, trigger_rows=None,
                          s_to_bf16=False, return_stats=False):
    """The block-wise algorithm of section 计算流程, in float64.

    Per token: cut the topk slots into blocks of B_TOPK (the last block may be
    short).  Keep running_max, running_max_for_softmax, running_sumexp [h_q]
    (initially -inf, -inf, 0) and out_accum [h_q, d_v] (initially 0).  For each
    block: gather its rows; P = Q @ G^T scaled by sm_scale; cur_max = row max;
    running_max = max(running_max, cur_max); if some row has
    running_max - running_max_for_softmax > RESCALE_THRES, multiply out_accum
    and running_sumexp by exp(running_max_for_softmax - running_max) and set
    running_max_for_softmax = running_max ("skip scale" when no row does);
    then S = exp(x - running_max_for_softmax), out_accum += S @ G[:, :d_v],
    running_sumexp += sum(S).

    ``trigger_rows``: rows that share one rescale decision (consecutive groups
    of that many rows); None means all h_q rows, as on the page.
    ``s_to_bf16``: round S to bf16 before the product with V (the page's cast),
    a numerics model; off by default so that the result is exact.
    Returns (out, lse) and, if ``return_stats``, a dict with the number of
    block steps and of rescale events.
    """
    q = _as_f64(q)
    kv = _as_f64(kv)
    idx = np.asarray(indices)
    s_q, h_q, d_qk = q.shape
    s_kv = kv.shape[0]
    topk = idx.shape[1]
    scale = float(np.float32(sm_scale))
    group = h_q if trigger_rows is None else int(trigger_rows)
    assert h_q % group == 0
    valid = valid_slot_mask(idx, s_kv)
    out = np.zeros((s_q, h_q, d_v))
    lse = np.full((s_q, h_q), -np.inf)
    n_blocks = 0
    n_rescales = 0
    for t in range(s_q):
        running_max = np.full(h_q, -np.inf)
        running_max_for_softmax = np.full(h_q, -np.inf)
        running_sumexp = np.zeros(h_q)
        out_accum = np.zeros((h_q, d_v))
        for k0 in range(0, topk, b_topk):
            blk = idx[t, k0:k0 + b_topk]
            ok = valid[t, k0:k0 + b_topk]
            # step 1: sparse gather; masked slots are not read, their logit is -inf
            g = np.zeros((blk.size, d_qk))
            g[ok] = kv[blk[ok]]
            # step 2: P = Q @ G^T, scaled
            x = (q[t] @ g.T) * scale
            x[:, ~ok] = -np.inf
            # steps 3-4: block row max, running max
            cur_max = x.max(axis=1)
            running_max = np.maximum(running_max, cur_max)
            # step 5: trigger test per decision group
            has = np.isfinite(running_max)
            gap = np.full(h_q, -np.inf)
            gap[has] = running_max[has] - running_max_for_softmax[has]
            trig = (gap > rescale_thres).reshape(-1, group).any(axis=1)
            trig = np.repeat(trig, group)
            # step 6: conditional rescale.  A row that has seen no valid slot
            # keeps its zero state (exp(-inf - (-inf)) is never formed).
            if trig.any():
                n_rescales += int(trig.reshape(-1, group)[:, 0].sum())
                upd = trig & has
                alpha = np.zeros(h_q)
                fin = upd & np.isfinite(running_max_for_softmax)
                alpha[fin] = np.exp(running_max_for_softmax[fin] - running_max[fin])
                out_accum[upd] *= alpha[upd, None]
                running_sumexp[upd] *= alpha[upd]
                running_max_for_softmax[upd] = running_max[upd]
            # step 7: S = exp(x - running_max_for_softmax), accumulate S @ V
            s = np.zeros_like(x)
            live = np.isfinite(running_max_for_softmax)
            s[live] = np.exp(x[live] - running_max_for_softmax[live, None])
            s_pv = round_to_bf16(s) if s_to_bf16 else s
            out_accum += s_pv @ g[:, :d_v]
            # step 8: running_sumexp += S.sum(-1)
            running_sumexp += s.sum(axis=1)
            n_blocks += 1
        nz = running_sumexp > 0
        out[t, nz] = out_accum[nz] / running_sumexp[nz, None]
        lse[t, nz] = running_max_for_softmax[nz] + np.log(running_sumexp[nz])
    if return_stats:
        return out, lse, {"blocks": n_blocks, "rescales": n_rescales}
    return out, lse


def lse_combine(outs, lses):
    """Merge partial results of disjoint slot sets.

    ``outs`` [n, ..., d_v] are the normalised partial outputs and ``lses``
    [n, ...] their log-sum-exps.  With Z_s = exp(lse_s):
      lse = ln(sum_s Z_s),  out = sum_s (Z_s / Z) * out_s.
    A part with lse_s = -inf (no valid slot) has weight 0; if every part is
    empty the result is out = 0, lse = -inf.
    """
    outs = _as_f64(outs)
    lses = _as_f64(lses)
    m = lses.max(axis=0)
    fin = np.isfinite(m)
    safe_m = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_m[None]), 0.0)
    z = w.sum(axis=0)
    lse = np.where(fin, safe_m + np.log(np.where(fin, z, 1.0)), -np.inf)
    wn = np.where(fin[None], w / np.where(fin, z, 1.0)[None], 0.0)
    out = (wn[..., None] * outs).sum(axis=0)
    return out, lse


def split_bounds(topk: int, num_splits: int):
    """Contiguous, near-equal parts [lo, hi) of the topk slots."""
    per = -(-topk // num_splits)
    return [(min(s * per, topk), min((s + 1) * per, topk)) for s in range(num_splits)]


def sparse_mla_fwd_split(q, kv, indices, sm_scale, d_v, *, num_splits, **online_kw):
    """Split-topk evaluation: each contiguous part of every token's slots runs
    the block-wise algorithm on its own, then ``lse_combine`` merges them."""
    idx = np.asarray(indices)
    parts_o, parts_l = [], []
    for lo, hi in split_bounds(idx.shape[1], num_splits):
        o, l = sparse_mla_fwd_online(q, kv, idx[:, lo:hi], sm_scale, d_v, **online_kw)
        parts_o.append(o)
        parts_l.append(l)
    return lse_combine(np.stack(parts_o), np.stack(parts_l))
