"""Seeded synthetic inputs for the sparse MLA attention forward pass.

This is the one module that both the HIP path (tests, benchmark) and the CPU
oracle consume.  It only draws random numbers and lays them out; it holds
none of the method's arithmetic.  All tensors are returned on the CPU.

Random numbers come from ``numpy.random.default_rng(seed)`` (PCG64), drawn in
the order Q, KV, indices.  Q and KV are N(0, 1) float32 rounded to bf16 (round
to nearest even, torch's cast).  The five named workloads:

* ``tiny``:       4 tokens, h_q 16, topk 128, s_kv 2048.
* ``prefill``:    4096 tokens, h_q 64, topk 2048, one shared KV of 65536 rows;
                  each token's indices uniform without replacement.
* ``causal``:     8192 tokens at positions 0..8191, h_q 64, topk 2048,
                  s_kv 8192; token t draws without replacement from [0, t],
                  slots past t+1 hold -1 (masked); Q is scaled by 4 (exact in
                  bf16) so that rescales happen often.
* ``decode``:     64 sequences x 1 token, h_q 128, topk 512, 32768 KV rows per
                  sequence stacked into one [64*32768, 576] tensor; indices are
                  global row ids inside the token's own sequence; 4 splits.
* ``decode_paged``: the ``decode`` shapes over a paged KV cache: pages of 64
                  rows, the 32768 pages of the pool dealt to the 64 sequences in
                  a random order (each sequence's block table lists its 512
                  pages); indices are logical positions in [0, 32768).
* ``decode_fp4``: as ``decode_fp8`` with an FP4 (E2M1) cache: one float32
                  scale per 128-column group (scale = absmax / 6, code = the
                  nearest E2M1 value of value / scale, ties to the even
                  mantissa).
* ``decode_fp8``: 128 sequences x 1 token, h_q 64, topk 2048, 16384 rows per
                  sequence, KV quantised to FP8 E4M3 with one float32 scale per
                  128-column group of each row (scale = absmax / 448, code =
                  round-to-nearest-even E4M3 of value / scale).

The page "Ascend Sparse Attention Forward 算法与优化技术简析" measures on
"DeepSeek v4.1 typical conditions" without stating shapes; these workloads
stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

D_QK = 576
D_V = 512
FP8_GROUP = 128
FP8_MAX = 448.0
FP4_MAX = 6.0
# E2M1 magnitudes of codes 0..7 and the midpoints between neighbours
_FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_FP4_MID = (_FP4_GRID[1:] + _FP4_GRID[:-1]) / 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    s_q: int
    h_q: int
    topk: int
    s_kv: int
    seqs: int = 1            # decode: number of sequences (one token each)
    rows_per_seq: int = 0    # decode: KV rows per sequence
    causal: bool = False
    q_mult: float = 1.0
    kv_format: str = "bf16"  # "bf16", "fp8" or "fp4"
    num_splits: int = 1      # split-topk parts the workload asks for (0: auto)
    page_size: int = 0       # paged KV: rows per page (0: not paged)
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(D_QK)))

    @property
    def valid_slots(self) -> int:
        if self.causal:
            return sum(min(t + 1, self.topk) for t in range(self.s_q))
        return self.s_q * self.topk

    @property
    def flops(self) -> float:
        """2·h_q·(d_qk + d_v) per valid slot: QK^T and PV multiply-adds."""
        return 2.0 * self.h_q * (D_QK + D_V) * self.valid_slots


WORKLOADS = {
    "tiny": Workload("tiny", s_q=4, h_q=16, topk=128, s_kv=2048, seed=1),
    "prefill": Workload("prefill", s_q=4096, h_q=64, topk=2048, s_kv=65536, seed=2),
    "causal": Workload("causal", s_q=8192, h_q=64, topk=2048, s_kv=8192, causal=True,
                       q_mult=4.0, seed=3),
    "decode": Workload("decode", s_q=64, h_q=128, topk=512, s_kv=64 * 32768, seqs=64,
                       rows_per_seq=32768, num_splits=4, seed=4),
    "decode_paged": Workload("decode_paged", s_q=64, h_q=128, topk=512, s_kv=64 * 32768, seqs=64,
                             rows_per_seq=32768, num_splits=4, page_size=64, seed=6),
    "decode_fp8": Workload("decode_fp8", s_q=128, h_q=64, topk=2048, s_kv=128 * 16384,
                           seqs=128, rows_per_seq=16384, kv_format="fp8", num_splits=0,
                           seed=5),
    "decode_fp4": Workload("decode_fp4", s_q=128, h_q=64, topk=2048, s_kv=128 * 16384,
                           seqs=128, rows_per_seq=16384, kv_format="fp4", num_splits=0,
                           seed=7),
}


def _normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bf16, generated in row chunks to bound
    host memory for multi-GB KV tensors."""
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = torch.empty((rows, inner), dtype=torch.bfloat16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, inner), dtype=np.float32)
        out[r0:r1] = torch.from_numpy(x).to(torch.bfloat16)
    return out.reshape(shape)


def _normal_fp8_groups(rng: np.random.Generator, rows: int, cols: int,
                       chunk_rows: int = 1 << 16):
    """N(0,1) float32 rows quantised per 128-column group to E4M3 codes plus a
    float32 scale per group (scale = absmax / 448)."""
    ng = -(-cols // FP8_GROUP)
    codes = torch.empty((rows, cols), dtype=torch.uint8)
    scales = torch.empty((rows, ng), dtype=torch.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.from_numpy(rng.standard_normal((r1 - r0, cols), dtype=np.float32))
        for g in range(ng):
            c0, c1 = g * FP8_GROUP, min(cols, (g + 1) * FP8_GROUP)
            xs = x[:, c0:c1]
            amax = xs.abs().amax(dim=1)
            sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            y = (xs / sc[:, None]).clamp_(-FP8_MAX, FP8_MAX)
            codes[r0:r1, c0:c1] = y.to(torch.float8_e4m3fn).view(torch.uint8)
            scales[r0:r1, g] = sc
    return codes, scales


def _normal_fp4_groups(rng: np.random.Generator, rows: int, cols: int,
                       chunk_rows: int = 1 << 16):
    """N(0,1) float32 rows quantised per 128-column group to E2M1 codes (one
    4-bit code per byte: bit 3 sign, bits 2..0 the magnitude index) plus a
    float32 scale per group (scale = absmax / 6); the code is the nearest E2M1
    value of value / scale, ties to the even mantissa."""
    ng = -(-cols // FP8_GROUP)
    codes = torch.empty((rows, cols), dtype=torch.uint8)
    scales = torch.empty((rows, ng), dtype=torch.float32)
    mids = torch.from_numpy(_FP4_MID)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.from_numpy(rng.standard_normal((r1 - r0, cols), dtype=np.float32))
        for g in range(ng):
            c0, c1 = g * FP8_GROUP, min(cols, (g + 1) * FP8_GROUP)
            xs = x[:, c0:c1]
            amax = xs.abs().amax(dim=1)
            sc = torch.where(amax > 0, amax / np.float32(FP4_MAX), torch.ones_like(amax))
            a = (xs / sc[:, None]).abs().to(torch.float64).clamp_(max=FP4_MAX)
            mag = torch.bucketize(a, mids, right=False)      # nearest; a tie takes the lower
            tie_up = (mag < 7) & (a == mids[mag.clamp(max=6)]) & (mag % 2 == 1)
            mag = (mag + tie_up.to(mag.dtype)).to(torch.uint8)   # ties to the even mantissa
            codes[r0:r1, c0:c1] = mag | torch.where((xs < 0) & (mag > 0), 8, 0).to(torch.uint8)
            scales[r0:r1, g] = sc
    return codes, scales


def _indices(rng: np.random.Generator, w: Workload) -> np.ndarray:
    idx = np.full((w.s_q, w.topk), -1, dtype=np.int32)
    if w.causal:
        for t in range(w.s_q):
            n = t + 1
            if n <= w.topk:
                idx[t, :n] = rng.permutation(n)
            else:
                idx[t] = rng.choice(n, w.topk, replace=False)
    elif w.page_size:
        for b in range(w.s_q):               # logical positions in the sequence
            idx[b] = rng.choice(w.rows_per_seq, w.topk, replace=False)
    elif w.seqs > 1:
        for b in range(w.s_q):
            idx[b] = b * w.rows_per_seq + rng.choice(w.rows_per_seq, w.topk, replace=False)
    else:
        for t in range(w.s_q):
            idx[t] = rng.choice(w.s_kv, w.topk, replace=False)
    return idx


def make_inputs(w: Workload | str, seed: int | None = None) -> dict:
    """Materialise a workload on the CPU.

    Returns a dict with ``q`` (bf16 [s_q, h_q, 576]), ``indices`` (int32
    [s_q, topk]), ``sm_scale`` (float), ``d_v`` (512), and either ``kv`` (bf16
    [s_kv, 576]) or ``kv_codes`` (uint8 [s_kv, 576]) with ``kv_scales``
    (float32 [s_kv, 5]) for the fp8 workload.  Paged workloads add
    ``block_table`` (int32 [s_q, pages per sequence]) and ``page_size``; their
    ``kv`` is the page pool, rows of page p at [p * page_size, (p+1) * page_size).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _normal_bf16(rng, (w.s_q, w.h_q, D_QK))
    if w.q_mult != 1.0:
        q = (q.float() * w.q_mult).to(torch.bfloat16)
    out = {"workload": w, "q": q, "sm_scale": w.sm_scale, "d_v": D_V}
    if w.kv_format == "fp8":
        out["kv_codes"], out["kv_scales"] = _normal_fp8_groups(rng, w.s_kv, D_QK)
    elif w.kv_format == "fp4":
        out["kv_codes"], out["kv_scales"] = _normal_fp4_groups(rng, w.s_kv, D_QK)
    else:
        out["kv"] = _normal_bf16(rng, (w.s_kv, D_QK))
    out["kv_format"] = w.kv_format
    out["indices"] = torch.from_numpy(_indices(rng, w))
    if w.page_size:
        # the pool's pages dealt to the sequences in a random order
        per = w.rows_per_seq // w.page_size
        perm = rng.permutation(w.s_kv // w.page_size).astype(np.int32)
        out["block_table"] = torch.from_numpy(perm[: w.s_q * per].reshape(w.s_q, per).copy())
        out["page_size"] = w.page_size
    return out


def make_random(*, s_q: int, h_q: int, topk: int, s_kv: int, seed: int,
                d_qk: int = D_QK, invalid_frac: float = 0.0, dup_frac: float = 0.0,
                q_mult: float = 1.0, kv_format: str = "bf16") -> dict:
    """Small seeded cases for parity and edge tests.

    Indices are uniform over [0, s_kv) with replacement unless ``dup_frac`` is
    0 and topk <= s_kv (then without).  ``invalid_frac`` of the slots, chosen
    at random, get an out-of-range id (-1, s_kv, or a large negative value);
    ``dup_frac`` of the slots copy another slot of the same token.
    """
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (s_q, h_q, d_qk))
    if q_mult != 1.0:
        q = (q.float() * q_mult).to(torch.bfloat16)
    res = {"q": q, "sm_scale": float(np.float32(1.0 / math.sqrt(d_qk))), "d_v": D_V,
           "kv_format": kv_format}
    if kv_format == "fp8":
        res["kv_codes"], res["kv_scales"] = _normal_fp8_groups(rng, s_kv, d_qk)
    elif kv_format == "fp4":
        res["kv_codes"], res["kv_scales"] = _normal_fp4_groups(rng, s_kv, d_qk)
    else:
        res["kv"] = _normal_bf16(rng, (s_kv, d_qk))
    idx = np.empty((s_q, topk), dtype=np.int64)
    for t in range(s_q):
        if topk <= s_kv and dup_frac == 0.0:
            idx[t] = rng.choice(s_kv, topk, replace=False)
        else:
            idx[t] = rng.integers(0, s_kv, topk)
    if dup_frac > 0:
        m = rng.random((s_q, topk)) < dup_frac
        src = rng.integers(0, topk, (s_q, topk))
        idx = np.where(m, np.take_along_axis(idx, src, axis=1), idx)
    if invalid_frac > 0:
        m = rng.random((s_q, topk)) < invalid_frac
        bad = rng.choice(np.array([-1, s_kv, -(2 ** 31), 2 ** 31 - 1], dtype=np.int64),
                         (s_q, topk))
        idx = np.where(m, bad, idx)
    res["indices"] = torch.from_numpy(idx.astype(np.int32))
    return res


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/float32 tensor (for the oracle)."""
    return t.to(torch.float64).numpy()


def make_random_paged(*, s_q: int, h_q: int, topk: int, page_size: int, num_pages: int,
                      table_width: int, seed: int, unallocated_frac: float = 0.0,
                      invalid_frac: float = 0.0, kv_format: str = "bf16") -> dict:
    """Small seeded paged cases: a pool of ``num_pages`` pages of ``page_size``
    rows (``kv`` or ``kv_codes``/``kv_scales`` of num_pages * page_size rows),
    a block table of random pages (repeats across and within tokens allowed),
    ``unallocated_frac`` of its entries -1, and logical indices uniform over
    [0, table_width * page_size) with ``invalid_frac`` of them out of range."""
    rng = np.random.default_rng(seed)
    res = make_random(s_q=s_q, h_q=h_q, topk=1, s_kv=num_pages * page_size, seed=seed,
                      kv_format=kv_format)
    table = rng.integers(0, num_pages, (s_q, table_width)).astype(np.int32)
    if unallocated_frac > 0:
        table[rng.random((s_q, table_width)) < unallocated_frac] = -1
    n = table_width * page_size
    idx = rng.integers(0, n, (s_q, topk)).astype(np.int64)
    if invalid_frac > 0:
        m = rng.random((s_q, topk)) < invalid_frac
        idx = np.where(m, rng.choice(np.array([-1, n, n + 5, -(2 ** 31)], dtype=np.int64), (s_q, topk)), idx)
    res["indices"] = torch.from_numpy(idx.astype(np.int32))
    res["block_table"] = torch.from_numpy(table)
    res["page_size"] = page_size
    return res
