"""Pins for the CPU oracle (no GPU).

The oracle is trusted only through checks that do not retype it: brute force
along a different algebraic route, a library attention routine on the dense
special case, closed forms, invariants, the page's printed cost table, and
the OCP E4M3 definition against torch's fp8 conversion.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import (RESCALE_THRES, dequant_fp4_rows, dequant_fp8_rows, e2m1_decode, e4m3fn_decode,
                    lse_combine,
                    sparse_mla_fwd_exact, sparse_mla_fwd_online, sparse_mla_fwd_split)
from oracle.cost_model import cost_model_cycles
from oracle.paged import sparse_mla_fwd_paged
from oracle.sparse_mla import round_to_bf16, split_bounds
import workloads

GOLDEN = __file__.rsplit("/", 1)[0] + "/golden"


def _rand_case(seed, s_q=3, h_q=4, d_qk=12, d_v=7, s_kv=9, topk=10, invalid=0.2, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((s_q, h_q, d_qk)) * scale
    kv = rng.standard_normal((s_kv, d_qk))
    idx = rng.integers(0, s_kv, (s_q, topk))          # with repeats
    bad = rng.random((s_q, topk)) < invalid
    idx = np.where(bad, rng.choice([-1, s_kv, -7, s_kv + 3], (s_q, topk)), idx)
    return q, kv, idx, 0.37, d_v


def _brute(q, kv, idx, sm_scale, d_v):
    """Pure-Python loops, softmax weights as 1 / sum_k exp(x_k - x_j) and the
    log-sum-exp through math.fsum: a different route from the oracle's
    max-shifted matrix form."""
    s_q, h_q, d_qk = q.shape
    s_kv = kv.shape[0]
    scale = float(np.float32(sm_scale))
    out = np.zeros((s_q, h_q, d_v))
    lse = np.full((s_q, h_q), -math.inf)
    for t in range(s_q):
        rows = [int(r) for r in idx[t] if 0 <= r < s_kv]
        if not rows:
            continue
        for h in range(h_q):
            xs = [scale * math.fsum(float(q[t, h, d]) * float(kv[r, d]) for d in range(d_qk))
                  for r in rows]
            ws = [1.0 / math.fsum(math.exp(xk - xj) for xk in xs) for xj in xs]
            for c in range(d_v):
                out[t, h, c] = math.fsum(w * float(kv[r, c]) for w, r in zip(ws, rows))
            lse[t, h] = math.log(math.fsum(math.exp(x) for x in xs))
    return out, lse


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_matches_brute_force(seed):
    q, kv, idx, sc, d_v = _rand_case(seed)
    idx[1] = -1                                       # one fully masked token
    o, l = sparse_mla_fwd_exact(q, kv, idx, sc, d_v)
    ob, lb = _brute(q, kv, idx, sc, d_v)
    assert np.allclose(o, ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isinf(l), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.allclose(l[fin], lb[fin], rtol=0, atol=1e-12)
    assert np.all(o[1] == 0) and np.all(l[1] == -np.inf)


def test_dense_case_matches_torch_sdpa():
    """indices = all rows in order reduces the method to ordinary attention of
    h_q queries over s_kv keys with V = the first d_v key columns."""
    rng = np.random.default_rng(5)
    s_q, h_q, d_qk, d_v, s_kv = 3, 8, 40, 24, 33
    q = rng.standard_normal((s_q, h_q, d_qk))
    kv = rng.standard_normal((s_kv, d_qk))
    idx = np.tile(np.arange(s_kv), (s_q, 1))
    sc = float(np.float32(1 / math.sqrt(d_qk)))
    o, l = sparse_mla_fwd_exact(q, kv, idx, sc, d_v)
    qt = torch.from_numpy(q)                             # [s_q, h_q, d] as batch of queries
    k = torch.from_numpy(kv).expand(s_q, s_kv, d_qk)
    v = torch.from_numpy(kv[:, :d_v]).expand(s_q, s_kv, d_v)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=sc)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    lref = torch.logsumexp(qt @ k.transpose(1, 2) * sc, dim=-1)
    assert np.allclose(l, lref.numpy(), rtol=0, atol=1e-12)


def test_topk_one_is_a_copy():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 3, 16))
    kv = rng.standard_normal((5, 16))
    idx = np.array([[3], [0]])
    o, l = sparse_mla_fwd_exact(q, kv, idx, 0.5, 10)
    for t in range(2):
        assert np.array_equal(o[t], np.broadcast_to(kv[idx[t, 0], :10], (3, 10)))
        assert np.allclose(l[t], 0.5 * (q[t] @ kv[idx[t, 0]]), rtol=0, atol=1e-13)


def test_zero_query_is_mean_of_valid_rows():
    rng = np.random.default_rng(3)
    kv = rng.standard_normal((6, 8))
    idx = np.array([[0, 2, 2, -1, 5, 9]])            # 2 counted twice, -1 and 9 masked
    o, l = sparse_mla_fwd_exact(np.zeros((1, 2, 8)), kv, idx, 1.0, 4)
    mean = (kv[0] + 2 * kv[2] + kv[5])[:4] / 4
    assert np.allclose(o[0], mean, rtol=0, atol=1e-15)
    assert np.allclose(l[0], math.log(4), rtol=0, atol=1e-15)


@pytest.mark.parametrize("a,b", [(0.0, 1.0), (2.5, -3.0), (30.0, 29.5)])
def test_two_slots_are_a_logistic_mix(a, b):
    kv = np.zeros((2, 4))
    kv[0, 0] = 1.0
    kv[1, 1] = 1.0
    kv[0, 2], kv[1, 2] = 3.0, -5.0
    q = np.array([[[a, b, 0.0, 0.0]]])
    o, l = sparse_mla_fwd_exact(q, kv, np.array([[0, 1]]), 1.0, 3)
    w0 = 1.0 / (1.0 + math.exp(b - a))
    assert np.allclose(o[0, 0], [w0, 1 - w0, 3 * w0 - 5 * (1 - w0)], rtol=0, atol=1e-14)
    assert math.isclose(l[0, 0], max(a, b) + math.log1p(math.exp(-abs(a - b))), abs_tol=1e-13)


def test_all_slots_one_row():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 5, 20))
    kv = rng.standard_normal((7, 20))
    k = 37
    o, l = sparse_mla_fwd_exact(q, kv, np.full((1, k), 4), 0.25, 11)
    assert np.allclose(o[0], np.broadcast_to(kv[4, :11], (5, 11)), rtol=0, atol=1e-14)
    assert np.allclose(l[0], 0.25 * (q[0] @ kv[4]) + math.log(k), rtol=0, atol=1e-13)


def test_invariants_permutation_masking_weights():
    q, kv, idx, sc, d_v = _rand_case(7, invalid=0.0)
    o, l, ws = sparse_mla_fwd_exact(q, kv, idx, sc, d_v, return_weights=True)
    for w in ws:
        assert np.all(w >= 0) and np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    perm = np.random.default_rng(0).permutation(idx.shape[1])
    o2, l2 = sparse_mla_fwd_exact(q, kv, idx[:, perm], sc, d_v)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13)
    padded = np.concatenate([idx, np.full((idx.shape[0], 5), -1),
                             np.full((idx.shape[0], 3), kv.shape[0])], axis=1)
    o3, l3 = sparse_mla_fwd_exact(q, kv, padded, sc, d_v)
    assert np.array_equal(o, o3) and np.array_equal(l, l3)
    lo = kv[:, :d_v].min(axis=0)
    hi = kv[:, :d_v].max(axis=0)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


@pytest.mark.parametrize("b_topk,group,mult", [(64, None, 1.0), (96, None, 4.0),
                                               (128, 16, 4.0), (7, 1, 8.0), (3, 2, 1.0)])
def test_online_skip_scale_equals_exact(b_topk, group, mult):
    rng = np.random.default_rng(11)
    s_q, h_q, d = 3, 16, 32
    q = rng.standard_normal((s_q, h_q, d)) * mult
    kv = rng.standard_normal((300, d))
    idx = rng.integers(0, 300, (s_q, 257))
    idx[0, :100] = -1                                   # leading masked run
    idx[2, 5::9] = 300                                  # scattered masked slots
    o, l = sparse_mla_fwd_exact(q, kv, idx, 0.2, 24)
    o2, l2, st = sparse_mla_fwd_online(q, kv, idx, 0.2, 24, b_topk=b_topk,
                                       trigger_rows=group, return_stats=True)
    assert np.allclose(o, o2, rtol=0, atol=1e-12)
    assert np.allclose(l, l2, rtol=0, atol=1e-12)
    assert st["rescales"] >= s_q                         # every token triggers at least once


def test_skip_scale_rescales_more_with_larger_logits():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 16, 64))
    kv = rng.standard_normal((4096, 64))
    idx = np.stack([rng.permutation(4096)[:2048] for _ in range(4)])
    counts = []
    for mult in (1.0, 4.0):
        _, _, st = sparse_mla_fwd_online(q * mult, kv, idx, 1 / 8, 32, b_topk=64,
                                         return_stats=True)
        counts.append(st["rescales"])
    assert counts[1] > counts[0] >= 4
    # threshold 0: rescale whenever a max grows; still exact
    o, l = sparse_mla_fwd_exact(q * 4, kv, idx, 1 / 8, 32)
    o2, l2 = sparse_mla_fwd_online(q * 4, kv, idx, 1 / 8, 32, b_topk=64, rescale_thres=0.0)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)


def test_online_all_masked_and_late_first_valid():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 4, 8))
    kv = rng.standard_normal((10, 8))
    idx = np.full((2, 40), -1)
    idx[1, 39] = 3                                      # only the very last slot is valid
    o, l = sparse_mla_fwd_online(q, kv, idx, 1.0, 5, b_topk=8)
    assert np.all(o[0] == 0) and np.all(l[0] == -np.inf)
    assert np.allclose(o[1], np.broadcast_to(kv[3, :5], (4, 5)), atol=1e-15)
    assert np.allclose(l[1], q[1] @ kv[3], atol=1e-14)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 40])
def test_split_combine_equals_exact(n):
    q, kv, idx, sc, d_v = _rand_case(21, s_q=4, topk=33, invalid=0.3, scale=3.0)
    idx[3, :20] = -1                                    # some splits of token 3 are empty
    o, l = sparse_mla_fwd_exact(q, kv, idx, sc, d_v)
    o2, l2 = sparse_mla_fwd_split(q, kv, idx, sc, d_v, num_splits=n, b_topk=5)
    assert np.allclose(o, o2, rtol=0, atol=1e-12)
    assert np.array_equal(np.isinf(l), np.isinf(l2))
    assert np.allclose(l[np.isfinite(l)], l2[np.isfinite(l2)], rtol=0, atol=1e-12)
    bounds = split_bounds(33, n)
    assert bounds[0][0] == 0 and bounds[-1][1] == 33
    assert all(a[1] == b[0] for a, b in zip(bounds, bounds[1:]))


def test_lse_combine_weights():
    outs = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[5.0, 5.0]]])
    lses = np.array([[math.log(1.0)], [math.log(3.0)], [-math.inf]])
    o, l = lse_combine(outs, lses)
    assert np.allclose(o, [[0.25, 0.75]], atol=1e-15)
    assert np.allclose(l, [math.log(4.0)], atol=1e-15)
    o, l = lse_combine(outs[2:], lses[2:])
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_e4m3fn_decode_spec_values():
    v = e4m3fn_decode(np.array([0x7E, 0x08, 0x01, 0x07, 0x38, 0x80, 0xFE], dtype=np.uint8))
    assert list(v[:5]) == [448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 1.0]
    assert v[5] == 0 and math.copysign(1, v[5]) == -1 and v[6] == -448.0


def test_dequant_fp8_rows_groups():
    codes = np.full((2, 576), 0x38, dtype=np.uint8)            # every code is 1.0
    scales = np.array([[1, 2, 3, 4, 5], [0.5, 0.25, 8, 16, 2 ** -10]], dtype=np.float32)
    v = dequant_fp8_rows(codes, scales)
    for g, (c0, c1) in enumerate([(0, 128), (128, 256), (256, 384), (384, 512), (512, 576)]):
        assert np.all(v[:, c0:c1] == scales[:, g:g + 1].astype(np.float64))


def test_round_to_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000) * np.exp(
        np.random.default_rng(1).uniform(-20, 20, 100000))
    mine = round_to_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_cost_model_reproduces_page_table():
    rows = [list(map(int, ln.split())) for ln in open(GOLDEN + "/ascend_cost_model.txt")
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 8
    for h_q, topk, cube, mem in rows:
        c, m = cost_model_cycles(h_q, topk, 512, 4096, 5e12, 32, 1650e6)
        assert c == cube and round(m) == mem


def test_workload_generators_are_seeded_and_shaped():
    a = workloads.make_inputs("tiny")
    b = workloads.make_inputs("tiny")
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["kv"], b["kv"])
    assert torch.equal(a["indices"], b["indices"])
    assert a["q"].shape == (4, 16, 576) and a["q"].dtype == torch.bfloat16
    assert a["kv"].shape == (2048, 576) and a["indices"].shape == (4, 128)
    idx = a["indices"].numpy()
    assert all(len(set(r)) == 128 for r in idx) and idx.min() >= 0 and idx.max() < 2048
    assert a["sm_scale"] == float(np.float32(1 / 24))
    w = workloads.WORKLOADS["causal"]
    assert w.valid_slots == sum(min(t + 1, 2048) for t in range(8192)) == 14681088


def test_causal_generator_structure_small():
    w = workloads.Workload("c", s_q=70, h_q=16, topk=32, s_kv=70, causal=True, q_mult=4.0, seed=9)
    x = workloads.make_inputs(w)
    idx = x["indices"].numpy()
    for t in range(70):
        n = min(t + 1, 32)
        assert np.all(idx[t, n:] == -1)
        assert len(set(idx[t, :n])) == n and idx[t, :n].max() <= t and idx[t, :n].min() >= 0
    q1 = workloads.make_inputs(w)["q"]
    assert torch.equal(x["q"], q1)


def test_fp8_generator_dequantises_close_to_normal_draws():
    x = workloads.make_random(s_q=1, h_q=16, topk=4, s_kv=64, seed=3, kv_format="fp8")
    codes, scales = x["kv_codes"].numpy(), x["kv_scales"].numpy()
    v = dequant_fp8_rows(codes, scales)
    assert np.isfinite(v).all()
    for g in range(5):
        blk = np.abs(v[:, g * 128:(g + 1) * 128])
        assert np.allclose(blk.max(axis=1), 448 * scales[:, g].astype(np.float64), rtol=1e-6)


def test_online_bf16_numerics_model_is_within_tolerance():
    """The S->bf16 cast of the flow changes out by far less than the parity
    tolerance 2e-2·max|out| and leaves lse untouched (lse uses fp32/fp64 S)."""
    x = workloads.make_inputs("tiny")
    q, kv, idx = workloads.to_f64(x["q"]), workloads.to_f64(x["kv"]), x["indices"].numpy()
    o, l = sparse_mla_fwd_exact(q, kv, idx, x["sm_scale"], 512)
    o2, l2 = sparse_mla_fwd_online(q, kv, idx, x["sm_scale"], 512, b_topk=64, s_to_bf16=True)
    err = np.abs(o - o2).max() / np.abs(o).max()
    assert 0 < err < 2e-3
    assert np.allclose(l, l2, atol=1e-12)


# ---- paged KV cache (page "Flash Attention Infer算子性能优化", section
# 优化Paged Attention路径): logical position j of token t is row j % page_size
# of page block_table[t, j // page_size].

def _paged_case(seed, s_q=4, h_q=3, d_qk=10, d_v=6, page_size=3, num_pages=7, width=4, topk=9):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((s_q, h_q, d_qk))
    pages = rng.standard_normal((num_pages, page_size, d_qk))
    # pages shared between tokens, unallocated blocks (-1, num_pages + 2)
    table = rng.integers(0, num_pages, (s_q, width))
    table[0, 1] = -1
    if s_q > 2:
        table[2, 3] = num_pages + 2
    idx = rng.integers(-2, width * page_size + 2, (s_q, topk))
    return q, pages, table, idx, 0.41, d_v


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_paged_matches_brute_force_on_translated_rows(seed):
    """Brute force along another route: translate every logical index to a
    physical row of the flattened page pool with scalar Python arithmetic,
    then the plain loops of _brute over the pool."""
    q, pages, table, idx, sc, d_v = _paged_case(seed)
    num_pages, ps, d_qk = pages.shape
    width = table.shape[1]
    phys = np.full(idx.shape, -1, dtype=np.int64)
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            v = int(idx[t, j])
            if 0 <= v < width * ps:
                page = int(table[t, v // ps])
                if 0 <= page < num_pages:
                    phys[t, j] = page * ps + v % ps
    ob, lb = _brute(q, pages.reshape(-1, d_qk), phys, sc, d_v)
    o, l = sparse_mla_fwd_paged(q, pages, table, idx, sc, d_v)
    assert np.allclose(o, ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isinf(l), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.allclose(l[fin], lb[fin], rtol=0, atol=1e-12)


def test_paged_identity_table_is_the_flat_cache():
    q, kv, idx, sc, d_v = _rand_case(5, s_kv=12, invalid=0.3)
    ps = 4
    pages = kv.reshape(3, ps, kv.shape[1])
    table = np.tile(np.arange(3), (q.shape[0], 1))
    o, l = sparse_mla_fwd_paged(q, pages, table, idx, sc, d_v)
    oe, le = sparse_mla_fwd_exact(q, kv, idx, sc, d_v)
    assert np.array_equal(o, oe) and np.array_equal(l, le)


def test_paged_result_ignores_where_pages_live():
    """Moving the physical pages and rewriting the table accordingly leaves
    every output unchanged."""
    q, pages, table, idx, sc, d_v = _paged_case(9)
    perm = np.random.default_rng(1).permutation(pages.shape[0])
    moved = np.empty_like(pages)
    moved[perm] = pages                              # page p now lives at perm[p]
    ok = (table >= 0) & (table < pages.shape[0])
    table2 = np.where(ok, perm[np.clip(table, 0, pages.shape[0] - 1)], table)
    a = sparse_mla_fwd_paged(q, pages, table, idx, sc, d_v)
    b = sparse_mla_fwd_paged(q, moved, table2, idx, sc, d_v)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_paged_unallocated_block_and_one_row():
    """All valid slots name logical row r: out = V[r] exactly and
    lse = x_r + ln(count); slots into an unallocated block or past the table
    change nothing."""
    q, pages, table, idx, sc, d_v = _paged_case(4, s_q=1)
    ps = pages.shape[1]
    table[0] = [2, -1, 5, 0]
    r = 2 * ps + 1                                   # logical row in page 5
    idx[0] = [r, r, ps, ps + 2, r, 4 * ps, -1, r, r]  # ps.. in the unallocated block
    o, l = sparse_mla_fwd_paged(q, pages, table, idx, sc, d_v)
    v = pages[5, 1]
    assert np.allclose(o[0], np.broadcast_to(v[:d_v], o[0].shape), rtol=0, atol=1e-13)
    x = float(np.float32(sc)) * (q[0] @ v)
    assert np.allclose(l[0], x + math.log(5), rtol=0, atol=1e-12)


# ---- fp4 (OCP MX E2M1) KV-cache values

def test_e2m1_decode_spec_values():
    """The OCP MX specification's E2M1 figures: exponent bias 1, max normal
    6.0, min normal 1.0, the one subnormal 0.5, signed zeros; the eight
    magnitudes increase with the code and bit 3 is the sign."""
    v = e2m1_decode(np.arange(16))
    assert v[7] == 6.0 and v[2] == 1.0 and v[1] == 0.5 and v[0] == 0.0
    assert np.array_equal(v[8:], -v[:8]) and np.signbit(v[8]) and not np.signbit(v[0])
    assert np.all(np.diff(v[:8]) > 0)
    assert sorted(set(np.abs(v).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    with pytest.raises(ValueError):
        e2m1_decode([16])


def test_dequant_fp4_rows_groups():
    codes = np.tile(np.arange(576) % 16, (2, 1))
    scales = np.array([[1.0, 2.0, 4.0, 8.0, 0.25], [3.0, 3.0, 3.0, 3.0, 3.0]], dtype=np.float32)
    v = dequant_fp4_rows(codes, scales)
    for c in (0, 127, 128, 300, 511, 512, 575):
        assert v[0, c] == e2m1_decode(codes[0, c]) * scales[0, c // 128]
        assert v[1, c] == e2m1_decode(codes[1, c]) * 3.0


def test_fp4_generator_rounds_to_nearest_grid_value():
    """The fp4 workload quantiser: every dequantised element is the E2M1 grid
    value nearest to value / scale (same draws regenerated here), and the
    group maximum maps to +-6."""
    x = workloads.make_random(s_q=1, h_q=16, topk=4, s_kv=64, seed=9, kv_format="fp4")
    rng = np.random.default_rng(9)
    rng.standard_normal((1, 16 * 576), dtype=np.float32)          # Q draws
    raw = rng.standard_normal((64, 576), dtype=np.float32)
    codes, scales = x["kv_codes"].numpy(), x["kv_scales"].numpy()
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for g in range(5):
        c0, c1 = 128 * g, min(576, 128 * (g + 1))
        y = raw[:, c0:c1] / scales[:, g:g + 1]
        got = e2m1_decode(codes[:, c0:c1])
        err = np.abs(np.abs(y)[..., None] - grid).min(axis=-1)
        assert np.allclose(np.abs(np.abs(y) - np.abs(got)), err, atol=1e-6)
        assert np.all(np.abs(got).max(axis=1) == 6.0)
