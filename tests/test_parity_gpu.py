"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: out max-abs error <= 2e-2 * max|out_ref| over the case, lse within 1e-3
absolute, and -inf exactly where the oracle has -inf (tokens without a valid
slot).  Index handling and masking are checked bit-exactly where the result
has a unique bf16 value (all slots on one row; poisoned unreferenced rows).
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import dequant_fp8_rows, sparse_mla_fwd_exact

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mla_attention_fwd_amd as smla  # loads libsmla.so; fails loudly if absent
    return torch.device("cuda:0"), smla


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def oracle_tokens(x, tokens=None):
    """Run the oracle on a subset of tokens, gathering only the KV rows they
    reference (indices are remapped; masked slots stay masked)."""
    idx = x["indices"].numpy()
    q = x["q"]
    if tokens is not None:
        idx = idx[tokens]
        q = q[tokens]
    s_kv = x["kv"].shape[0] if "kv" in x else x["kv_codes"].shape[0]
    valid = (idx >= 0) & (idx < s_kv)
    rows = np.unique(idx[valid])
    remap = np.full(idx.shape, -1, dtype=np.int64)
    remap[valid] = np.searchsorted(rows, idx[valid])
    if "kv" in x:
        kv = workloads.to_f64(x["kv"][torch.from_numpy(rows)]) if rows.size else np.zeros((1, 576))
    else:
        kv = dequant_fp8_rows(x["kv_codes"][torch.from_numpy(rows)].numpy(),
                              x["kv_scales"][torch.from_numpy(rows)].numpy()) if rows.size else np.zeros((1, 576))
    return sparse_mla_fwd_exact(workloads.to_f64(q), kv, remap, x["sm_scale"], 512)


def run_gpu(dev, x, **kw):
    device, smla = dev
    q = x["q"].to(device)
    idx = x["indices"].to(device)
    if "kv" in x:
        kv = x["kv"].to(device)
        out, lse = smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], **kw)
    else:
        kv = smla.pack_fp8_kv(x["kv_codes"], x["kv_scales"], device)
        out, lse = smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], kv_format="fp8", **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def check(out, lse, ro, rl, what=""):
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    neg = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf lse mismatch"
    assert np.all(out[neg] == 0), f"{what}: empty rows must be zero"
    scale = max(np.abs(ro).max(), 1e-30)
    err = np.abs(out - ro).max()
    lerr = np.abs(lse[~neg] - rl[~neg]).max() if (~neg).any() else 0.0
    _say(f"  {what}: out err {err:.3e} (tol {OUT_TOL * scale:.3e}), lse err {lerr:.3e}")
    assert err <= OUT_TOL * scale, f"{what}: out error {err} > {OUT_TOL} * {scale}"
    assert lerr <= LSE_TOL, f"{what}: lse error {lerr}"
    return err / scale, lerr


def test_tiny_workload_all_tokens(dev):
    x = workloads.make_inputs("tiny")
    out, lse = run_gpu(dev, x)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, "tiny")


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("b_topk", [32, 64, 128])
def test_random_cases_heads_and_blocks(dev, h_q, b_topk):
    # topk 257: several blocks plus a ragged tail of one slot
    x = workloads.make_random(s_q=3, h_q=h_q, topk=257, s_kv=1000, seed=h_q + b_topk)
    out, lse = run_gpu(dev, x, b_topk=b_topk, num_splits=1)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"h{h_q} B{b_topk}")


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 0])
def test_splits_and_combine(dev, num_splits):
    x = workloads.make_random(s_q=5, h_q=64, topk=300, s_kv=4096, seed=40 + num_splits,
                              invalid_frac=0.3)
    x["indices"][1, :] = -1                  # token 1: every split empty
    x["indices"][2, :200] = -1               # token 2: the first splits empty
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"splits={num_splits}")


def test_masking_duplicates_and_ragged(dev):
    x = workloads.make_random(s_q=6, h_q=64, topk=130, s_kv=777, seed=7, invalid_frac=0.25,
                              dup_frac=0.2, q_mult=4.0)
    idx = x["indices"]
    idx[0, :] = -1                           # no valid slot at all
    idx[1, :129] = -1                        # only the last slot valid
    idx[2, 1:] = 10 ** 6                     # only the first slot valid (rest past s_kv)
    out, lse = run_gpu(dev, x)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, "masking")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("topk", [1, 2, 31, 33, 64, 65, 2048])
def test_topk_edges(dev, topk):
    x = workloads.make_random(s_q=2, h_q=64, topk=topk, s_kv=3000, seed=topk)
    out, lse = run_gpu(dev, x)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"topk={topk}")


@pytest.mark.parametrize("k", [1, 64, 2048])
def test_all_slots_one_row_is_bit_exact(dev, k):
    """Every slot names row r: all logits are equal, S = 1 exactly, the sum is
    exact in fp32 and out/l rounds back to the bf16 row itself."""
    x = workloads.make_random(s_q=3, h_q=64, topk=k, s_kv=500, seed=k)
    rows = [5, 499, 0]
    for t, r in enumerate(rows):
        x["indices"][t, :] = r
    for ns in (1, 4) if k >= 4 else (1,):
        out, lse = run_gpu(dev, x, num_splits=ns)
        for t, r in enumerate(rows):
            v = x["kv"][r, :512].float().numpy()
            assert np.array_equal(out[t], np.broadcast_to(v, out[t].shape)), f"row {r} not exact"
            xr = (workloads.to_f64(x["q"][t]) @ workloads.to_f64(x["kv"][r])) * x["sm_scale"]
            assert np.abs(lse[t] - (xr + math.log(k))).max() < 1e-4


def test_unreferenced_rows_are_never_read(dev):
    """Rows no valid slot names are NaN; any read of them would leak a NaN."""
    x = workloads.make_random(s_q=8, h_q=64, topk=200, s_kv=2048, seed=3, invalid_frac=0.3)
    idx = x["indices"].numpy()
    used = np.zeros(2048, dtype=bool)
    used[idx[(idx >= 0) & (idx < 2048)]] = True
    kv = x["kv"].clone()
    kv[torch.from_numpy(~used)] = float("nan")
    x2 = dict(x, kv=kv)
    out, lse = run_gpu(dev, x2)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, "poisoned")


@pytest.mark.parametrize("h_q,kv_format,num_splits", [(64, "bf16", 1), (128, "bf16", 4), (64, "fp8", 2), (16, "bf16", 3)])
def test_deterministic(dev, h_q, kv_format, num_splits):
    """Ten runs of one plan are bit-identical: no data atomics, a fixed
    reduction order in every kernel and in the combine."""
    x = workloads.make_random(s_q=16, h_q=h_q, topk=512, s_kv=8192, seed=11 + h_q, q_mult=4.0,
                              kv_format=kv_format, invalid_frac=0.1)
    a = run_gpu(dev, x, num_splits=num_splits)
    for _ in range(9):
        b = run_gpu(dev, x, num_splits=num_splits)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_block_sizes_agree(dev):
    x = workloads.make_random(s_q=4, h_q=64, topk=1000, s_kv=8192, seed=12, q_mult=4.0)
    ro, rl = oracle_tokens(x)
    for bt in (32, 64, 128):
        check(*run_gpu(dev, x, b_topk=bt), ro, rl, f"B{bt}")


# ---- B_TOPK 128: one online-softmax step per 128 slots (short splits: the
# one-block kernel; longer splits: the 128-slot block loop)


@pytest.mark.parametrize("h_q", [16, 64, 128])
@pytest.mark.parametrize("topk,num_splits", [(300, 1), (1100, 1), (2048, 1), (2048, 2), (700, 6)])
def test_b128_cases(dev, h_q, topk, num_splits):
    """Ragged last blocks, masked and duplicate slots, Q x4 (rescales across
    blocks), an empty token, leading and trailing blocks without a valid slot,
    a token whose only valid slot is the last; rows no valid slot names are
    NaN (a read of one would leak into the output)."""
    x = workloads.make_random(s_q=6, h_q=h_q, topk=topk, s_kv=5000, seed=topk + h_q + num_splits + 128,
                              invalid_frac=0.2, dup_frac=0.05, q_mult=4.0)
    idx = x["indices"]
    idx[1, :] = -1
    idx[2, : topk // 2] = -1
    idx[3, : topk - 1] = 10 ** 6
    idx[4, 40:] = -1
    used = np.zeros(5000, dtype=bool)
    iv = idx.numpy()
    used[iv[(iv >= 0) & (iv < 5000)]] = True
    kv = x["kv"].clone()
    kv[torch.from_numpy(~used)] = float("nan")
    out, lse = run_gpu(dev, dict(x, kv=kv), num_splits=num_splits, b_topk=128)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"B128 h{h_q} topk={topk} splits={num_splits}")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_b128_all_slots_one_row_is_bit_exact(dev):
    x = workloads.make_random(s_q=2, h_q=64, topk=2048, s_kv=500, seed=1281)
    rows = [7, 499]
    for t, r in enumerate(rows):
        x["indices"][t, :] = r
    out, lse = run_gpu(dev, x, b_topk=128, num_splits=1)
    for t, r in enumerate(rows):
        v = x["kv"][r, :512].float().numpy()
        assert np.array_equal(out[t], np.broadcast_to(v, out[t].shape)), f"row {r} not exact"
        xr = (workloads.to_f64(x["q"][t]) @ workloads.to_f64(x["kv"][r])) * x["sm_scale"]
        assert np.abs(lse[t] - (xr + math.log(2048))).max() < 1e-4


def test_strided_views(dev):
    """Non-default strides: Q and out as head-sliced views, KV rows padded."""
    device, smla = dev
    x = workloads.make_random(s_q=3, h_q=16, topk=100, s_kv=300, seed=5)
    qbig = torch.zeros((3, 24, 576 + 64), dtype=torch.bfloat16)
    qbig[:, 4:20, :576] = x["q"]
    kvbig = torch.zeros((300, 576 + 128), dtype=torch.bfloat16)
    kvbig[:, :576] = x["kv"]
    q = qbig.to(device)[:, 4:20, :576]
    kv = kvbig.to(device)[:, :576]
    idx = torch.zeros((3, 136), dtype=torch.int32)
    idx[:, :100] = x["indices"]
    idx = idx.to(device)[:, :100]
    outbig = torch.full((3, 20, 520), 7.0, dtype=torch.bfloat16, device=device)
    out = outbig[:, 2:18, :512]
    lsebig = torch.full((3, 40), 7.0, dtype=torch.float32, device=device)
    lse = lsebig[:, 8:24]
    smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle_tokens(x)
    check(out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), ro, rl, "strided")
    ob = outbig.cpu()
    assert torch.all(ob[:, :2] == 7) and torch.all(ob[:, 18:] == 7) and torch.all(ob[:, :, 512:] == 7)
    lb = lsebig.cpu()
    assert torch.all(lb[:, :8] == 7) and torch.all(lb[:, 24:] == 7)


# ---- full-size workloads: the launch the benchmark times, every token compared


def check_whole_config(out, lse, ro, rl, what):
    """The parity bar over the whole configuration (tolerance from max|out|
    over every token), plus the worst per-token ratio err_t / max|out_t| as a
    diagnostic."""
    rel, lerr = check(out, lse, ro, rl, what)
    den = np.maximum(np.abs(ro).reshape(ro.shape[0], -1).max(axis=1), 1e-30)
    per = np.abs(out - ro).reshape(ro.shape[0], -1).max(axis=1) / den
    worst = int(np.argmax(per))
    _say(f"  {what}: {ro.shape[0]} tokens, worst token {worst} at {per[worst]:.3e} of its own max|out|")
    return rel, lerr


def _whole(dev, x, **kw):
    out, lse = run_gpu(dev, x, **kw)
    ro, rl = oracle_tokens(x)
    return check_whole_config(out, lse, ro, rl, f"{x['workload'].name} all tokens")


def test_prefill_full_size_all_tokens(dev):
    _whole(dev, workloads.make_inputs("prefill"))


def test_causal_full_size_all_tokens(dev):
    _whole(dev, workloads.make_inputs("causal"))


def test_prefill_full_size_all_tokens_b128(dev):
    _whole(dev, workloads.make_inputs("prefill"), b_topk=128)


@pytest.mark.parametrize("h_q", [16, 64])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_fp8_random_cases(dev, h_q, num_splits):
    x = workloads.make_random(s_q=3, h_q=h_q, topk=300, s_kv=2000, seed=60 + h_q + num_splits,
                              kv_format="fp8", invalid_frac=0.2, q_mult=2.0)
    x["indices"][2, :] = -1
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"fp8 h{h_q} splits={num_splits}")


@pytest.mark.parametrize("h_q", [64, 128])
@pytest.mark.parametrize("topk,num_splits", [(1100, 1), (2048, 2)])
def test_fp8_long_split_cases(dev, h_q, topk, num_splits):
    """The pipelined fp8 kernel over many blocks: whole blocks masked before
    the first valid slot (the running max is still -inf there), a single
    valid slot at the end, trailing blocks skipped, no valid slot."""
    x = workloads.make_random(s_q=6, h_q=h_q, topk=topk, s_kv=5000, seed=topk + h_q + 7 * num_splits,
                              kv_format="fp8", invalid_frac=0.2, dup_frac=0.05, q_mult=2.0)
    idx = x["indices"]
    idx[1, :] = -1                           # no valid slot
    idx[2, :700] = -1                        # leading blocks without a valid slot
    idx[3, :topk - 1] = 10 ** 6              # only the last slot valid
    idx[4, 40:] = -1                         # trailing blocks skipped
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"fp8 long h{h_q} topk={topk} splits={num_splits}")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("h_q,topk,num_splits", [(64, 1500, 1), (64, 2048, 2), (128, 2048, 3)])
def test_fp8_pipelined_frequent_rescales(dev, h_q, topk, num_splits):
    """The 64-head fp8 kernel with Q x 8: the running max moves in most blocks,
    so the per-head-tile rescale of the accumulators runs often, also after
    leading blocks that are fully masked (token 1) and between valid blocks
    separated by masked ones (token 2)."""
    x = workloads.make_random(s_q=5, h_q=h_q, topk=topk, s_kv=6000, seed=300 + h_q + num_splits,
                              kv_format="fp8", invalid_frac=0.1, q_mult=8.0)
    idx = x["indices"]
    idx[1, :700] = -1
    idx[2, 100:900] = -1
    idx[2, 1200:1800] = -1
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"fp8 Qx8 h{h_q} splits={num_splits}")


def test_fp8_single_row_matches_dequant(dev):
    """All slots on one row: out is that row's V = code * scale.  The codes are
    used exactly and the scale enters through the bf16 S operand, so each
    element is within two bf16 roundings (unit roundoff 2^-8 each, so 2^-7
    relative) of the exact value;
    lse is the row's logit plus ln(topk)."""
    x = workloads.make_random(s_q=2, h_q=64, topk=64, s_kv=100, seed=8, kv_format="fp8")
    x["indices"][0, :] = 17
    x["indices"][1, :] = 99
    out, lse = run_gpu(dev, x, num_splits=1)
    for t, r in enumerate((17, 99)):
        row = dequant_fp8_rows(x["kv_codes"][r:r + 1].numpy(), x["kv_scales"][r:r + 1].numpy())[0]
        v = row[:512]
        assert np.all(np.abs(out[t] - v) <= 2.0 ** -7 * np.abs(v) + 1e-30)
        xr = (workloads.to_f64(x["q"][t]) @ row) * x["sm_scale"]
        assert np.abs(lse[t] - (xr + math.log(64))).max() < 1e-4


def test_decode_fp8_full_size_all_tokens(dev):
    x = workloads.make_inputs("decode_fp8")
    _whole(dev, x, num_splits=x["workload"].num_splits)


def test_decode_full_size_all_tokens(dev):
    x = workloads.make_inputs("decode")
    _whole(dev, x, num_splits=x["workload"].num_splits)


# every finite E4M3 code (254 of 256: 0x7F and 0xFF are NaN), walked along the
# V columns of 16 rows, each row a different rotation of the list
FP8_FINITE_CODES = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)


@pytest.mark.parametrize("h_q,num_splits", [(16, 1), (32, 1), (64, 1), (64, 2), (128, 2)])
def test_fp8_every_code_bit_exact(dev, h_q, num_splits):
    """Unit scales and every slot of token t on row t: all logits are equal,
    S = 1, the product sums k copies of the code value exactly in fp32, and
    out/l rounds back to the code value.  So out must equal the E4M3 value of
    each column's code exactly, for all 254 finite codes (subnormals and both
    zeros included; the sign of a zero is not pinned, the accumulator starts at
    +0).  Pins the in-kernel conversion of every code in both the pipelined
    (64 heads per workgroup) and the cooperative (16, 32 heads) kernels."""
    n = 16
    x = workloads.make_random(s_q=n, h_q=h_q, topk=64, s_kv=n, seed=h_q + num_splits, kv_format="fp8")
    cols = np.arange(576)
    codes = np.stack([FP8_FINITE_CODES[(cols * 3 + 17 * r) % FP8_FINITE_CODES.size] for r in range(n)])
    assert all(np.unique(codes[r, :512]).size == FP8_FINITE_CODES.size for r in range(n))
    x["kv_codes"] = torch.from_numpy(codes.astype(np.uint8))
    x["kv_scales"] = torch.ones((n, 5), dtype=torch.float32)
    x["indices"] = torch.arange(n, dtype=torch.int32)[:, None].repeat(1, 64)
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    want = dequant_fp8_rows(codes, np.ones((n, 5), dtype=np.float32))[:, :512]
    assert np.array_equal(out, np.broadcast_to(want[:, None, :], out.shape))
    for t in range(n):
        xr = (workloads.to_f64(x["q"][t]) @ dequant_fp8_rows(codes[t:t + 1], np.ones((1, 5)))[0]) * x["sm_scale"]
        assert np.abs(lse[t] - (xr + math.log(64))).max() < 1e-3


# ---- long splits (>= 1024 slots, 64 heads per workgroup): the pipelined kernel


@pytest.mark.parametrize("h_q", [64, 128])
@pytest.mark.parametrize("topk,num_splits", [(1024, 1), (1100, 1), (2048, 1), (2048, 2)])
def test_long_split_cases(dev, h_q, topk, num_splits):
    x = workloads.make_random(s_q=6, h_q=h_q, topk=topk, s_kv=5000, seed=topk + h_q + num_splits,
                              invalid_frac=0.2, dup_frac=0.05, q_mult=4.0)
    idx = x["indices"]
    idx[1, :] = -1                           # no valid slot
    idx[2, :700] = -1                        # leading blocks without a valid slot
    idx[3, :topk - 1] = 10 ** 6              # only the last slot valid
    idx[4, 40:] = -1                         # trailing blocks skipped
    out, lse = run_gpu(dev, x, num_splits=num_splits)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"long h{h_q} topk={topk} splits={num_splits}")


def test_long_split_unreferenced_rows_are_never_read(dev):
    """Invalid slots gather a padding row; it must be a referenced one."""
    x = workloads.make_random(s_q=4, h_q=64, topk=1024, s_kv=6000, seed=21, invalid_frac=0.4)
    x["indices"][2, :600] = -1
    idx = x["indices"].numpy()
    used = np.zeros(6000, dtype=bool)
    used[idx[(idx >= 0) & (idx < 6000)]] = True
    kv = x["kv"].clone()
    kv[torch.from_numpy(~used)] = float("nan")
    out, lse = run_gpu(dev, dict(x, kv=kv))
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, "long poisoned")


@pytest.mark.parametrize("topk", [300, 2048])
def test_kv_beyond_32bit_offsets(dev, topk):
    """A bf16 KV of 4.2 M rows (4.8 GB) no longer fits 32-bit byte offsets:
    the gathers take 64-bit addresses.  Indices span the whole table."""
    device, smla = dev
    s_kv = 4_200_000
    x = workloads.make_random(s_q=3, h_q=64, topk=topk, s_kv=1, seed=31)
    rng = np.random.default_rng(32)
    idx = np.stack([rng.choice(s_kv, topk, replace=False) for _ in range(3)])
    idx[0, :5] = s_kv - 1 - np.arange(5)     # the last rows
    idx[1, 7] = -1
    rows = np.unique(idx[idx >= 0])
    sub = torch.from_numpy(rng.standard_normal((rows.size, 576)).astype(np.float32)).to(torch.bfloat16)
    kv = torch.zeros((s_kv, 576), dtype=torch.bfloat16, device=device)
    kv[torch.from_numpy(rows).to(device)] = sub.to(device)
    q = x["q"].to(device)
    out, lse = smla.sparse_mla_fwd(q, kv, torch.from_numpy(idx.astype(np.int32)).to(device), x["sm_scale"])
    torch.cuda.synchronize()
    remap = np.full(idx.shape, -1, dtype=np.int64)
    ok = idx >= 0
    remap[ok] = np.searchsorted(rows, idx[ok])
    ro, rl = sparse_mla_fwd_exact(workloads.to_f64(x["q"]), workloads.to_f64(sub), remap, x["sm_scale"], 512)
    del kv
    torch.cuda.empty_cache()
    check(out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), ro, rl, f"kv 4.8 GB topk={topk}")


@pytest.mark.parametrize("topk,num_splits,b_topk", [(512, 4, 32), (300, 3, 32), (128, 1, 32),
                                                    (512, 4, 64), (97, 1, 64), (700, 6, 32)])
def test_h128_short_splits_one_gather_for_both_head_groups(dev, topk, num_splits, b_topk):
    """h_q 128 with splits of at most 128 slots: one workgroup gathers a split's
    rows once and runs both 64-head groups over them.  Ragged last blocks,
    masked slots, an empty token and a token whose first splits are empty;
    rows no valid slot names are NaN (a read of one would leak)."""
    x = workloads.make_random(s_q=6, h_q=128, topk=topk, s_kv=3000, seed=topk + num_splits + b_topk,
                              invalid_frac=0.3, q_mult=4.0)
    x["indices"][1, :] = -1
    x["indices"][2, : topk // 2] = -1
    idx = x["indices"].numpy()
    used = np.zeros(3000, dtype=bool)
    used[idx[(idx >= 0) & (idx < 3000)]] = True
    kv = x["kv"].clone()
    kv[torch.from_numpy(~used)] = float("nan")
    out, lse = run_gpu(dev, dict(x, kv=kv), num_splits=num_splits, b_topk=b_topk)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"h128 topk={topk} ns={num_splits} B{b_topk}")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_h128_short_splits_one_row_is_bit_exact(dev):
    x = workloads.make_random(s_q=2, h_q=128, topk=512, s_kv=700, seed=128)
    rows = [3, 699]
    for t, r in enumerate(rows):
        x["indices"][t, :] = r
    out, lse = run_gpu(dev, x, num_splits=4)
    for t, r in enumerate(rows):
        v = x["kv"][r, :512].float().numpy()
        assert np.array_equal(out[t], np.broadcast_to(v, out[t].shape)), f"row {r} not exact"
        xr = (workloads.to_f64(x["q"][t]) @ workloads.to_f64(x["kv"][r])) * x["sm_scale"]
        assert np.abs(lse[t] - (xr + math.log(512))).max() < 1e-4


def test_tuned_plan_is_a_valid_plan_and_matches_the_oracle(dev):
    """smla_fwd_tune times the candidate plans on a decode-like shape; the
    outputs it leaves and those of the chosen plan both meet the parity bar."""
    device, smla = dev
    x = workloads.make_random(s_q=16, h_q=128, topk=512, s_kv=20000, seed=31, invalid_frac=0.1)
    q, kv, idx = x["q"].to(device), x["kv"].to(device), x["indices"].to(device)
    ns, bt, us = smla.tune_plan(q, kv, idx, x["sm_scale"], iterations=3)
    assert bt in (32, 64) and 1 <= ns <= 512 and us > 0
    _say(f"  tuned plan: num_splits={ns} b_topk={bt} ({us:.1f} us)")
    out, lse = run_gpu(dev, x, num_splits=ns, b_topk=bt)
    ro, rl = oracle_tokens(x)
    check(out, lse, ro, rl, f"tuned ns={ns} B{bt}")


def test_binding_rejects_host_rows_and_bad_outputs_before_launch(dev):
    """Device q with host KV (the default of pack_fp8_kv), a float64 lse or an
    fp32 out: the binding raises before the library sees a pointer, and a
    correct call afterwards still runs (nothing was enqueued)."""
    device, smla = dev
    x = workloads.make_random(s_q=2, h_q=16, topk=40, s_kv=100, seed=3, kv_format="fp8")
    q, idx = x["q"].to(device), x["indices"].to(device)
    host_rows = smla.pack_fp8_kv(x["kv_codes"], x["kv_scales"])
    with pytest.raises(ValueError, match="device"):
        smla.sparse_mla_fwd(q, host_rows, idx, x["sm_scale"], kv_format="fp8")
    rows = host_rows.to(device)
    with pytest.raises(ValueError):
        smla.sparse_mla_fwd(q, rows, idx, x["sm_scale"], kv_format="fp8",
                            lse=torch.empty((2, 16), dtype=torch.float64, device=device))
    with pytest.raises(ValueError):
        smla.sparse_mla_fwd(q, rows, idx, x["sm_scale"], kv_format="fp8",
                            out=torch.empty((2, 16, 512), dtype=torch.float32, device=device))
    out, lse = smla.sparse_mla_fwd(q, rows, idx, x["sm_scale"], kv_format="fp8")
    torch.cuda.synchronize()
    ro, rl = oracle_tokens(x)
    check(out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), ro, rl, "after rejections")
