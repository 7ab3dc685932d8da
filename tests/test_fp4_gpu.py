"""GPU parity of the fp4 (OCP MX E2M1) KV cache against the float64 oracle.

The kernels convert the E2M1 codes to bf16 exactly and fold the five group
scales in fp32 (QK partial sums) and into the bf16 S operand (PV), as for the
fp8 cache.  Same bar as the other parity tests.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import dequant_fp4_rows, sparse_mla_fwd_exact
from test_parity_gpu import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mla_attention_fwd_amd as smla  # loads libsmla.so; fails loudly if absent
    return torch.device("cuda:0"), smla


def run_fp4(dev, x, **kw):
    device, smla = dev
    kv = smla.pack_fp4_kv(x["kv_codes"], x["kv_scales"], device)
    out, lse = smla.sparse_mla_fwd(x["q"].to(device), kv, x["indices"].to(device), x["sm_scale"],
                                   kv_format="fp4", **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def oracle_fp4(x, tokens=None):
    """The oracle on the dequantised rows the (sampled) tokens reference."""
    idx = x["indices"].numpy()
    q = x["q"]
    if tokens is not None:
        idx, q = idx[tokens], q[tokens]
    s_kv = x["kv_codes"].shape[0]
    valid = (idx >= 0) & (idx < s_kv)
    rows = np.unique(idx[valid])
    remap = np.full(idx.shape, -1, dtype=np.int64)
    remap[valid] = np.searchsorted(rows, idx[valid])
    sel = torch.from_numpy(rows)
    kv = dequant_fp4_rows(x["kv_codes"][sel].numpy(), x["kv_scales"][sel].numpy()) \
        if rows.size else np.zeros((1, 576))
    return sparse_mla_fwd_exact(workloads.to_f64(q), kv, remap, x["sm_scale"], 512)


@pytest.mark.parametrize("h_q", [16, 64, 128])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_fp4_random_cases(dev, h_q, num_splits):
    """Several blocks and a ragged tail, masked and repeated slots, a token
    without a valid slot."""
    x = workloads.make_random(s_q=3, h_q=h_q, topk=300, s_kv=2000, seed=90 + h_q + num_splits,
                              kv_format="fp4", invalid_frac=0.2, dup_frac=0.1, q_mult=2.0)
    x["indices"][2, :] = -1
    out, lse = run_fp4(dev, x, num_splits=num_splits)
    ro, rl = oracle_fp4(x)
    check(out, lse, ro, rl, f"fp4 h{h_q} splits={num_splits}")
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))


def test_fp4_single_row_matches_dequant(dev):
    """All slots on one row: out is that row's V = e2m1(code) * scale.  The
    codes are used exactly and the scale enters through the bf16 S operand, so
    each element is within two bf16 roundings (2^-7 relative) of the exact
    value; lse is the row's logit plus ln(topk)."""
    x = workloads.make_random(s_q=2, h_q=64, topk=64, s_kv=100, seed=18, kv_format="fp4")
    x["indices"][0, :] = 17
    x["indices"][1, :] = 99
    out, lse = run_fp4(dev, x, num_splits=1)
    for t, r in enumerate((17, 99)):
        row = dequant_fp4_rows(x["kv_codes"][r:r + 1].numpy(), x["kv_scales"][r:r + 1].numpy())[0]
        v = row[:512]
        assert np.all(np.abs(out[t] - v) <= 2.0 ** -7 * np.abs(v) + 1e-30)
        xr = (workloads.to_f64(x["q"][t]) @ row) * x["sm_scale"]
        assert np.abs(lse[t] - (xr + math.log(64))).max() < 1e-4


def test_fp4_every_code_and_nibble_order(dev):
    """Row r's codes are a known permutation of all 16 codes at every column
    with unit scales, and each token's slots name one row: the output is the
    E2M1 value of every column's code (exact in bf16), which pins the
    conversion of each code and the low-nibble-first packing."""
    x = workloads.make_random(s_q=16, h_q=16, topk=8, s_kv=16, seed=5, kv_format="fp4")
    cols = np.arange(576)
    codes = np.stack([(cols + r) % 16 for r in range(16)]).astype(np.uint8)
    x["kv_codes"] = torch.from_numpy(codes)
    x["kv_scales"] = torch.ones((16, 5), dtype=torch.float32)
    x["indices"] = torch.arange(16, dtype=torch.int32)[:, None].repeat(1, 8)
    out, _ = run_fp4(dev, x, num_splits=1)
    want = dequant_fp4_rows(codes, np.ones((16, 5), dtype=np.float32))[:, :512]
    assert np.array_equal(out, np.broadcast_to(want[:, None, :], out.shape))


def test_decode_fp4_full_size_all_tokens(dev):
    """The fp4 decode workload (128 sequences, 16384 rows each, h_q 64,
    topk 2048), in the launch configuration bench.py times, every token
    compared with the oracle."""
    from test_parity_gpu import check_whole_config
    x = workloads.make_inputs("decode_fp4")
    out, lse = run_fp4(dev, x, num_splits=x["workload"].num_splits)
    ro, rl = oracle_fp4(x)
    check_whole_config(out, lse, ro, rl, "decode_fp4 all tokens")


@pytest.mark.parametrize("h_q", [64, 128])
@pytest.mark.parametrize("topk,num_splits", [(1100, 1), (2048, 2), (2048, 3), (40, 1)])
def test_fp4_long_splits_pipelined(dev, h_q, topk, num_splits):
    """The 64-head fp4 kernel over many blocks (its raw-stage ring wraps
    around several times): ragged last blocks, masked and repeated slots, Q x 4
    (rescales across blocks), an empty token, leading and trailing slots
    without a valid index, a token whose only valid slot is the last.  Rows no
    valid slot names get NaN scales: a read of one would leak into the output."""
    x = workloads.make_random(s_q=6, h_q=h_q, topk=topk, s_kv=5000, seed=topk + h_q + num_splits + 4,
                              kv_format="fp4", invalid_frac=0.2, dup_frac=0.05, q_mult=4.0)
    idx = x["indices"]
    idx[1, :] = -1
    idx[2, : topk // 2] = -1
    idx[3, : topk - 1] = 10 ** 6
    idx[4, 20:] = -1
    iv = idx.numpy()
    used = np.zeros(5000, dtype=bool)
    used[iv[(iv >= 0) & (iv < 5000)]] = True
    scales = x["kv_scales"].clone()
    scales[torch.from_numpy(~used)] = float("nan")
    out, lse = run_fp4(dev, dict(x, kv_scales=scales), num_splits=num_splits)
    ro, rl = oracle_fp4(x)
    check(out, lse, ro, rl, f"fp4 long h{h_q} topk={topk} splits={num_splits}")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
