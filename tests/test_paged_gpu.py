"""GPU parity of the paged-KV entry point (smla_fwd_paged through the C ABI)
against the float64 paged oracle (page "Flash Attention Infer算子性能优化",
section 优化Paged Attention路径: logical position j of token t is row
j % page_size of page block_table[t, j // page_size]).

Same bar as the other parity tests: out max-abs error <= 2e-2 * max|out_ref|,
lse within 1e-3, -inf exactly where the oracle has it; index translation and
masking bit-exact where the result has a unique bf16 value.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import dequant_fp4_rows, dequant_fp8_rows
from oracle.paged import sparse_mla_fwd_paged
from test_parity_gpu import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mla_attention_fwd_amd as smla  # loads libsmla.so; fails loudly if absent
    return torch.device("cuda:0"), smla


def run_paged(dev, x, **kw):
    device, smla = dev
    q = x["q"].to(device)
    idx = x["indices"].to(device)
    bt = x["block_table"].to(device)
    if "kv" in x:
        kv = x["kv"].to(device)
        out, lse = smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], block_table=bt,
                                       page_size=x["page_size"], **kw)
    else:
        kv = smla.pack_fp8_kv(x["kv_codes"], x["kv_scales"], device)
        out, lse = smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], kv_format="fp8", block_table=bt,
                                       page_size=x["page_size"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def oracle_paged(x, tokens=None):
    """The paged oracle on a subset of tokens, given only the pages their
    block-table rows name (the table is remapped onto that compact pool)."""
    ps = x["page_size"]
    table = x["block_table"].numpy()
    idx = x["indices"].numpy()
    q = x["q"]
    if tokens is not None:
        table, idx, q = table[tokens], idx[tokens], q[tokens]
    rows_total = x["kv"].shape[0] if "kv" in x else x["kv_codes"].shape[0]
    num_pages = rows_total // ps
    ok = (table >= 0) & (table < num_pages)
    pages = np.unique(table[ok])
    remap = np.full(table.shape, -1, dtype=np.int64)
    remap[ok] = np.searchsorted(pages, table[ok])
    rows = torch.from_numpy((pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1))
    if "kv" in x:
        kv = workloads.to_f64(x["kv"][rows]) if pages.size else np.zeros((ps, 576))
    else:
        kv = dequant_fp8_rows(x["kv_codes"][rows].numpy(), x["kv_scales"][rows].numpy()) \
            if pages.size else np.zeros((ps, 576))
    kv_pages = kv.reshape(-1, ps, 576)
    return sparse_mla_fwd_paged(workloads.to_f64(q), kv_pages, remap, idx, x["sm_scale"], 512)


@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("h_q,num_splits", [(64, 1), (64, 0), (128, 4), (128, 1)])
def test_paged_random_cases(dev, page_size, h_q, num_splits):
    """Pages shared between tokens, unallocated blocks (-1), positions past
    the table, ragged block counts."""
    width = max(2, 640 // page_size)
    x = workloads.make_random_paged(s_q=5, h_q=h_q, topk=300, page_size=page_size,
                                    num_pages=width + 7, table_width=width,
                                    seed=page_size * 10 + h_q + num_splits,
                                    unallocated_frac=0.2, invalid_frac=0.2)
    x["block_table"][1, :] = -1                       # token 1: nothing allocated
    out, lse = run_paged(dev, x, num_splits=num_splits)
    ro, rl = oracle_paged(x)
    check(out, lse, ro, rl, f"paged ps={page_size} h{h_q} ns={num_splits}")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("num_splits", [0, 2])
def test_paged_fp8_cases(dev, num_splits):
    x = workloads.make_random_paged(s_q=4, h_q=64, topk=700, page_size=16, num_pages=70,
                                    table_width=64, seed=77 + num_splits, unallocated_frac=0.15,
                                    invalid_frac=0.1, kv_format="fp8")
    out, lse = run_paged(dev, x, num_splits=num_splits)
    ro, rl = oracle_paged(x)
    check(out, lse, ro, rl, f"paged fp8 ns={num_splits}")


@pytest.mark.parametrize("h_q,num_splits", [(64, 0), (64, 2), (32, 1), (128, 4)])
def test_paged_fp4_cases(dev, h_q, num_splits):
    """An fp4 (E2M1) page pool through the block table: the translated rows
    feed the fp4 kernels (64-head pipelined, 16/32-head cooperative) unchanged."""
    x = workloads.make_random_paged(s_q=4, h_q=h_q, topk=700, page_size=16, num_pages=70,
                                    table_width=64, seed=88 + h_q + num_splits, unallocated_frac=0.15,
                                    invalid_frac=0.1, kv_format="fp4")
    device, smla = dev
    kv = smla.pack_fp4_kv(x["kv_codes"], x["kv_scales"], device)
    out, lse = smla.sparse_mla_fwd(x["q"].to(device), kv, x["indices"].to(device), x["sm_scale"],
                                   kv_format="fp4", block_table=x["block_table"].to(device),
                                   page_size=x["page_size"], num_splits=num_splits)
    torch.cuda.synchronize()
    # the oracle on the whole (small) dequantised pool
    kv_pages = dequant_fp4_rows(x["kv_codes"].numpy(), x["kv_scales"].numpy()).reshape(-1, 16, 576)
    ro, rl = sparse_mla_fwd_paged(workloads.to_f64(x["q"]), kv_pages, x["block_table"].numpy().astype(np.int64),
                                  x["indices"].numpy(), x["sm_scale"], 512)
    check(out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), ro, rl,
          f"paged fp4 h{h_q} ns={num_splits}")


def test_identity_table_is_bit_identical_to_flat_kv(dev):
    """Pages in pool order and logical = physical positions: the paged call
    runs the same kernels on the same rows as smla_fwd, so every bit agrees."""
    device, smla = dev
    x = workloads.make_random(s_q=6, h_q=128, topk=400, s_kv=4096, seed=5, invalid_frac=0.2)
    ps = 32
    bt = torch.arange(4096 // ps, dtype=torch.int32).repeat(6, 1)
    a = smla.sparse_mla_fwd(x["q"].to(device), x["kv"].to(device), x["indices"].to(device), x["sm_scale"])
    b = smla.sparse_mla_fwd(x["q"].to(device), x["kv"].to(device), x["indices"].to(device), x["sm_scale"],
                            block_table=bt.to(device), page_size=ps)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_paged_one_row_is_bit_exact(dev):
    """Every valid slot names logical row r (page 5, row 3); slots into an
    unallocated block or past the table are masked: out = V[r] exactly."""
    x = workloads.make_random_paged(s_q=1, h_q=64, topk=64, page_size=8, num_pages=12,
                                    table_width=6, seed=3)
    x["block_table"][0] = torch.tensor([2, -1, 5, 0, 11, 3], dtype=torch.int32)
    r = 2 * 8 + 3
    idx = np.full(64, r, dtype=np.int32)
    idx[::7] = 9                                     # block 1: unallocated
    idx[::11] = 48                                   # past the table (6 * 8)
    x["indices"] = torch.from_numpy(idx[None, :].copy())
    out, lse = run_paged(dev, x)
    v = x["kv"][5 * 8 + 3, :512].float().numpy()
    assert np.array_equal(out[0], np.broadcast_to(v, out[0].shape))
    k = int(np.sum(idx == r))
    xr = (workloads.to_f64(x["q"][0]) @ workloads.to_f64(x["kv"][5 * 8 + 3])) * x["sm_scale"]
    assert np.abs(lse[0] - (xr + math.log(k))).max() < 1e-4


def test_decode_paged_full_size_all_tokens(dev):
    """The paged decode workload (64 sequences, pages of 64 rows dealt in a
    random order, h_q 128, topk 512, 4 splits), in the launch configuration
    bench.py times, every token compared with the oracle (run on chunks of
    tokens so that only the pages of a chunk are expanded at a time)."""
    from test_parity_gpu import check_whole_config
    x = workloads.make_inputs("decode_paged")
    w = x["workload"]
    out, lse = run_paged(dev, x, num_splits=w.num_splits)
    parts = [oracle_paged(x, list(range(t0, min(w.s_q, t0 + 8)))) for t0 in range(0, w.s_q, 8)]
    ro = np.concatenate([p[0] for p in parts])
    rl = np.concatenate([p[1] for p in parts])
    check_whole_config(out, lse, ro, rl, "decode_paged all tokens")
