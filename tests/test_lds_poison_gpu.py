"""Race and unwritten-LDS checks with the LDS-poisoning debug build.

libsmla_poison.so is the same source compiled with SMLA_DEBUG_LDS_POISON:
every kernel fills its LDS with all-ones bytes at entry and poisons the
destination of each direct-to-LDS load just before issuing it.  All-ones reads
as NaN in bf16, fp32 and E4M3, so a read of LDS that no store or completed load
has written, or a read that races a refill by another wave, puts NaN into the
results instead of a plausible stale value.  (Page "FlashMLA算子Ascend 950移植：
从tiling到访存优化全解读", section 5.4, traces pipeline bubbles and wrong results
to the synchronisation between loads and compute; this build makes a missing
wait or barrier visible.)

All cases keep the KV inside the 32-bit buffer window: there a poisoned index
(-1) that a racing gather used as a row would become an out-of-window offset,
which the hardware drops, instead of an address below the KV.

Each case runs the product library and the debug library on the same inputs.
The debug run must be finite, bit-identical to the product run (the poison
writes add waits, never arithmetic) and within the parity bar of the oracle.
One case per kernel family: the pipelined bf16 kernel (with and without
precomputed block counts), the 16- and 32-head kernels, B_TOPK 64 and 128,
the one-block short-split kernel (shared gather for 128 heads), split parts
and their combine, the fp8 and fp4 kernels (pipelined and cooperative), the
persistent schedule and the paged cache.
"""
import os

import numpy as np
import pytest
import torch

import workloads
from sparse_mla_attention_fwd_amd import _lib
from test_fp4_gpu import oracle_fp4, run_fp4
from test_paged_gpu import oracle_paged, run_paged
from test_parity_gpu import _say, check, oracle_tokens, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(_lib.POISON_LIB_PATH), "libsmla_poison.so is missing: run __graft_entry__.build()"
    import sparse_mla_attention_fwd_amd as smla
    return torch.device("cuda:0"), smla


def _both(call):
    ref = call()
    with _lib.library(_lib.POISON_LIB_PATH):
        got = call()
    return ref, got


def _check_pair(ref, got, ro, rl, what):
    _say(f"{what}: debug build")
    check(got[0], got[1], ro, rl, what + " (poisoned LDS)")
    assert np.array_equal(ref[0], got[0]), f"{what}: out differs from the product build"
    assert np.array_equal(ref[1], got[1]), f"{what}: lse differs from the product build"


BF16_CASES = [
    # (name, h_q, topk, s_kv, num_splits, b_topk, invalid_frac, q_mult)
    ("pipelined", 64, 1100, 6000, 1, 32, 0.2, 4.0),
    ("pipelined, every slot valid", 64, 2048, 9000, 1, 32, 0.0, 1.0),
    ("16 heads", 16, 700, 3000, 1, 32, 0.2, 1.0),
    ("32 heads B64", 32, 700, 3000, 2, 64, 0.2, 1.0),
    ("B64 64 heads", 64, 1000, 5000, 1, 64, 0.1, 4.0),
    ("B128 block loop", 64, 1100, 5000, 1, 128, 0.1, 1.0),
    ("B128 one block", 128, 300, 4000, 3, 128, 0.1, 1.0),
    ("one-block 128 heads", 128, 512, 5000, 4, 32, 0.15, 1.0),
    ("splits and combine", 64, 300, 4096, 3, 32, 0.3, 1.0),
]


@pytest.mark.parametrize("name,h_q,topk,s_kv,num_splits,b_topk,invalid,q_mult", BF16_CASES)
def test_poisoned_lds_bf16(dev, name, h_q, topk, s_kv, num_splits, b_topk, invalid, q_mult):
    x = workloads.make_random(s_q=9, h_q=h_q, topk=topk, s_kv=s_kv, seed=900 + h_q + topk,
                              invalid_frac=invalid, q_mult=q_mult)
    x["indices"][1, :] = -1                       # a token without a valid slot
    x["indices"][2, topk // 3:] = -1              # a token whose last blocks are masked
    ref, got = _both(lambda: run_gpu(dev, x, num_splits=num_splits, b_topk=b_topk))
    ro, rl = oracle_tokens(x)
    _check_pair(ref, got, ro, rl, name)


@pytest.mark.parametrize("h_q,num_splits", [(64, 1), (64, 2), (32, 1), (16, 3)])
def test_poisoned_lds_fp8(dev, h_q, num_splits):
    x = workloads.make_random(s_q=6, h_q=h_q, topk=1100, s_kv=5000, seed=950 + h_q + num_splits,
                              kv_format="fp8", invalid_frac=0.15)
    x["indices"][1, :] = -1
    ref, got = _both(lambda: run_gpu(dev, x, num_splits=num_splits))
    ro, rl = oracle_tokens(x)
    _check_pair(ref, got, ro, rl, f"fp8 h{h_q} s{num_splits}")


@pytest.mark.parametrize("h_q,num_splits", [(64, 1), (64, 2), (32, 1)])
def test_poisoned_lds_fp4(dev, h_q, num_splits):
    x = workloads.make_random(s_q=6, h_q=h_q, topk=1100, s_kv=5000, seed=970 + h_q + num_splits,
                              kv_format="fp4", invalid_frac=0.15)
    x["indices"][1, :] = -1
    ref, got = _both(lambda: run_fp4(dev, x, num_splits=num_splits))
    ro, rl = oracle_fp4(x)
    _check_pair(ref, got, ro, rl, f"fp4 h{h_q} s{num_splits}")


def test_poisoned_lds_persistent(dev):
    from test_persistent_gpu import _varied
    x = _varied(seed=990, s_q=30, topk=1100)

    def call():
        device, smla = dev
        out, lse = smla.sparse_mla_fwd(x["q"].to(device), x["kv"].to(device), x["indices"].to(device),
                                       x["sm_scale"], schedule="persistent", persistent_workgroups=7)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)

    ref, got = _both(call)
    ro, rl = oracle_tokens(x)
    _check_pair(ref, got, ro, rl, "persistent")


def test_poisoned_lds_paged(dev):
    x = workloads.make_random_paged(s_q=6, h_q=128, topk=512, page_size=16, num_pages=60, table_width=48,
                                    seed=995, unallocated_frac=0.1, invalid_frac=0.1)
    ref, got = _both(lambda: run_paged(dev, x, num_splits=4))
    ro, rl = oracle_paged(x)
    _check_pair(ref, got, ro, rl, "paged")
