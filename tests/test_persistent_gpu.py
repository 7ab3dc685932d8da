"""The persistent schedule (page "Flash Attention Infer算子性能优化", section
优化多核负载均衡: tokens dealt to workgroups by valid-block weight) against the
float64 oracle and, bit for bit, against the one-workgroup-per-token grid.

Few persistent workgroups are forced so that each runs many tokens in one
stream: token boundaries inside the gather pipeline, tokens of one block,
empty tokens, trailing masked blocks, and the next token's Q switched in
while the current token's last blocks compute.  Masked slots and positions
past a run load nothing, so rows no valid slot names are poisoned with NaN.
"""
import numpy as np
import pytest
import torch

import workloads
from test_parity_gpu import check, oracle_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smla():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mla_attention_fwd_amd as m
    return m


def _poison_unreferenced(x):
    idx = x["indices"].numpy()
    s_kv = x["kv"].shape[0]
    used = np.zeros(s_kv, dtype=bool)
    used[idx[(idx >= 0) & (idx < s_kv)]] = True
    kv = x["kv"].clone()
    kv[torch.from_numpy(~used)] = float("nan")
    return kv


def _run(smla, x, kv, **kw):
    dev = torch.device("cuda:0")
    out, lse = smla.sparse_mla_fwd(x["q"].to(dev), kv.to(dev), x["indices"].to(dev), x["sm_scale"], **kw)
    torch.cuda.synchronize()
    return out, lse


def _varied(seed, s_q, topk, s_kv=5000):
    """Tokens with very different valid-block counts."""
    x = workloads.make_random(s_q=s_q, h_q=64, topk=topk, s_kv=s_kv, seed=seed, invalid_frac=0.15,
                              dup_frac=0.05, q_mult=4.0)
    idx = x["indices"]
    rng = np.random.default_rng(seed)
    for t in range(s_q):
        kind = t % 6
        if kind == 1:
            idx[t, :] = -1                                   # no valid slot
        elif kind == 2:
            idx[t, 1:] = -1                                  # one block: only slot 0
        elif kind == 3:
            idx[t, : topk - 1] = 10 ** 7                     # only the last slot valid
        elif kind == 4:
            idx[t, int(rng.integers(1, topk)):] = -1         # trailing blocks masked
    return x


@pytest.mark.parametrize("workgroups", [1, 3, 7, 24])
@pytest.mark.parametrize("topk", [1024, 1100, 2048])
def test_persistent_runs_match_oracle_and_grid(smla, workgroups, topk):
    x = _varied(topk + workgroups, 24, topk)
    kv = _poison_unreferenced(x)
    po, pl = _run(smla, x, kv, schedule="persistent", persistent_workgroups=workgroups)
    go, gl = _run(smla, x, kv, schedule="grid", num_splits=1)
    ro, rl = oracle_tokens(x)
    check(po.float().cpu().numpy(), pl.cpu().numpy().astype(np.float64), ro, rl,
          f"persistent wg={workgroups} topk={topk}")
    assert torch.equal(po, go), "persistent output differs from the grid schedule"
    assert torch.equal(pl, gl), "persistent lse differs from the grid schedule"
    assert np.all(po[1::6].float().cpu().numpy() == 0) and torch.all(torch.isneginf(pl[1::6]))


def test_persistent_causal_stream(smla):
    """Causal-shaped weights: token t sees min(t + 1, topk) slots, so the
    first tokens are one block long and the runs of the workgroups hold very
    different token counts."""
    s_q, topk = 300, 1024
    x = workloads.make_random(s_q=s_q, h_q=64, topk=topk, s_kv=2000, seed=77, q_mult=4.0)
    idx = x["indices"]
    for t in range(s_q):
        idx[t, min(t + 1, topk):] = -1
    kv = _poison_unreferenced(x)
    po, pl = _run(smla, x, kv, schedule="persistent", persistent_workgroups=16)
    go, gl = _run(smla, x, kv, schedule="grid", num_splits=1)
    ro, rl = oracle_tokens(x)
    check(po.float().cpu().numpy(), pl.cpu().numpy().astype(np.float64), ro, rl, "persistent causal")
    assert torch.equal(po, go) and torch.equal(pl, gl)


def test_many_tokens_persistent_matches_grid(smla):
    """600 tokens on one persistent workgroup per compute unit against the
    grid's one workgroup per token (whose block counts are also computed
    ahead): same bits."""
    x = workloads.make_random(s_q=600, h_q=64, topk=1024, s_kv=30000, seed=78, invalid_frac=0.1)
    x["indices"][5, :] = -1
    ao, al = _run(smla, x, x["kv"], schedule="persistent")
    ro, rl = oracle_tokens(x)
    check(ao.float().cpu().numpy(), al.cpu().numpy().astype(np.float64), ro, rl, "persistent, 600 tokens")
    go, gl = _run(smla, x, x["kv"], schedule="grid", num_splits=1)
    assert torch.equal(ao, go) and torch.equal(al, gl)
    assert torch.all(ao[5] == 0) and torch.all(torch.isneginf(al[5]))
