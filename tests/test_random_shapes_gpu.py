"""GPU parity over seeded random configurations: head counts, KV formats,
block sizes, split counts, ragged topk, small and large caches, masked and
repeated slots, large logits.  Each case is drawn from its own seed, so a
failure names a reproducible configuration."""
import numpy as np
import pytest
import torch

import workloads
from oracle import dequant_fp4_rows, dequant_fp8_rows, sparse_mla_fwd_exact
from test_parity_gpu import check

pytestmark = pytest.mark.gpu

MAX_PART = {"bf16": 2048, "fp8": 1536, "fp4": 2048}


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    fmt = ["bf16", "fp8", "fp4"][seed % 3]
    h_q = int(rng.choice([16, 32, 64, 128]))
    topk = int(rng.choice([1, 7, 31, 32, 33, 95, 128, 129, 300, 511, 1000, 1537, 2048, 2500]))
    s_kv = int(rng.choice([1, 40, 3000, 70000]))
    min_ns = -(-topk // MAX_PART[fmt])
    ns = int(rng.choice([0, min_ns, min_ns + 1, min_ns + 4]))
    b_topk = int(rng.choice([0, 32, 64])) if fmt == "bf16" else 0
    return dict(fmt=fmt, h_q=h_q, topk=topk, s_kv=s_kv, num_splits=ns, b_topk=b_topk,
                invalid=float(rng.choice([0.0, 0.3, 0.9])), dup=float(rng.choice([0.0, 0.2])),
                q_mult=float(rng.choice([1.0, 4.0, 8.0])), s_q=int(rng.integers(1, 5)))


@pytest.mark.parametrize("seed", range(24))
def test_random_configuration(seed):
    c = draw(seed)
    dev = torch.device("cuda:0")
    import sparse_mla_attention_fwd_amd as smla
    x = workloads.make_random(s_q=c["s_q"], h_q=c["h_q"], topk=c["topk"], s_kv=c["s_kv"], seed=seed,
                              invalid_frac=c["invalid"], dup_frac=c["dup"], q_mult=c["q_mult"],
                              kv_format=c["fmt"])
    q, idx = x["q"].to(dev), x["indices"].to(dev)
    if c["fmt"] == "bf16":
        kv = x["kv"].to(dev)
        rows = workloads.to_f64(x["kv"])
    else:
        pack = smla.pack_fp8_kv if c["fmt"] == "fp8" else smla.pack_fp4_kv
        dq = dequant_fp8_rows if c["fmt"] == "fp8" else dequant_fp4_rows
        kv = pack(x["kv_codes"], x["kv_scales"], dev)
        rows = dq(x["kv_codes"].numpy(), x["kv_scales"].numpy())
    out, lse = smla.sparse_mla_fwd(q, kv, idx, x["sm_scale"], kv_format=c["fmt"],
                                   num_splits=c["num_splits"], b_topk=c["b_topk"])
    torch.cuda.synchronize()
    ro, rl = sparse_mla_fwd_exact(workloads.to_f64(x["q"]), rows, x["indices"].numpy(), x["sm_scale"], 512)
    check(out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), ro, rl, f"seed {seed}: {c}")
