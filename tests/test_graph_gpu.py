"""HIP graph capture of the forward pass (torch.cuda.CUDAGraph on ROCm).

The entry points validate on the host and enqueue only kernel launches (no
allocation, no memset, no synchronisation), so a whole step can be captured
once and replayed, which removes the per-launch host overhead of decode
steps.  Each case captures one call with preallocated outputs and workspace,
replays the graph several times with the process's own eager work and
synchronisations in between, and checks every replay bit for bit against an
eager call of the same plan (the kernels are deterministic).
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smla():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mla_attention_fwd_amd as m  # loads libsmla.so; fails loudly if absent
    return m


def _inputs(kind):
    dev = torch.device("cuda:0")
    if kind == "bf16_split":
        x = workloads.make_random(s_q=16, h_q=128, topk=512, s_kv=8192, seed=71, invalid_frac=0.1)
        kw = dict(num_splits=4)
    elif kind == "persistent":
        x = workloads.make_random(s_q=20, h_q=64, topk=1100, s_kv=6000, seed=74, invalid_frac=0.2)
        x["indices"][3, :] = -1
        kw = dict(schedule="persistent", persistent_workgroups=4)
    elif kind == "paged":
        x = workloads.make_random_paged(s_q=8, h_q=64, topk=700, page_size=16, num_pages=80,
                                        table_width=64, seed=72, unallocated_frac=0.1)
        kw = dict(num_splits=2, block_table=x["block_table"].to(dev), page_size=16)
    else:
        x = workloads.make_random(s_q=8, h_q=64, topk=1500, s_kv=6000, seed=73, kv_format=kind)
        kw = dict(num_splits=2, kv_format=kind)
    q, idx = x["q"].to(dev), x["indices"].to(dev)
    if "kv" in x:
        kv = x["kv"].to(dev)
    else:
        import sparse_mla_attention_fwd_amd as m
        pack = m.pack_fp8_kv if kind == "fp8" else m.pack_fp4_kv
        kv = pack(x["kv_codes"], x["kv_scales"], dev)
    return q, kv, idx, x["sm_scale"], kw


@pytest.mark.parametrize("kind", ["bf16_split", "persistent", "paged", "fp8", "fp4"])
def test_graph_replays_match_eager(smla, kind):
    q, kv, idx, sm_scale, kw = _inputs(kind)
    dev = q.device
    s_q, h_q, _ = q.shape
    ref_out, ref_lse = smla.sparse_mla_fwd(q, kv, idx, sm_scale, **kw)
    out = torch.empty((s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s_q, h_q), dtype=torch.float32, device=dev)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up on the capture stream
        smla.sparse_mla_fwd(q, kv, idx, sm_scale, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        smla.sparse_mla_fwd(q, kv, idx, sm_scale, out=out, lse=lse, workspace=ws, **kw)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.zero_()
        ws.fill_(0xAB)                                  # stale scratch must not matter
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"{kind}: replay {rep} output differs"
        assert torch.equal(lse, ref_lse), f"{kind}: replay {rep} lse differs"
        smla.sparse_mla_fwd(q, kv, idx, sm_scale, **kw)  # eager work between replays
        torch.cuda.synchronize()
