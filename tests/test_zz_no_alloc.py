"""smla_fwd_static_scratch: the forward pass with the split partials in the
library's static per-device scratch instead of a caller workspace, for callers
that cannot allocate.  Called through the C ABI and compared with smla_fwd (the
same plan with a caller workspace) bit for bit, and with the float64 oracle to
the parity bar, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's larger contents)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from test_parity_gpu import check, oracle_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_mla_attention_fwd_amd import _lib
    return _lib


def _call(_lib, x, num_splits, kv_format="bf16", **extra):
    """(static-scratch result, workspace result) of one configuration."""
    import sparse_mla_attention_fwd_amd as smla
    dev = torch.device("cuda:0")
    q, idx = x["q"].to(dev), x["indices"].to(dev)
    if kv_format == "bf16":
        kv, fmt = x["kv"].to(dev), _lib.SMLA_KV_BF16
    else:
        kv, fmt = smla.pack_fp8_kv(x["kv_codes"], x["kv_scales"], dev), _lib.SMLA_KV_FP8_E4M3
    s_q, h_q, _ = q.shape
    res = []
    for static in (True, False):
        out = torch.full((s_q, h_q, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((s_q, h_q), float("nan"), dtype=torch.float32, device=dev)
        p = _lib.make_params(q, kv, idx, x["sm_scale"], out, lse, kv_format=fmt, num_splits=num_splits,
                             **extra)
        need = _lib.smla_fwd_workspace_size(p)
        assert 0 < need <= _lib.STATIC_SCRATCH_BYTES
        stream = torch.cuda.current_stream().cuda_stream
        if static:
            st = _lib.load().smla_fwd_static_scratch(ctypes.byref(p), ctypes.c_void_p(stream))
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            p.workspace, p.workspace_bytes = ws.data_ptr(), need
            st = _lib.load().smla_fwd(ctypes.byref(p), ctypes.c_void_p(stream))
        assert st == _lib.SMLA_OK, _lib.last_error()
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def test_static_scratch_matches_workspace_on_two_calls_in_a_row(lib):
    # call 1: a decode-like split plan with a large partial region
    big = workloads.make_random(s_q=24, h_q=128, topk=512, s_kv=9000, seed=501, invalid_frac=0.1, q_mult=2.0)
    big["indices"][3, :] = -1                       # one token without a valid slot
    # call 2: a smaller plan over different data, in the scratch call 1 left behind
    small = workloads.make_random(s_q=5, h_q=64, topk=300, s_kv=4000, seed=502, invalid_frac=0.3)
    small["indices"][1, :200] = -1                  # its first splits empty
    for x, ns, what in ((big, 4, "first call"), (small, 3, "second, smaller call")):
        (so, sl), (wo, wl) = _call(lib, x, ns)
        assert torch.equal(so, wo), f"{what}: output differs from smla_fwd"
        assert torch.equal(sl, wl), f"{what}: lse differs from smla_fwd"
        ro, rl = oracle_tokens(x)
        check(so.float().cpu().numpy(), sl.cpu().numpy().astype(np.float64), ro, rl, what)


def test_static_scratch_fp8_and_single_split(lib):
    x = workloads.make_random(s_q=6, h_q=64, topk=1700, s_kv=5000, seed=503, kv_format="fp8", invalid_frac=0.2)
    (so, sl), (wo, wl) = _call(lib, x, 2, kv_format="fp8")
    assert torch.equal(so, wo) and torch.equal(sl, wl)
    # a one-split plan needs no scratch at all
    import sparse_mla_attention_fwd_amd as smla
    dev = torch.device("cuda:0")
    y = workloads.make_random(s_q=3, h_q=16, topk=100, s_kv=500, seed=504)
    q, kv, idx = y["q"].to(dev), y["kv"].to(dev), y["indices"].to(dev)
    out = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((3, 16), dtype=torch.float32, device=dev)
    p = lib.make_params(q, kv, idx, y["sm_scale"], out, lse, num_splits=1)
    lib.smla_fwd_static_scratch(p)
    torch.cuda.synchronize()
    ref = smla.sparse_mla_fwd(q, kv, idx, y["sm_scale"], num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])


def test_static_scratch_persistent_schedule(lib):
    """The persistent schedule keeps its per-token block counts in the scratch."""
    x = workloads.make_random(s_q=30, h_q=64, topk=1100, s_kv=5000, seed=505, invalid_frac=0.2)
    x["indices"][4, :] = -1
    (so, sl), (wo, wl) = _call(lib, x, 1, schedule=lib.SMLA_SCHEDULE_PERSISTENT, persistent_workgroups=5)
    assert torch.equal(so, wo) and torch.equal(sl, wl)
    ro, rl = oracle_tokens(x)
    check(so.float().cpu().numpy(), sl.cpu().numpy().astype(np.float64), ro, rl, "static persistent")
