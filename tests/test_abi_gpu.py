"""The checks only the launching entry points make (workspace size and
alignment), exercised with real device buffers.  Every buffer is large enough
for the launch it describes, and a too-small workspace is only declared too
small: should a check ever regress, the kernels would still stay inside
allocated memory."""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_mla_attention_fwd_amd import _lib
    return _lib


def _setup(_lib, num_splits=3, paged=False):
    dev = torch.device("cuda:0")
    x = workloads.make_random(s_q=4, h_q=64, topk=300, s_kv=1024, seed=9)
    q, kv, idx = x["q"].to(dev), x["kv"].to(dev), x["indices"].to(dev)
    out = torch.empty((4, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((4, 64), dtype=torch.float32, device=dev)
    p = _lib.make_params(q, kv, idx, x["sm_scale"], out, lse, num_splits=num_splits)
    keep = [q, kv, idx, out, lse]
    g = None
    if paged:
        bt = torch.arange(64, dtype=torch.int32, device=dev).repeat(4, 1)   # identity table, 16-row pages
        g = _lib.make_paged(bt, 16)
        keep.append(bt)
    need = _lib.smla_fwd_paged_workspace_size(p, g) if paged else _lib.smla_fwd_workspace_size(p)
    ws = torch.empty(need + 512, dtype=torch.uint8, device=dev)
    keep.append(ws)
    return p, g, need, ws, keep


def test_split_workspace_too_small_or_misaligned_is_rejected(lib):
    p, _, need, ws, keep = _setup(lib)
    dll = lib.load()
    assert need > 0
    base = (ws.data_ptr() + 255) // 256 * 256
    p.workspace, p.workspace_bytes = base, need - 1
    assert dll.smla_fwd(ctypes.byref(p), None) == lib.SMLA_ERR_WORKSPACE
    p.workspace, p.workspace_bytes = base + 16, need
    assert dll.smla_fwd(ctypes.byref(p), None) == lib.SMLA_ERR_INVALID_ARGUMENT
    p.workspace, p.workspace_bytes = base, need
    assert dll.smla_fwd(ctypes.byref(p), None) == lib.SMLA_OK
    torch.cuda.synchronize()


def test_paged_workspace_too_small_or_misaligned_is_rejected(lib):
    p, g, need, ws, keep = _setup(lib, paged=True)
    dll = lib.load()
    base = (ws.data_ptr() + 255) // 256 * 256
    p.workspace, p.workspace_bytes = base, need - 1
    assert dll.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == lib.SMLA_ERR_WORKSPACE
    p.workspace, p.workspace_bytes = base + 16, need
    assert dll.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == lib.SMLA_ERR_INVALID_ARGUMENT
    p.workspace, p.workspace_bytes = base, need
    assert dll.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == lib.SMLA_OK
    torch.cuda.synchronize()


def test_tune_workspace_too_small_is_rejected(lib):
    p, _, _, _, keep = _setup(lib)
    dll = lib.load()
    need = lib.smla_fwd_tune_workspace_size(p)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda:0")
    base = (ws.data_ptr() + 255) // 256 * 256
    p.workspace, p.workspace_bytes = base, need - 1
    ns, bt, us = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    assert dll.smla_fwd_tune(ctypes.byref(p), None, 2, ctypes.byref(ns), ctypes.byref(bt),
                             ctypes.byref(us)) == lib.SMLA_ERR_WORKSPACE
    torch.cuda.synchronize()
