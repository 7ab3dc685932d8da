"""Sparse MLA attention forward for AMD MI355X (gfx950).

``sparse_mla_fwd(q, kv, indices, sm_scale) -> (out, lse)`` computes, for every
query token t independently (page "Ascend Sparse Attention Forward
算法与优化技术简析", section 数学建模):

    G = kv[indices[t]]                      (slots outside [0, s_kv) are masked)
    out[t] = softmax(q[t] @ G.T * sm_scale) @ G[:, :512]       bf16 [h_q, 512]
    lse[t] = logsumexp(q[t] @ G.T * sm_scale)                  fp32 [h_q]

with hand-written HIP kernels behind the C ABI in ``include/smla.h``.  With a
``block_table`` the KV is a paged cache and the indices are logical positions
(page "Flash Attention Infer算子性能优化", section 优化Paged Attention路径):
position j of token t is row j % page_size of page block_table[t, j // page_size].
This module only marshals tensors; there is no CPU path.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (D_QK, D_V, FP4_ROW_BYTES, FP8_ROW_BYTES, SMLA_KV_BF16, SMLA_KV_FP4_E2M1,  # noqa: F401
                   SMLA_KV_FP8_E4M3, SmlaError, make_paged, make_params, smla_fwd, smla_fwd_paged,
                   smla_fwd_paged_workspace_size, smla_fwd_plan, smla_fwd_tune,
                   smla_fwd_tune_workspace_size, smla_fwd_workspace_size, smla_pack_fp4_kv_host,
                   smla_pack_fp8_kv_host)

__all__ = ["sparse_mla_fwd", "pack_fp8_kv", "pack_fp4_kv", "smla_fwd", "smla_fwd_plan",
           "smla_fwd_workspace_size", "smla_fwd_paged", "smla_fwd_paged_workspace_size",
           "smla_fwd_tune", "smla_fwd_tune_workspace_size", "tune_plan", "smla_pack_fp8_kv_host",
           "smla_pack_fp4_kv_host", "SmlaError"]


def pack_fp8_kv(codes: torch.Tensor, scales: torch.Tensor, device=None) -> torch.Tensor:
    """fp8 KV cache in the library's row format (codes and scales of a token
    side by side, 640 bytes per row), optionally moved to ``device``."""
    packed = smla_pack_fp8_kv_host(codes.cpu(), scales.cpu())
    return packed.to(device) if device is not None else packed


def pack_fp4_kv(codes: torch.Tensor, scales: torch.Tensor, device=None) -> torch.Tensor:
    """fp4 KV cache in the library's row format (two E2M1 codes per byte, the
    five group scales beside them, 320 bytes per row), optionally moved to
    ``device``."""
    packed = smla_pack_fp4_kv_host(codes.cpu(), scales.cpu())
    return packed.to(device) if device is not None else packed


def tune_plan(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float, *,
              kv_format: str = "bf16", iterations: int = 10) -> tuple[int, int, float]:
    """Time the library's candidate plans on these inputs (smla_fwd_tune) and
    return ``(num_splits, b_topk, microseconds)`` of the fastest; pass the
    first two to ``sparse_mla_fwd``.  Blocks until the timing is done."""
    fmt = {"bf16": SMLA_KV_BF16, "fp8": SMLA_KV_FP8_E4M3, "fp4": SMLA_KV_FP4_E2M1}[kv_format]
    s_q, h_q, _ = q.shape
    out = torch.empty((s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    p = make_params(q, kv, indices, sm_scale, out, lse, kv_format=fmt)
    need = smla_fwd_tune_workspace_size(p)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    return smla_fwd_tune(p, iterations)


def sparse_mla_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                   d_v: int = D_V, *, kv_format: str = "bf16", num_splits: int = 0,
                   b_topk: int = 0, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream: int | None = None, block_table: torch.Tensor | None = None,
                   page_size: int | None = None):
    """Run the forward pass on the tensors' GPU and return ``(out, lse)``.

    q: bf16 [s_q, h_q, 576]; kv: bf16 [s_kv, 576] or, with ``kv_format="fp8"``,
    uint8 [s_kv, 640] packed rows (see ``pack_fp8_kv``), or with
    ``kv_format="fp4"`` uint8 [s_kv, 320] (see ``pack_fp4_kv``); indices: int32
    [s_q, topk].  ``num_splits``/``b_topk`` 0 let the library plan.  Outputs and
    the split workspace are allocated with torch unless given.

    Paged KV: ``block_table`` int32 [s_q, table_width] and ``page_size``; kv is
    then the page pool, [num_pages, page_size, 576] (bf16) or
    [num_pages, page_size, 640] (packed fp8), or the same rows flattened, and
    ``indices`` holds logical positions.
    """
    if not q.is_cuda:
        raise ValueError("sparse_mla_fwd runs on the GPU only: q must be a device tensor")
    fmt = {"bf16": SMLA_KV_BF16, "fp8": SMLA_KV_FP8_E4M3, "fp4": SMLA_KV_FP4_E2M1}[kv_format]
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    if fmt == SMLA_KV_BF16 and kv.dtype != torch.bfloat16:
        raise TypeError("bf16 KV must be a bfloat16 tensor")
    if fmt != SMLA_KV_BF16 and kv.dtype != torch.uint8:
        raise TypeError("quantised KV must be a uint8 tensor of packed rows")
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    if (block_table is None) != (page_size is None):
        raise ValueError("block_table and page_size go together")
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise TypeError("block_table must be an int32 [s_q, table_width] tensor")
        if not block_table.is_cuda or block_table.shape[0] != q.shape[0]:
            raise ValueError("block_table must be a device tensor with one row per query token")
        if kv.dim() == 3:
            kv = kv.reshape(kv.shape[0] * kv.shape[1], kv.shape[2])
    s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((s_q, h_q, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    p = make_params(q, kv, indices, sm_scale, out, lse, kv_format=fmt, num_splits=num_splits,
                    b_topk=b_topk)
    paged = make_paged(block_table, page_size) if block_table is not None else None
    need = smla_fwd_workspace_size(p) if paged is None else smla_fwd_paged_workspace_size(p, paged)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if paged is None:
        smla_fwd(p, stream)
    else:
        smla_fwd_paged(p, paged, stream)
    return out, lse
