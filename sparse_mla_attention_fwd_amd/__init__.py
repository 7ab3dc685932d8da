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
                   SMLA_KV_FP8_E4M3, SMLA_SCHEDULE_AUTO, SMLA_SCHEDULE_GRID, SMLA_SCHEDULE_PERSISTENT, SmlaError, make_paged, make_params, smla_fwd, smla_fwd_paged,
                   smla_fwd_paged_workspace_size, smla_fwd_plan, smla_fwd_schedule, smla_fwd_static_scratch,
                   smla_fwd_tune,
                   smla_fwd_tune_workspace_size, smla_fwd_workspace_size, smla_pack_fp4_kv_host,
                   smla_pack_fp8_kv_host)

__all__ = ["sparse_mla_fwd", "pack_fp8_kv", "pack_fp4_kv", "smla_fwd", "smla_fwd_static_scratch", "smla_fwd_plan",
           "smla_fwd_schedule",
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


_ROW_WIDTH = {SMLA_KV_BF16: D_QK, SMLA_KV_FP8_E4M3: FP8_ROW_BYTES, SMLA_KV_FP4_E2M1: FP4_ROW_BYTES}


def check_tensors(q, kv, indices, fmt, *, out=None, lse=None, workspace=None, block_table=None):
    """Reject, before any pointer reaches the library, what the C ABI cannot
    see: tensors on another device than q (a host pointer handed to a gather
    would fault the GPU), the wrong dtype or shape of an output (the kernels
    write bf16 out [s_q, h_q, 512] and float32 lse [s_q, h_q]), a strided
    innermost dimension, and an index table that does not have one row per
    query token.  kv is a 2-D table of rows here (a paged pool is flattened
    by the caller)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [s_q, h_q, {D_QK}], got {tuple(q.shape)}")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    if fmt == SMLA_KV_BF16 and kv.dtype != torch.bfloat16:
        raise TypeError("bf16 KV must be a bfloat16 tensor")
    if fmt != SMLA_KV_BF16 and kv.dtype != torch.uint8:
        raise TypeError("quantised KV must be a uint8 tensor of packed rows")
    if kv.dim() != 2 or kv.shape[1] < _ROW_WIDTH[fmt]:
        raise ValueError(f"kv must be a 2-D table of rows at least {_ROW_WIDTH[fmt]} wide, "
                         f"got {tuple(kv.shape)}")
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    if indices.dim() != 2 or indices.shape[0] != q.shape[0]:
        raise ValueError(f"indices must be [s_q, topk] with s_q = {q.shape[0]}, got {tuple(indices.shape)}")
    s_q, h_q = q.shape[0], q.shape[1]
    if out is not None:
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (s_q, h_q, D_V):
            raise ValueError(f"out must be bfloat16 [{s_q}, {h_q}, {D_V}], got {out.dtype} {tuple(out.shape)}")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (s_q, h_q):
            raise ValueError(f"lse must be float32 [{s_q}, {h_q}], got {lse.dtype} {tuple(lse.shape)}")
        if lse.stride(1) != 1:
            raise ValueError("lse must have its heads contiguous")
    named = [("q", q), ("kv", kv), ("indices", indices), ("out", out), ("lse", lse),
             ("workspace", workspace), ("block_table", block_table)]
    for name, t in named:
        if t is None:
            continue
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: every tensor must be on q's device")
        if t.dim() > 0 and t.numel() > 0 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have a contiguous innermost dimension")
    if block_table is not None and (block_table.dtype != torch.int32 or block_table.dim() != 2
                                    or block_table.shape[0] != s_q):
        raise ValueError("block_table must be an int32 [s_q, table_width] tensor")


def tune_plan(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float, *,
              kv_format: str = "bf16", iterations: int = 10) -> tuple[int, int, float]:
    """Time the library's candidate plans on these inputs (smla_fwd_tune) and
    return ``(num_splits, b_topk, microseconds)`` of the fastest; pass the
    first two to ``sparse_mla_fwd``.  Blocks until the timing is done."""
    if not q.is_cuda:
        raise ValueError("tune_plan runs on the GPU only: q must be a device tensor")
    fmt = {"bf16": SMLA_KV_BF16, "fp8": SMLA_KV_FP8_E4M3, "fp4": SMLA_KV_FP4_E2M1}[kv_format]
    check_tensors(q, kv, indices, fmt)
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
                   b_topk: int = 0, schedule: str = "auto", persistent_workgroups: int = 0,
                   out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream: int | None = None, block_table: torch.Tensor | None = None,
                   page_size: int | None = None):
    """Run the forward pass on the tensors' GPU and return ``(out, lse)``.

    q: bf16 [s_q, h_q, 576]; kv: bf16 [s_kv, 576] or, with ``kv_format="fp8"``,
    uint8 [s_kv, 640] packed rows (see ``pack_fp8_kv``), or with
    ``kv_format="fp4"`` uint8 [s_kv, 320] (see ``pack_fp4_kv``); indices: int32
    [s_q, topk].  Every tensor must be on q's device (pack the quantised rows
    with ``device=``).  ``num_splits``/``b_topk`` 0 let the library plan;
    ``schedule`` is ``"auto"``, ``"grid"`` (one workgroup per token, split
    and head group) or ``"persistent"`` (``persistent_workgroups`` workgroups,
    0 = one per compute unit, on runs of tokens of equal block weight).
    Outputs and the split workspace are allocated with torch unless given.

    Paged KV: ``block_table`` int32 [s_q, table_width] and ``page_size``; kv is
    then the page pool, [num_pages, page_size, 576] (bf16) or
    [num_pages, page_size, 640] (packed fp8), or the same rows flattened, and
    ``indices`` holds logical positions.
    """
    if not q.is_cuda:
        raise ValueError("sparse_mla_fwd runs on the GPU only: q must be a device tensor")
    if d_v != D_V:
        raise ValueError(f"d_v must be {D_V}")
    fmt = {"bf16": SMLA_KV_BF16, "fp8": SMLA_KV_FP8_E4M3, "fp4": SMLA_KV_FP4_E2M1}[kv_format]
    if (block_table is None) != (page_size is None):
        raise ValueError("block_table and page_size go together")
    if block_table is not None and kv.dim() == 3:
        kv = kv.reshape(kv.shape[0] * kv.shape[1], kv.shape[2])
    check_tensors(q, kv, indices, fmt, out=out, lse=lse, workspace=workspace, block_table=block_table)
    s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((s_q, h_q, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    sched = {"auto": SMLA_SCHEDULE_AUTO, "grid": SMLA_SCHEDULE_GRID,
             "persistent": SMLA_SCHEDULE_PERSISTENT}[schedule]
    p = make_params(q, kv, indices, sm_scale, out, lse, kv_format=fmt, num_splits=num_splits,
                    b_topk=b_topk, schedule=sched, persistent_workgroups=persistent_workgroups)
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
