"""float64 oracle of the sparse MLA forward pass over a paged KV cache -- test
infrastructure (same rules as the rest of ``oracle/``).

Source: the page "Flash Attention Infer算子性能优化" (catlass), section
优化Paged Attention路径 (the paged-attention path).  There the KV cache is
stored in fixed-size pages (blocks) whose rows are contiguous, and a block
table per sequence names, in order, the physical page holding each logical
block of the sequence; the sequence length is rounded up to a whole number of
blocks.  The kernel reaches a KV row through that table.

Reading taken for the sparse forward pass (the page describes dense
attention, where every logical position up to the sequence length is used):

* A token's logical KV sequence is the concatenation of the pages its block
  table row names, in table order: logical position j is row j % page_size of
  page block_table[t, j // page_size].
* The token's indices name logical positions.  A slot is masked (weight zero,
  row never read) when its position is outside [0, table_width * page_size) or
  the table entry of its block is outside [0, num_pages) (an unallocated
  block, for example -1).
* Everything else is the definition of ``sparse_mla_fwd_exact`` applied to the
  token's logical sequence.
"""
from __future__ import annotations

import numpy as np

from .sparse_mla import sparse_mla_fwd_exact


def logical_sequence(kv_pages, block_table_row, page_size: int):
    """The token's logical KV sequence: its pages concatenated in table order.
    Returns (rows [width * page_size, d], present [width * page_size] bool);
    rows of an unallocated block are zero and not present."""
    kv_pages = np.asarray(kv_pages)
    num_pages = kv_pages.shape[0]
    blocks = []
    present = []
    for p in np.asarray(block_table_row):
        if 0 <= p < num_pages:
            blocks.append(np.asarray(kv_pages[p], dtype=np.float64))
            present.append(np.ones(page_size, dtype=bool))
        else:
            blocks.append(np.zeros(kv_pages.shape[1:], dtype=np.float64))
            present.append(np.zeros(page_size, dtype=bool))
    return np.concatenate(blocks, axis=0), np.concatenate(present)


def sparse_mla_fwd_paged(q, kv_pages, block_table, indices, sm_scale, d_v):
    """Sparse MLA forward with logical indices into each token's paged KV.

    q [s_q, h_q, d_qk], kv_pages [num_pages, page_size, d_qk] (float64 values
    of the stored rows), block_table [s_q, width] (physical page of each
    logical block), indices [s_q, topk] (logical positions).  Returns
    (out [s_q, h_q, d_v], lse [s_q, h_q]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    kv_pages = np.asarray(kv_pages)
    page_size = kv_pages.shape[1]
    block_table = np.asarray(block_table)
    indices = np.asarray(indices, dtype=np.int64)
    s_q, h_q, _ = q.shape
    out = np.zeros((s_q, h_q, d_v))
    lse = np.full((s_q, h_q), -np.inf)
    for t in range(s_q):
        seq, present = logical_sequence(kv_pages, block_table[t], page_size)
        idx = indices[t].copy()
        inside = (idx >= 0) & (idx < seq.shape[0])
        ok = inside.copy()
        ok[inside] = present[idx[inside]]
        idx[~ok] = -1                         # masked slot
        o, l = sparse_mla_fwd_exact(q[t:t + 1], seq, idx[None, :], sm_scale, d_v)
        out[t], lse[t] = o[0], l[0]
    return out, lse
