"""CPU oracle for the sparse MLA attention forward pass (test infrastructure).

This package is the checker, not the product.  Only ``tests/``, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library: it never imports
``sparse_mla_attention_fwd_amd`` and the library never imports it.  The only
code both sides use is the seeded input generator in ``workloads/``, which
holds none of the method's arithmetic.

Everything here is plain numpy in float64.  The functions take already
materialised inputs (bf16 or fp8 values upcast exactly to float64) and follow
the page "Ascend Sparse Attention Forward 算法与优化技术简析":

* ``sparse_mla_fwd_exact`` -- the definition in its section 数学建模
  (mathematical model): gather, P = Q·Gᵀ, S = softmax(P·sm_scale),
  out = S·G[:, :d_v], plus the per-row log-sum-exp the section 计算流程
  maintains.
* ``sparse_mla_fwd_online`` -- the block-wise online-softmax algorithm with
  the "skip scale" rule of section 计算流程 (computation flow), step by step.
* ``lse_combine`` / ``sparse_mla_fwd_split`` -- split-topk partial results
  merged by their log-sum-exp weights (the decode split; the pages are silent
  on it, so it is the standard exact merge of two softmax partitions).
* ``sparse_mla_fwd_paged`` -- the same definition over a paged KV cache
  reached through a per-token block table (page "Flash Attention
  Infer算子性能优化", section 优化Paged Attention路径).
* ``e2m1_decode`` / ``dequant_fp4_rows`` -- the fp4 KV-cache values, decoded
  from the OCP Microscaling specification's E2M1 element format.
* ``e4m3fn_decode`` / ``dequant_fp8_rows`` -- the fp8 KV-cache values,
  decoded from the OCP 8-bit floating point specification (E4M3, "fn"
  variant: no infinities, max 448).
"""
from .sparse_mla import (  # noqa: F401
    RESCALE_THRES,
    sparse_mla_fwd_exact,
    sparse_mla_fwd_online,
    sparse_mla_fwd_split,
    lse_combine,
    valid_slot_mask,
)
from .fp8 import e4m3fn_decode, dequant_fp8_rows, FP8_GROUP  # noqa: F401
from .fp4 import e2m1_decode, dequant_fp4_rows  # noqa: F401
from .paged import sparse_mla_fwd_paged, logical_sequence  # noqa: F401
