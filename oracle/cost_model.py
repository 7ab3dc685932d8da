"""The page's compute-versus-memory model -- test infrastructure.

Page "Ascend Sparse Attention Forward 算法与优化技术简析", section 讨论 /
"每个 AI Core 负责多少个 q head" (how many q heads per AI core): per core and
per query token, matrix-unit cycles are h_q * topk * (d + d) / FMA-per-cycle
(the two products QK^T and PV, each h_q * topk * d multiply-adds), and memory
cycles are the bytes of Q and O (h_q * d * 2 * 2) plus the gathered KV
(topk * d * 2) divided by the per-core, per-cycle share of the L2 bandwidth.

The page prints this model's output for its own chip; the golden fixture
``tests/golden/ascend_cost_model.txt`` holds that printed table.  With
MI355X constants the same model tells which unit, the matrix cores or the
memory system, bounds the kernel.
"""
from __future__ import annotations


def cost_model_cycles(h_q: int, topk: int, d: int, fma_per_cycle: int,
                      l2_bytes_per_s: float, num_cores: int, freq_hz: float):
    """(matrix-unit cycles, memory cycles) per core for one query token."""
    cube_cycles = h_q * topk * (d + d) // fma_per_cycle
    l2_bw = l2_bytes_per_s / num_cores / freq_hz
    qo_mem = h_q * d * 2 * 2
    kv_mem = topk * d * 2
    return cube_cycles, (qo_mem + kv_mem) / l2_bw
