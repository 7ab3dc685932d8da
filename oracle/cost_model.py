"""The page's compute-versus-memory model of one query token -- test
infrastructure.

Page "Ascend Sparse Attention Forward 算法与优化技术简析", section 讨论 /
"每个 AI Core 负责多少个 q head" (how many q heads per AI core).  The model
asks, for one query token on one core, whether the matrix unit or the memory
system takes longer:

* work: the two products QKᵀ and PV each take h_q · topk · d multiply-adds
  (the page uses one width d for keys and values), so the matrix unit needs
  2 · h_q · topk · d / (multiply-adds per cycle) cycles, rounded down to whole
  cycles;
* traffic: the token's Q is read and its output written (h_q · d bf16 values
  each way) and its topk gathered rows are read (d bf16 values each); the
  core's share of the L2 bandwidth, per clock cycle, turns those bytes into
  cycles.

The page prints this model's output for its own chip; the golden fixture
``tests/golden/ascend_cost_model.txt`` holds that printed table.
"""
from __future__ import annotations

BF16_BYTES = 2


def cost_model_cycles(h_q: int, topk: int, d: int, fma_per_cycle: int,
                      l2_bytes_per_s: float, num_cores: int, freq_hz: float):
    """(matrix-unit cycles, memory cycles) per core for one query token."""
    macs = 2 * h_q * topk * d                        # QKᵀ and PV
    matrix_cycles = macs // fma_per_cycle
    q_and_out_bytes = 2 * h_q * d * BF16_BYTES       # read Q, write the output
    gathered_bytes = topk * d * BF16_BYTES           # the token's KV rows
    bytes_per_core_cycle = l2_bytes_per_s / (num_cores * freq_hz)
    return matrix_cycles, (q_and_out_bytes + gathered_bytes) / bytes_per_core_cycle
