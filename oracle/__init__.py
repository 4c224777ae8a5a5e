"""CPU fp64 oracle for the MoBA prefill forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. It shares no code with the HIP path.
"""
from .moba import (NEAR_TIE_REL, algorithmic_flops, attend, attend_with_idx, attended_keys,
                   dense_attention, eligible_blocks, forward, forward_head, num_blocks,
                   pool_keys, select_blocks, theoretical_sparsity)

__all__ = ["NEAR_TIE_REL", "algorithmic_flops", "attend", "attend_with_idx", "attended_keys",
           "dense_attention", "eligible_blocks", "forward", "forward_head", "num_blocks",
           "pool_keys", "select_blocks", "theoretical_sparsity"]
