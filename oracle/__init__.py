"""FP64 CPU oracle for the BF16 attention forward.

TEST INFRASTRUCTURE ONLY: ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package; the HIP library and its binding never do. It shares
no code with the GPU path; only the seeded input generators (``workloads``) feed both.
Every function cites the passage of the pages it follows.
"""
from .attention import (attention_dense, attention_rows, attention_varlen, bf16_bits_to_f64,
                        scale_as_used, softmax_probabilities)
from .compare import LSE_TOL, MAX_ABS_TOL, REL_L2_TOL, bf16_faithful, bf16_round_f64, bf16_spacing, compare
from .prologue import grid_positions, pair_frequencies, qk_norm, qk_norm_rope, v_head_major

__all__ = ["attention_dense", "attention_rows", "attention_varlen", "bf16_bits_to_f64",
           "scale_as_used", "softmax_probabilities", "compare", "REL_L2_TOL", "MAX_ABS_TOL", "LSE_TOL",
           "bf16_faithful", "bf16_round_f64", "bf16_spacing",
           "grid_positions", "pair_frequencies", "qk_norm", "qk_norm_rope", "v_head_major"]
