"""Seeded synthetic attention inputs (BF16 bit patterns), shared by the oracle tests and the HIP path."""
from .synth import (WORKLOADS, Workload, f32_to_bf16_bits, make_dense, make_linear_inputs, make_projected, make_ragged, make_varlen,
                    random_dense, random_varlen, rmsnorm_rows, rope_interleaved, rope_tables,
                    sample_rows)

__all__ = ["WORKLOADS", "Workload", "f32_to_bf16_bits", "make_dense", "make_linear_inputs", "make_projected", "make_ragged", "make_varlen",
           "random_dense", "random_varlen", "rmsnorm_rows", "rope_interleaved", "rope_tables",
           "sample_rows"]
