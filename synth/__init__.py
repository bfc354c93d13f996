"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package draws random numbers and describes workload shapes. It holds none
of the block's arithmetic: no normalisation, projection, rotary embedding,
attention or residual math lives here, so the oracle and the HIP path never
share any of the computation they are compared on.
"""
from .configs import DIMS, Dims, Segment, RopeLayout, WORKLOADS, workload
from .gen import (bf16_round_bits, bf16_bits_to_f32, block_weights, tokens,
                  modulation, modulation_weights, io_weights, edge_inputs, TEXT_DIM,
                  LATENT_DIM, WEIGHT_STD, MOD_STD)

__all__ = ["DIMS", "Dims", "Segment", "RopeLayout", "WORKLOADS", "workload",
           "bf16_round_bits", "bf16_bits_to_f32", "block_weights", "tokens",
           "modulation", "modulation_weights", "io_weights", "edge_inputs", "TEXT_DIM",
           "LATENT_DIM", "WEIGHT_STD", "MOD_STD"]
