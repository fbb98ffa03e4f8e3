"""Seeded synthetic inputs shared by the CPU oracle and the GPU path (no attention arithmetic here)."""
from .gen import (ROW_DIM, LATENT_DIM, ROPE_DIM, SOFTMAX_SCALE_F32, WORKLOADS, Workload, Inputs,
                  generate, ragged, Ragged, rope_cache, decode_positions, poison_unused, permute_pages, repack, gather_rows,
                  f32_to_bf16_bits, f32_to_e4m3fn_codes, BF16_NAN, FP8_NAN)

__all__ = ["ROW_DIM", "LATENT_DIM", "ROPE_DIM", "SOFTMAX_SCALE_F32", "WORKLOADS", "Workload", "Inputs",
           "generate", "ragged", "Ragged", "rope_cache", "decode_positions", "poison_unused", "permute_pages", "repack", "gather_rows",
           "f32_to_bf16_bits", "f32_to_e4m3fn_codes", "BF16_NAN", "FP8_NAN"]
