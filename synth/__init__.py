"""Seeded synthetic inputs shared by the oracle side and the HIP side.

Random draws and data layout only; no arithmetic of the method lives here.
"""
from .configs import CONFIGS, ORDERED, PAGE_SIZE, MLAConfig, small  # noqa: F401
from .gen import (Workload, bf16_bits_to_f32, block_table, f32_to_bf16_bits,  # noqa: F401
                  append_recipe, chain_recipe, generate, hidden_recipe, pages_per_seq, query, query_multi,
                  seq_lens,
                  sequence_rows, token_chunk, weights)
