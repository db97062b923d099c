"""Seeded synthetic workloads for the paged-attention read path and its K/V
write (inputs only)."""
from .gen import (PagedInputs, MixedInputs, AppendInputs, RaggedInputs, pack_ragged, make_random,
                  SharedGroups, make_shared, c5_decode_grouped,
                  make_append, make_config,
                  make_c1, make_c2, make_c2_fp8, make_c3, make_c3_fp8, make_c4, make_c5, f32_to_bf16_bits,
                  bf16_bits_to_f32, SEEDS, GARBAGE_DEFAULT)

__all__ = ["PagedInputs", "MixedInputs", "AppendInputs", "RaggedInputs", "pack_ragged",
           "SharedGroups", "make_shared", "c5_decode_grouped",
           "make_random", "make_append",
           "make_config", "make_c1", "make_c2", "make_c2_fp8", "make_c3", "make_c3_fp8", "make_c4", "make_c5",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "SEEDS", "GARBAGE_DEFAULT"]
