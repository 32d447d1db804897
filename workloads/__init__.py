"""Seeded synthetic workloads (shapes and random draws) for paged decode attention."""
from .configs import (BASE_SEED, CHUNKED_PREFILL, CONFIGS, DecodeConfig, EXTRA_CONFIGS, FP8_LONG,
                      INT4_LONG, INT8_LONG, LLAMA3_70B_FULL, LLAMA3_8B_LAYER, SHARED_PREFIX_MQA, SPEC_VERIFY,
                      STREAMING_WINDOW, TINY, variant)
from .generate import (POISON_BF16, POISON_F16, POISON_I8, DecodeCase, bf16_bits_to_f32,
                       f32_to_bf16_bits, history_rows_device, make_case)

__all__ = [
    "BASE_SEED", "CONFIGS", "DecodeConfig", "EXTRA_CONFIGS", "STREAMING_WINDOW", "SPEC_VERIFY",
    "CHUNKED_PREFILL", "INT8_LONG", "INT4_LONG", "FP8_LONG", "LLAMA3_70B_FULL", "LLAMA3_8B_LAYER",
    "SHARED_PREFIX_MQA", "TINY", "variant", "POISON_BF16", "POISON_F16", "POISON_I8",
    "DecodeCase", "bf16_bits_to_f32", "f32_to_bf16_bits", "history_rows_device", "make_case",
]
