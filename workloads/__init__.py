"""Seeded synthetic workloads (inputs only) for the paged-KV attention path."""
from .gen import (BLOCK, PRESETS, PagedBatch, f32_to_bf16_bits, make_batch,
                  long_context, mixed_prefill, norm_weights, packed_qkv,
                  qwen25_05b_decode, qwen3_06b_decode, tiny_f32)

__all__ = ["BLOCK", "PRESETS", "PagedBatch", "f32_to_bf16_bits", "make_batch",
           "long_context", "mixed_prefill", "norm_weights", "packed_qkv", "qwen25_05b_decode",
           "qwen3_06b_decode", "tiny_f32"]
