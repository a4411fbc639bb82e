"""Seeded synthetic inputs and workload shapes, shared by the oracle's tests
and the GPU path.  Holds no decode arithmetic."""
from .configs import (ModelShape, Phase, Workload, WORKLOADS, SMOLLM2_135M, QWEN3_06B,
                      LLAMA32_1B, LLAMA3_8B, LLAMA2_13B, QWEN3_8B, TINY_LLAMA, TINY_QWEN,
                      SMALL_LLAMA_H64, SMALL_QWEN_H128, SMALL_MHA_H128, SMALL_MHA_H64, SMALL_WIDE_FFN)
from .generate import (BF16_NAN_SENTINEL, weight_specs, make_weights, make_tensor,
                       make_kv_cache, make_kv_layer, make_paged_kv, draw_contexts, draw_tokens, kv_capacity, bf16_bits,
                       lm_head_name)
