"""Model shapes and decode workloads used by the tests and the benchmark.

Pure data: this module holds no part of the decode arithmetic, so both the
float64 oracle and the GPU path may import it.

The five workloads are the ones the decode-megakernel pages evaluate on a
single GPU (ForgeMegakernel, "5.1 Setup": bf16 weights and KV cache, batch
1-16, contexts up to a few thousand).  Shapes follow the public Hugging Face
configurations of the named model families; values the pages do not fix
(rope theta for two families, RMSNorm epsilon) take the family defaults.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied_embeddings: bool
    qk_norm: bool
    rope_theta: float
    rms_eps: float

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class Phase:
    """A run of `steps` greedy decode steps at a fixed batch.

    `contexts[i]` is the number of cached positions sequence i has before the
    phase's first step (for a sequence continuing from an earlier phase it is
    implied by that phase and left as None here).
    """
    batch: int
    steps: int


@dataclass(frozen=True)
class Workload:
    key: str
    shape: ModelShape
    seed: int
    batch_cap: int
    ctx_lo: int            # prompt context drawn uniformly in [ctx_lo, ctx_hi]
    ctx_hi: int
    phases: tuple = field(default_factory=tuple)
    note: str = ""

    @property
    def total_steps(self) -> int:
        return sum(p.steps for p in self.phases)

    @property
    def max_batch(self) -> int:
        return max(p.batch for p in self.phases)


SMOLLM2_135M = ModelShape("smollm2-135m", 30, 576, 9, 3, 64, 1536, 49152,
                          True, False, 1e4, 1e-5)
QWEN3_06B = ModelShape("qwen3-0.6b", 28, 1024, 16, 8, 128, 3072, 151936,
                       True, True, 1e6, 1e-6)
LLAMA32_1B = ModelShape("llama3.2-1b", 16, 2048, 32, 8, 64, 8192, 128256,
                        True, False, 5e5, 1e-5)
LLAMA3_8B = ModelShape("llama3-8b", 32, 4096, 32, 8, 128, 14336, 128256,
                       False, False, 5e5, 1e-5)
LLAMA2_13B = ModelShape("llama2-13b", 40, 5120, 40, 40, 128, 13824, 32000,
                        False, False, 1e4, 1e-5)
# the model of the pages' context-length sweep (Qwen3-8B: QK-norm, untied)
QWEN3_8B = ModelShape("qwen3-8b", 36, 4096, 32, 8, 128, 12288, 151936,
                      False, True, 1e6, 1e-6)

WORKLOADS = {
    "smollm2-135m-b1": Workload(
        "smollm2-135m-b1", SMOLLM2_135M, 1001, 1, 128, 128, (Phase(1, 8),),
        "batch 1, 128 prompt positions, 8 greedy steps"),
    "qwen3-0.6b-b1": Workload(
        "qwen3-0.6b-b1", QWEN3_06B, 1002, 1, 1024, 1024, (Phase(1, 64),),
        "batch 1, context 1024, 64 greedy steps"),
    "llama3.2-1b-b8": Workload(
        "llama3.2-1b-b8", LLAMA32_1B, 1003, 8, 64, 4096, (Phase(8, 32),),
        "ragged batch of 8, contexts uniform in [64, 4096], 32 steps"),
    "llama3-8b-b1": Workload(
        "llama3-8b-b1", LLAMA3_8B, 1004, 1, 4096, 4096, (Phase(1, 32),),
        "batch 1 at context 4096, 32 steps"),
    "llama3-8b-b8to9": Workload(
        "llama3-8b-b8to9", LLAMA3_8B, 1014, 9, 256, 8192, (Phase(8, 16), Phase(9, 16)),
        "ragged batch of 8 (contexts uniform in [256, 8192]) for 16 steps, then a "
        "9th sequence joins with its own prompt for 16 more steps"),
    "llama2-13b-b16": Workload(
        "llama2-13b-b16", LLAMA2_13B, 1005, 16, 512, 8192, (Phase(16, 32),),
        "ragged batch of 16, contexts uniform in [512, 8192], 32 steps"),
}

# Small shapes that the oracle finishes in well under a second yet still
# span several 16-row tiles, K-blocks with a ragged tail and multi-chunk
# attention.  Used by parity tests.
TINY_LLAMA = ModelShape("tiny-llama", 2, 192, 4, 2, 64, 320, 1000,
                        True, False, 1e4, 1e-5)
TINY_QWEN = ModelShape("tiny-qwen", 2, 256, 4, 2, 64, 384, 777,
                       True, True, 1e6, 1e-6)
SMALL_LLAMA_H64 = ModelShape("small-llama-h64", 3, 512, 8, 2, 64, 1408, 4000,
                             False, False, 5e5, 1e-5)
SMALL_QWEN_H128 = ModelShape("small-qwen-h128", 2, 768, 8, 4, 128, 2048, 3000,
                             True, True, 1e6, 1e-6)
SMALL_MHA_H128 = ModelShape("small-mha-h128", 2, 640, 5, 5, 128, 1792, 2000,
                            False, False, 1e4, 1e-5)
SMALL_MHA_H64 = ModelShape("small-mha-h64", 2, 384, 6, 6, 64, 1024, 1500,
                           True, False, 1e4, 1e-5)
# A 2-layer model wide enough (hidden 2048, 4 K blocks; down projection 8 K
# blocks) that row-owner tasks at batch 7 and above need several LDS input
# windows, so the K-split tiles run on both the VALU and the MFMA path.
SMALL_WIDE_FFN = ModelShape("small-wide-ffn", 2, 2048, 16, 4, 128, 4096, 8000,
                            False, False, 1e4, 1e-5)
