"""Float64 CPU oracle of the decode step.

TEST INFRASTRUCTURE: only the test suite, the graft entry point's smoke check
and the benchmark's CPU-baseline leg may import it.  It shares no code with the
GPU path (which must fail loudly rather than fall back to anything here).
"""
from .decode import (bf16_to_f64, rms_norm, rope, rope_frequencies, softmax, attend, silu,
                     greedy_token, Weights, KVState, layer_forward, lm_head, decode_step)
