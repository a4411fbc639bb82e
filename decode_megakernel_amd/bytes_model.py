"""Algorithmic bytes per decode step, B(b, S), and model bandwidth utilization.

Following the ForgeMegakernel paper summary ("2.2 Model bandwidth
utilization"): MBU = B(b, S) / (step time x peak HBM bandwidth), where B counts
the model-dependent reads of one step -- every layer weight, the final norm,
the LM head, the KV rows attended -- and, for the embedding, only the b rows
gathered rather than the whole table.  For a tied model the LM head *is* the
embedding table and is read in full by the head.  All tensors are bf16.

Writes (new KV rows, activations, logits) and the RoPE table are not counted.
seq_lens[i] counts every position sequence i attends, the new one included.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12      # MI355X HBM3E


def layer_param_count(shape) -> int:
    d, hd, I = shape.hidden, shape.head_dim, shape.intermediate
    n = d * shape.q_dim + 2 * d * shape.kv_dim + shape.q_dim * d   # q, k, v, o
    n += 3 * d * I                                                  # gate, up, down
    n += 2 * d                                                      # two RMSNorm weights
    if shape.qk_norm:
        n += 2 * hd
    return n


def weight_read_bytes(shape, batch: int) -> int:
    d = shape.hidden
    n = shape.n_layers * layer_param_count(shape) + d + shape.vocab * d + batch * d
    return 2 * n


def kv_read_bytes(shape, seq_lens) -> int:
    return 2 * 2 * shape.n_layers * shape.n_kv_heads * shape.head_dim * sum(int(s) for s in seq_lens)


def step_bytes(shape, seq_lens) -> int:
    """B(b, S) for one decode step of len(seq_lens) sequences."""
    return weight_read_bytes(shape, len(seq_lens)) + kv_read_bytes(shape, seq_lens)


def mbu(shape, seq_lens, step_seconds: float, peak: float = HBM_PEAK_BYTES_PER_S) -> float:
    return step_bytes(shape, seq_lens) / (step_seconds * peak)
