"""B(b, S): the closed form used for MBU, pinned to (1) the oracle's own
enumeration of the bytes it reads and (2) the numbers the pages print for the
Qwen3-0.6B b1x128 cell."""
import json
import os

import numpy as np
import pytest

import oracle
from decode_megakernel_amd.bytes_model import step_bytes, weight_read_bytes, HBM_PEAK_BYTES_PER_S
from mkinputs import (QWEN3_06B, LLAMA3_8B, LLAMA2_13B, TINY_LLAMA, TINY_QWEN, SMALL_LLAMA_H64,
                      make_weights, make_kv_cache, bf16_bits, weight_specs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "forge_qwen3_0p6b_b1x128.json")


@pytest.mark.parametrize("shape", [TINY_LLAMA, TINY_QWEN, SMALL_LLAMA_H64.replace(n_layers=1)],
                         ids=lambda s: s.name)
def test_closed_form_equals_oracle_enumeration(shape):
    ctx = [3, 10, 1]
    w = make_weights(shape, 5)
    bits = {k: bf16_bits(v) for k, v in w.items()}
    K, V = make_kv_cache(shape, 5, ctx, 3, 16)
    W = oracle.Weights(shape, bits)
    kv = oracle.KVState(shape, bf16_bits(K), bf16_bits(V), ctx)
    oracle.decode_step(shape, W, kv, [1, 2, 3], ctx)
    enumerated = W.bytes_read + kv.stats["kv_bytes"]
    assert enumerated == step_bytes(shape, [c + 1 for c in ctx])


def test_weight_bytes_equal_tensor_inventory():
    # every tensor of the model once, except that the embedding contributes b
    # gathered rows; a tied model reads the table in full again as its head.
    for shape in (QWEN3_06B, LLAMA3_8B, LLAMA2_13B, TINY_QWEN):
        d, V = shape.hidden, shape.vocab
        for b in (1, 3, 16):
            total = 0
            for name, shp, _ in weight_specs(shape):
                total += b * d if name == "model.embed_tokens.weight" else int(np.prod(shp))
            if shape.tied_embeddings:
                total += V * d
            assert weight_read_bytes(shape, b) == 2 * total


def test_pages_qwen3_cell_pins_byte_count():
    g = json.load(open(GOLDEN))
    B = step_bytes(QWEN3_06B, [128])
    assert B == 1_206_781_952
    implied = B / (g["step_time_us"] * 1e-6 * g["h100_peak_bytes_per_s"])
    assert round(100 * implied, 1) == g["mbu_percent"]
    assert round(100 * g["mbu_percent"] / g["cell_ceiling_percent"], 1) == g["fraction_of_ceiling_percent"]


def test_untied_full_table_inflation_within_pages_bound():
    g = json.load(open(GOLDEN))
    for shape, S in ((LLAMA3_8B, [4097]), (LLAMA2_13B, [4000] * 16)):
        B = step_bytes(shape, S)
        full = B + 2 * shape.vocab * shape.hidden - 2 * len(S) * shape.hidden
        assert 1.0 < full / B <= g["untied_full_table_inflation_max"]


def test_peak_is_mi355x_hbm():
    assert HBM_PEAK_BYTES_PER_S == 8.0e12
