"""Stage placement of the host schedule (no GPU: mk_plan builds and validates
the per-CU streams on the host).

Rules pinned here:
  * a row-owner stage avoids the CUs of the previous stage when that stage
    left CUs idle and avoiding them raises its sub-tiles per CU by at most
    one;
  * attention numbers first the CUs its layer's QKV stage left idle, and
    the slot cap is their count;
  * the O projection then avoids the capped attention CUs;
  * every layer's attention slot map is a permutation of the CUs.
"""
import math

import pytest

from decode_megakernel_amd import binding
from mkinputs import LLAMA3_8B, LLAMA32_1B, QWEN3_06B, SMOLLM2_135M, TINY_LLAMA, TINY_QWEN

QKV, ATTN, O, GU, DOWN, LM = range(6)


def _tiles(shape, stage):
    rows = {QKV: (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim, O: shape.hidden,
            GU: 2 * shape.intermediate, DOWN: shape.hidden}[stage]
    return math.ceil(rows / 16)


def test_qwen3_b1_consecutive_stages_use_disjoint_cus():
    st = binding.plan(QWEN3_06B, 1, 256)
    cus, shared = st["stage_cus"], st["stage_shared_prev"]
    # O and down (64 tiles each) leave 192 CUs idle: QKV and gate/up take those
    assert cus[O] == _tiles(QWEN3_06B, O) and cus[DOWN] == _tiles(QWEN3_06B, DOWN)
    assert cus[QKV] == 256 - cus[DOWN] and cus[GU] == 256 - cus[O]
    # attention is capped at the CUs QKV left idle; O avoids them
    assert st["attn_slot_cap"] == 256 - cus[QKV] == cus[ATTN]
    for stage in (QKV, ATTN, O, GU, DOWN):
        assert shared[stage] == 0, (stage, shared)
    assert st["attn_slots_valid"] == 1


def test_skip_needs_at_most_one_more_subtile_per_cu():
    # QKV of Qwen3: 256 sub-tiles on 192 CUs is two per CU instead of one: allowed
    st = binding.plan(QWEN3_06B, 1, 256)
    assert math.ceil(_tiles(QWEN3_06B, QKV) / st["stage_cus"][QKV]) == math.ceil(_tiles(QWEN3_06B, QKV) / 256) + 1
    # SmolLM2: gate/up (192 sub-tiles) avoids the 36 O CUs at one sub-tile per CU
    st = binding.plan(SMOLLM2_135M, 1, 256)
    assert st["stage_cus"][GU] == _tiles(SMOLLM2_135M, GU) and st["stage_shared_prev"][GU] == 0


def test_no_idle_cus_means_no_skipping_and_no_attention_cap():
    # Llama-3-8B at batch 1: every layer stage has at least one sub-tile per CU
    st = binding.plan(LLAMA3_8B, 1, 256)
    assert st["stage_cus"][:5] == [256] * 5
    assert st["stage_shared_prev"][:5] == [256] * 5
    assert st["attn_slot_cap"] == 0 and st["attn_slots_valid"] == 1


@pytest.mark.parametrize("shape,batch,ncu", [(QWEN3_06B, 1, 256), (SMOLLM2_135M, 1, 256), (LLAMA32_1B, 8, 256),
                                             (LLAMA3_8B, 9, 256), (TINY_QWEN, 3, 64), (TINY_LLAMA, 5, 40)])
def test_attention_slots_are_permutations(shape, batch, ncu):
    st = binding.plan(shape, batch, ncu, max_batch=16)
    assert st["attn_slots_valid"] == 1
    assert 0 <= st["attn_slot_cap"] < ncu
    # a cap, when set, is the number of CUs QKV left idle
    if st["attn_slot_cap"]:
        assert st["attn_slot_cap"] == ncu - st["stage_cus"][QKV]


def _stage_balance(shape, batch):
    """Per GEMV stage (layer 0, and the LM head): mean / max weight bytes per
    CU over the 256 CUs, and the most K windows one CU's K-split units span
    (each distinct window is one more staging of the input), from the
    exported task streams."""
    streams, _ = binding.plan_streams(shape, batch, 256)
    per, wins, ksplit = {}, {}, set()
    for c, tasks in enumerate(streams):
        for t in tasks:
            if t["type"] == 2 and (t["layer"] == 0 or t["stage"] == LM):
                per.setdefault(t["stage"], [0] * 256)[c] += 16 * t["nsub"] * (t["k1"] - t["k0"]) * 2
                if t["flags"] & 2:  # a K-split piece
                    ksplit.add(t["stage"])
                    wins.setdefault(t["stage"], [set() for _ in range(256)])[c].add(t["k0"])
    bal = {st: sum(v) / len(v) / max(v) for st, v in per.items()}
    return bal, {st: max(len(x) for x in v) for st, v in wins.items()}, ksplit


@pytest.mark.parametrize("key,batch", [("llama3.2-1b-b8", 8), ("llama3-8b-b1", 1), ("llama3-8b-b8to9", 8),
                                       ("llama3-8b-b8to9", 9), ("llama2-13b-b16", 16)])
def test_large_stages_are_balanced(key, batch):
    """Gate/up, down and the LM head (the stages that carry most weight
    bytes) put within 3% of the mean number of bytes on the busiest CU, or
    within 7% for K-split stages, whose units are dealt piece by piece so
    that every CU stages a single input window (a CU that straddled two
    pieces restaged and ran ~9 us behind, more than the extra unit costs).
    QKV and O may be coarser: their finer tilings measured slower (one-tile
    stream-K groups, row-owner, stream-K instead of K-split)."""
    from mkinputs import WORKLOADS
    bal, wins, ksplit = _stage_balance(WORKLOADS[key].shape, batch)
    for st in (GU, DOWN, LM):
        assert bal[st] >= (0.93 if st in ksplit else 0.97), (key, batch, st, bal)
    for st in ksplit:
        assert wins[st] == 1, (key, batch, st, wins)
    assert min(bal.values()) >= 0.74, bal
