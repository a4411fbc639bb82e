"""Parity of the HIP decode step against the float64 oracle, through the C ABI.

Small shapes span several 16-row tiles, ragged K tails, multi-chunk split-KV
attention pieces and ragged batches; the full-size workloads are checked in
test_gpu_workloads.py."""
import pytest
import torch

from gpu_harness import Case, run_step, assert_step_ok, log
from mkinputs import TINY_LLAMA, TINY_QWEN, SMALL_LLAMA_H64, SMALL_QWEN_H128, SMALL_MHA_H128, SMALL_MHA_H64

pytestmark = pytest.mark.gpu

CASES = [
    # (shape, contexts, steps)
    (TINY_LLAMA, [5], 3),
    (TINY_QWEN, [9], 3),
    (TINY_LLAMA, [0], 2),                     # first token: attends only to itself
    (TINY_QWEN, [3, 40, 1, 77], 3),          # ragged batch
    (SMALL_LLAMA_H64, [100, 7, 250], 3),     # hd 64, G 4, untied, split-K down
    (SMALL_QWEN_H128, [300], 3),             # hd 128, QK-norm, multi-chunk attention
    (SMALL_MHA_H128, [64, 129, 1, 500, 33], 2),  # MHA, ragged
    (SMALL_LLAMA_H64, [17] * 8, 2),          # batch 8: MFMA tiles, equal lengths
    (SMALL_QWEN_H128, [5, 300, 77, 1000, 2, 64, 129, 511, 3], 2),  # batch 9 ragged MFMA
    (SMALL_MHA_H128, [int(x) for x in torch.randint(1, 600, (16,), generator=torch.Generator().manual_seed(3))], 2),
    (SMALL_MHA_H64, [0, 63, 64, 65, 300, 1], 3),  # MHA at head_dim 64: one K/V row per lane, chunk edges
    (SMALL_MHA_H64, [int(x) for x in torch.randint(1, 400, (12,), generator=torch.Generator().manual_seed(5))], 2),
]


@pytest.mark.parametrize("shape,contexts,steps", CASES,
                         ids=[f"{c[0].name}-b{len(c[1])}-{i}" for i, c in enumerate(CASES)])
def test_parity_small(shape, contexts, steps):
    log(f"case {shape.name} contexts={contexts} steps={steps}")
    case = Case(shape, contexts, steps, seed=4321)
    try:
        for s in range(steps):
            r = run_step(case)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
    finally:
        case.close()
