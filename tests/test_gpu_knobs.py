"""Every schedule and tile variant the planner can choose, checked against the
float64 oracle through the C ABI (the environment switches are read when a
handle is created):

  * MK_KSPLIT_MIN_WINDOWS=2 forces K-split stages (pieces publish partial
    tiles, finish tasks sum them) wherever a task needs two input windows,
    on the VALU (batch 7) and MFMA (batch 9, 16) tiles;
  * MK_GEMV_MODE=1 forces row-owner tiling, =2 stream-K tiling, for every stage;
  * MK_MFMA_MIN_BATCH=4 runs batches 4-7 on the MFMA tiles;
  * MK_KSPLIT=0 turns K-split off (Llama-2-13B-width model at batch 16);
  * MK_KSPLIT_ALIGNED=0 deals K-split units evenly over the CUs instead of
    piece by piece; MK_NUM_CU=2 runs on two CUs (fewer CUs than K pieces).
The default choices are covered by the other parity tests."""
import pytest

from gpu_harness import Case, run_step, assert_step_ok, log
from mkinputs import SMALL_WIDE_FFN, SMALL_MHA_H128, SMALL_LLAMA_H64

pytestmark = pytest.mark.gpu

CTX7 = [3, 40, 1, 77, 9, 120, 15]
CTX9 = [5, 300, 77, 100, 2, 64, 129, 211, 3]
CTX16 = [12, 1, 40, 77, 5, 300, 19, 2, 60, 150, 33, 8, 90, 4, 250, 7]

CASES = [
    ({"MK_KSPLIT_MIN_WINDOWS": "2"}, SMALL_WIDE_FFN, CTX7),
    ({"MK_KSPLIT_MIN_WINDOWS": "2"}, SMALL_WIDE_FFN, CTX9),
    ({"MK_KSPLIT_MIN_WINDOWS": "2"}, SMALL_MHA_H128, CTX16),
    ({"MK_GEMV_MODE": "1"}, SMALL_LLAMA_H64, CTX9),
    ({"MK_GEMV_MODE": "1"}, SMALL_LLAMA_H64, CTX7[:2]),
    ({"MK_GEMV_MODE": "2"}, SMALL_LLAMA_H64, CTX9),
    ({"MK_GEMV_MODE": "2"}, SMALL_WIDE_FFN, CTX7[:5]),
    ({"MK_MFMA_MIN_BATCH": "4"}, SMALL_LLAMA_H64, CTX7[:4]),
    ({"MK_MFMA_MIN_BATCH": "4"}, SMALL_MHA_H128, CTX7),
    ({"MK_KSPLIT": "0"}, SMALL_MHA_H128, CTX16),
    # K-split units dealt evenly over the CUs (not piece by piece), and a
    # 2-CU launch with fewer CUs than K pieces
    ({"MK_KSPLIT_MIN_WINDOWS": "2", "MK_KSPLIT_ALIGNED": "0"}, SMALL_WIDE_FFN, CTX9),
    ({"MK_KSPLIT_MIN_WINDOWS": "2", "MK_NUM_CU": "2"}, SMALL_WIDE_FFN, CTX9),
]


@pytest.mark.parametrize("env,shape,contexts", CASES,
                         ids=[f"{'-'.join(k + v for k, v in c[0].items())}-{c[1].name}-b{len(c[2])}"
                              for c in CASES])
def test_knob_parity(monkeypatch, env, shape, contexts):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    log(f"env {env} shape {shape.name} contexts {contexts}")
    case = Case(shape, contexts, 2, seed=2024)
    for k in env:
        monkeypatch.delenv(k)
    try:
        for s in range(2):
            r = run_step(case)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
    finally:
        case.close()


@pytest.mark.parametrize("bound,ctx", [(64, [3, 40, 1, 60]), (400, [100, 7, 250]), (3000, [5, 300, 77, 1000, 2, 64, 129, 511, 3])],
                         ids=["bound64-b4", "bound400-b3", "bound3000-b9"])
def test_context_routing_parity(bound, ctx):
    """Steps routed to a context bucket (mk_set_context_bound) match the oracle."""
    log(f"context bound {bound} contexts {ctx}")
    case = Case(SMALL_MHA_H128 if len(ctx) < 9 else SMALL_LLAMA_H64, ctx, 2, seed=2025)
    case.engine.set_context_bound(bound)
    try:
        for s in range(2):
            r = run_step(case)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
    finally:
        case.close()
