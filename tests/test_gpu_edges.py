"""Edge cases of the decode step, through the C ABI, against the float64 oracle.

  * an empty batch enqueues nothing: outputs and cache stay as they were, and
    the next step is bit-identical to one with no empty call before it;
  * the last KV slot of the cache (p = seq_cap - 1) is written and attended
    like any other, and nothing past it changes;
  * a batch smaller than the engine's capacity and a KV cache with more
    sequence rows than the batch: only rows 0..b-1 change."""
import pytest
import torch

from decode_megakernel_amd.binding import DecodeEngine
from gpu_harness import Case, run_step, assert_step_ok, log
from mkinputs import TINY_LLAMA, TINY_QWEN, SMALL_QWEN_H128, make_weights, make_kv_cache

pytestmark = pytest.mark.gpu


def test_empty_batch_is_a_noop():
    sh = TINY_QWEN
    ctx = [6, 11]
    w = make_weights(sh, 17, device="cuda")
    K, V = make_kv_cache(sh, 17, ctx, len(ctx), 32, device="cuda")
    K0, V0 = K.clone(), V.clone()
    dev = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    toks, pos, lens = dev([4, 9]), dev(ctx), dev([c + 1 for c in ctx])
    eng = DecodeEngine(sh, w, max_batch=len(ctx), max_seq=32)
    try:
        ref_logits = torch.empty((2, sh.vocab), dtype=torch.float32, device="cuda")
        ref_next = torch.empty(2, dtype=torch.int32, device="cuda")
        eng.step(toks, pos, lens, K, V, ref_logits, ref_next)
        torch.cuda.synchronize()
        assert eng.status() == 0
        K.copy_(K0)
        V.copy_(V0)
        # batch 0: the outputs keep their sentinels, the cache its bytes
        logits = torch.full((2, sh.vocab), float("nan"), dtype=torch.float32, device="cuda")
        nxt = torch.full((2,), -7, dtype=torch.int32, device="cuda")
        eng.step(toks, pos, lens, K, V, logits, nxt, batch=0)
        torch.cuda.synchronize()
        assert eng.status() == 0
        assert bool(torch.isnan(logits).all()) and bool((nxt == -7).all())
        assert torch.equal(K.view(torch.int16), K0.view(torch.int16)) and torch.equal(V.view(torch.int16), V0.view(torch.int16))
        # the next real step is the same step as before
        eng.step(toks, pos, lens, K, V, logits, nxt)
        torch.cuda.synchronize()
        log(f"after an empty call: tokens {nxt.tolist()} reference {ref_next.tolist()}")
        assert eng.status() == 0
        assert torch.equal(logits, ref_logits) and torch.equal(nxt, ref_next)
    finally:
        eng.close()


def test_last_kv_slot():
    # seq_cap 64: step 0 writes position 62, step 1 position 63 (the last slot)
    case = Case(SMALL_QWEN_H128, [62, 5], 2, seed=808, seq_cap=64)
    log(f"case {case.shape.name} contexts {case.contexts} seq_cap {case.seq_cap}")
    try:
        for s in range(2):
            r = run_step(case)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
    finally:
        case.close()


def test_batch_below_capacity():
    # engine sized for 16 sequences, cache for 5, batch of 3
    case = Case(TINY_LLAMA, [4, 0, 31], 2, seed=99, batch_cap=5, engine_max_batch=16)
    log(f"case {case.shape.name} contexts {case.contexts} batch_cap {case.batch_cap} engine max_batch 16")
    try:
        for s in range(2):
            r = run_step(case)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
    finally:
        case.close()
