"""Parity at the full sizes of the benchmark workloads, through the C ABI.

Every workload runs its full model on the GPU and is compared with the
float64 oracle on the same seeded inputs the benchmark uses (same seeds,
shapes, contexts, batch caps) at every mid-state of every layer: the hidden
state entering and leaving each layer, the mid-layer residual, the K/V rows
written, logits and greedy tokens (teacher-forced), with KV slot indexing
checked bit-exact over the whole cache.

* SmolLM2-135M b1, Qwen3-0.6B b1 and Llama-3.2-1B b8 ragged run several steps
  with host copies of the whole cache;
* Llama-3-8B b1 (2 steps), Llama-3-8B b8 -> b9 (a step at batch 8, then the
  step where the ninth sequence joins, all nine sequences compared) and
  Llama-2-13B b16 (one step) take the oracle's prompt K/V rows, and the
  slot-indexing reference, from the seeded generator one layer at a time (the
  cache does not fit the host twice), never from the cache the kernel writes;
* 2-layer models of the full 8B / 13B width run every per-layer kernel shape,
  tiling and attention partition of the full model for a few steps.
"""
import gc

import pytest
import torch

import json

from gpu_harness import Case, run_step, assert_step_ok, log, TOL, LOGPROB_TOL
from mkinputs import WORKLOADS, draw_contexts, kv_capacity

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _contexts(wl, batch):
    return draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)[:batch]


def _run(case, batches, tag):
    worst = {}
    lp = []
    for s, b in enumerate(batches):
        r = run_step(case, check_kv_invariant=True, batch=b)
        lp += r["logprob_err"]
        log(f"  {tag} step {s} (batch {b}): {r}")
        assert_step_ok(r)
        for k in ("hidden_err", "hmid_err", "logits_err", "k_err", "v_err"):
            worst[k] = max(worst.get(k, 0.0), r[k])
    log(f"  {tag} worst over {len(batches)} steps: {worst}")
    # mean absolute log-probability error of the greedy tokens against float64
    rec = {"workload": tag, "tokens": len(lp), "mean_logprob_err": sum(lp) / len(lp), "max_logprob_err": max(lp),
           **{f"max_{k}": v for k, v in worst.items()}}
    log("LOGPROB " + json.dumps(rec))
    assert rec["mean_logprob_err"] <= LOGPROB_TOL, rec
    return worst


# steps compared per small workload: every step of SmolLM2's and Qwen3's
# runs, and the first 8 of Llama-3.2-1B's 32
SMALL_STEPS = {"smollm2-135m-b1": 8, "qwen3-0.6b-b1": 64, "llama3.2-1b-b8": 8}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["smollm2-135m-b1", "qwen3-0.6b-b1", "llama3.2-1b-b8"])
def test_full_workload_parity(key):
    wl = WORKLOADS[key]
    b = wl.phases[0].batch
    n = SMALL_STEPS[key]
    ctx = _contexts(wl, b)
    log(f"workload {key}: shape {wl.shape.name}, contexts {ctx}, {n} steps")
    case = Case(wl.shape, ctx, n, seed=wl.seed, batch_cap=wl.batch_cap,
                seq_cap=kv_capacity(max(ctx) + 1, wl.total_steps), keep_f64=True)
    try:
        _run(case, [b] * n, key)
    finally:
        case.close()
        del case
        _free()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("key", ["llama3-8b-b1", "llama3-8b-b8to9", "llama2-13b-b16"])
def test_full_depth_large(key):
    wl = WORKLOADS[key]
    sh = wl.shape
    ctx = draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)
    if len(wl.phases) == 1:
        b = wl.phases[0].batch
        batches = [b, b] if b == 1 else [b]
        ctx = ctx[:b]
    else:
        # batch growth: a step with the first phase's batch, then the step in
        # which the next sequence joins with its own prompt and first token
        batches = [wl.phases[0].batch, wl.phases[1].batch]
    log(f"workload {key}: shape {sh.name}, batches {batches}, contexts {ctx}")
    case = Case(sh, ctx, len(batches), seed=wl.seed, batch_cap=wl.batch_cap,
                seq_cap=kv_capacity(max(ctx) + 1, wl.total_steps), keep_f64=False, lazy_kv=True)
    log("  inputs ready")
    try:
        _run(case, batches, key)
    finally:
        case.close()
        del case
        _free()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key", ["llama3-8b-b1", "llama3-8b-b8to9", "llama2-13b-b16"])
def test_full_width_two_layers(key):
    wl = WORKLOADS[key]
    sh = wl.shape.replace(n_layers=2)
    ctx = _contexts(wl, wl.batch_cap)
    batches = [p.batch for p in wl.phases for _ in range(2)]
    log(f"workload {key} at 2 layers: contexts {ctx}, batches {batches}")
    case = Case(sh, ctx, len(batches), seed=wl.seed, batch_cap=wl.batch_cap, keep_f64=False)
    try:
        _run(case, batches, key + "-2l")
    finally:
        case.close()
        del case
        _free()
