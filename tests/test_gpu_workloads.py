"""Parity at the full sizes of the benchmark workloads, through the C ABI.

Three kinds of check, all against the float64 oracle on the same seeded
inputs the benchmark uses (same seeds, shapes, contexts, batch caps):

* complete mid-state parity (every layer's hidden state and mid-layer
  residual, the K/V rows written, logits, greedy tokens) for the workloads
  whose whole step the oracle finishes in seconds: SmolLM2-135M b1,
  Qwen3-0.6B b1, Llama-3.2-1B b8 ragged;
* for Llama-3-8B b1, Llama-3-8B b8 -> b9 and Llama-2-13B b16, where one
  float64 step over every layer takes minutes: the full model runs on the
  GPU and the oracle checks what it can compute from the original inputs
  alone -- the gathered embedding rows (bit-exact), the first layer's output,
  mid-layer residual and K/V rows -- plus properties that hold at any size
  (tokens are the argmax of the GPU's own logits, KV slot indexing is
  bit-exact on sampled layers, everything finite);
* complete parity for 2-layer models of the full 8B / 13B width at the same
  contexts and batches: every per-layer kernel shape, tiling and attention
  partition of the full model, with logits and tokens checked too.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Case, run_step, assert_step_ok, log, rel_l2, TOL
from decode_megakernel_amd.binding import DecodeEngine, STATE_HMID
from mkinputs import WORKLOADS, make_weights, make_kv_cache, bf16_bits, draw_contexts, draw_tokens, kv_capacity

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _contexts(wl, batch):
    return draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)[:batch]


@pytest.mark.parametrize("key", ["smollm2-135m-b1", "qwen3-0.6b-b1", "llama3.2-1b-b8"])
def test_full_workload_parity(key):
    wl = WORKLOADS[key]
    b = wl.phases[0].batch
    ctx = _contexts(wl, b)
    log(f"workload {key}: shape {wl.shape.name}, contexts {ctx}")
    case = Case(wl.shape, ctx, 2, seed=wl.seed, batch_cap=wl.batch_cap, keep_f64=True)
    try:
        for s in range(2):
            r = run_step(case, check_kv_invariant=True)
            log(f"  step {s}: {r}")
            assert_step_ok(r)
            assert r["k_err"] <= TOL and r["v_err"] <= TOL, r
            assert r["logits_err"] <= TOL, r
            assert r["tokens_oracle_ok"], r
    finally:
        case.close()
        del case
        _free()


def _check_first_layer_and_properties(shape, seed, batch_cap, ctx_by_step, sampled_layers):
    """Run the full model for len(ctx_by_step) steps (the batch may grow).
    Every step: tokens are the argmax of the GPU's logits, KV slot indexing is
    bit-exact on `sampled_layers`, logits are finite.  The oracle checks the
    embedding rows and layer 0 of every sequence whose inputs are still the
    original ones at that step (all of them at the first step, then the
    sequences that join), so no oracle input comes from the GPU."""
    all_ctx = ctx_by_step[-1]
    first_ctx = [ctx_by_step[0][i] if i < len(ctx_by_step[0]) else all_ctx[i] for i in range(len(all_ctx))]
    for s, ctx in enumerate(ctx_by_step):
        for i, c in enumerate(ctx):
            assert c == first_ctx[i] + sum(1 for t in range(s) if i < len(ctx_by_step[t]))
    seq_cap = kv_capacity(max(all_ctx) + 1, 1)
    w = make_weights(shape, seed, device="cuda")
    K, V = make_kv_cache(shape, seed, first_ctx, batch_cap, seq_cap, device="cuda")
    torch.cuda.synchronize()
    log(f"  weights and KV cache ready (seq_cap {seq_cap})")
    eng = DecodeEngine(shape, w, max_batch=batch_cap, max_seq=seq_cap)
    toks = draw_tokens(seed, len(all_ctx), shape.vocab)
    names = ["model.embed_tokens.weight"] + [n for n in w if n.startswith("model.layers.0.")]
    Wo = oracle.Weights(shape, {n: bf16_bits(w[n]) for n in names}, keep=True)
    try:
        for s, ctx in enumerate(ctx_by_step):
            b = len(ctx)
            fresh = list(range(len(ctx_by_step[s - 1]) if s else 0, b))
            tok_t = torch.tensor(toks[:b], dtype=torch.int32, device="cuda")
            pos_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
            logits = torch.full((b, shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
            nxt = torch.full((b,), -1, dtype=torch.int32, device="cuda")
            before = {l: (K[l].view(torch.int16).clone(), V[l].view(torch.int16).clone()) for l in sampled_layers}
            # prompt rows of layer 0 for the fresh sequences, as the oracle sees them
            k0 = {i: bf16_bits(K[0, i, :, :ctx[i], :]).copy() for i in fresh}
            v0 = {i: bf16_bits(V[0, i, :, :ctx[i], :]).copy() for i in fresh}
            eng.step(tok_t, pos_t, pos_t + 1, K, V, logits, nxt)
            torch.cuda.synchronize()
            st = eng.status()
            log(f"  step {s}: batch {b}, status {st}, oracle-checked sequences {fresh}")
            assert st == 0
            hidden = torch.empty((shape.n_layers + 1, b, shape.hidden), dtype=torch.float32, device="cuda")
            eng.copy_hidden(b, hidden)
            hmid = eng.state(STATE_HMID, b)
            torch.cuda.synchronize()
            g_logits = logits.cpu().numpy().astype(np.float64)
            g_next = nxt.cpu().numpy()
            # properties at any size
            assert np.all(np.isfinite(g_logits))
            own = [int(np.flatnonzero(g_logits[i] == g_logits[i].max())[0]) for i in range(b)]
            assert [int(t) for t in g_next] == own
            for l, (k_b, v_b) in before.items():
                ck = (K[l].view(torch.int16) != k_b).any(dim=-1)
                cv = (V[l].view(torch.int16) != v_b).any(dim=-1)
                exp = torch.zeros_like(ck)
                for i in range(b):
                    exp[i, :, ctx[i]] = True
                assert torch.equal(ck, exp) and torch.equal(cv, exp), f"KV slot indexing, layer {l}"
            del before
            # oracle: embedding rows and layer 0 of the fresh sequences
            xs = Wo.rows("model.embed_tokens.weight", np.asarray([toks[i] for i in fresh]))
            g_h0 = hidden[0].cpu().numpy().astype(np.float64)
            assert np.array_equal(g_h0[fresh], xs), "gathered embedding rows"
            pos_f = [ctx[i] for i in fresh]
            h1, hm, k_new, v_new = oracle.layer_forward(
                shape, Wo, 0, xs, pos_f,
                lambda j: (oracle.bf16_to_f64(k0[fresh[j]]), oracle.bf16_to_f64(v0[fresh[j]])))
            g_h1 = hidden[1].cpu().numpy().astype(np.float64)
            g_hm = hmid[0].cpu().numpy().astype(np.float64)
            errs = []
            for j, i in enumerate(fresh):
                errs.append(rel_l2(g_h1[i], h1[j]))
                errs.append(rel_l2(g_hm[i], hm[j]))
                errs.append(rel_l2(K[0, i, :, ctx[i], :].float().cpu().numpy(), k_new[j]))
                errs.append(rel_l2(V[0, i, :, ctx[i], :].float().cpu().numpy(), v_new[j]))
            log(f"  layer 0 max rel L2 {max(errs):.3e}")
            assert max(errs) <= TOL
            toks[:b] = [int(t) for t in g_next]
    finally:
        eng.close()
        del w, K, V
        _free()


@pytest.mark.parametrize("key", ["llama3-8b-b1", "llama3-8b-b8to9", "llama2-13b-b16"])
def test_full_model_first_layer_and_invariants(key):
    wl = WORKLOADS[key]
    sh = wl.shape
    base = draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)
    if len(wl.phases) == 1:
        b = wl.phases[0].batch
        ctx_by_step = [base[:b]]
    else:
        # batch growth: one step with the first phase's batch, then the next
        # step with one more sequence joining at its own position
        b0, b1 = wl.phases[0].batch, wl.phases[1].batch
        ctx_by_step = [base[:b0], [c + 1 for c in base[:b0]] + base[b0:b1]]
    log(f"workload {key}: shape {sh.name}, steps {[len(c) for c in ctx_by_step]}")
    _check_first_layer_and_properties(sh, wl.seed, wl.batch_cap, ctx_by_step,
                                      sampled_layers=sorted({0, sh.n_layers // 2, sh.n_layers - 1}))


@pytest.mark.parametrize("key", ["llama3-8b-b1", "llama3-8b-b8to9", "llama2-13b-b16"])
def test_full_width_two_layers(key):
    wl = WORKLOADS[key]
    sh = wl.shape.replace(n_layers=2)
    b = wl.phases[-1].batch
    ctx = _contexts(wl, b)
    log(f"workload {key} at 2 layers: contexts {ctx}")
    case = Case(sh, ctx, 1, seed=wl.seed, batch_cap=wl.batch_cap, keep_f64=False)
    try:
        r = run_step(case, check_kv_invariant=True)
        log(f"  {r}")
        assert_step_ok(r)
        assert r["k_err"] <= TOL and r["v_err"] <= TOL, r
        assert r["logits_err"] <= TOL, r
        assert r["tokens_oracle_ok"], r
    finally:
        case.close()
        del case
        _free()
