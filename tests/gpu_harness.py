"""Drives the HIP decode step and the float64 oracle on the same seeded
inputs and compares every mid-state.

Bars (from the decode-megakernel contract):
  * h_0 (gathered embedding rows): bit-exact;
  * hidden states after every layer, the K/V rows written, logits:
    relative L2 <= 1e-2 against float64, per (mid-state, layer, sequence);
  * KV-cache slot indexing: bit-exact -- exactly the rows (l, i, g, p_i)
    change in a step, every other byte of the cache is untouched;
  * greedy tokens: bit-exact against the argmax (lowest index on ties) of the
    GPU's own fp32 logits, and equal to the oracle's token whenever the
    oracle's top-1/top-2 gap exceeds twice the largest logit error (else the
    step is a certified near-tie, counted).
The oracle is teacher-forced with the GPU's tokens so trajectories stay
aligned; it keeps its own float64 rows for appended positions.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
from decode_megakernel_amd.binding import DecodeEngine, STATE_HMID
from mkinputs import make_weights, make_kv_cache, make_kv_layer, bf16_bits, draw_tokens

TOL = 1e-2
# mean absolute error of the greedy token's log-probability against float64
LOGPROB_TOL = 1e-2


def rel_l2(g, r) -> float:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / (den if den > 0 else 1.0))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class PromptKV:
    """The prompt K/V rows of one layer at a time, regenerated on the GPU from
    the seeded input recipe (never read from the cache the kernel writes), for
    the oracle and for the slot-indexing check of large caches."""

    def __init__(self, shape, seed, contexts, batch_cap, seq_cap, verbose=True):
        self.args = (shape, seed, list(contexts), batch_cap, seq_cap)
        self.l = None
        self.kv = None
        self.verbose = verbose

    def layer(self, l):
        if self.l != l:
            self.kv = None
            torch.cuda.empty_cache()
            sh, seed, ctx, bc, sc = self.args
            self.kv = make_kv_layer(sh, seed, ctx, bc, sc, l, device="cuda")
            self.l = l
            if self.verbose and (l % 8 == 0 or l == sh.n_layers - 1):
                log(f"    prompt K/V of layer {l} regenerated")
        return self.kv


class LazyBits:
    """Array-like view [l, i, :, :c, :] of prompt K (which=0) or V (which=1)
    bits for oracle.KVState: host uint16 copies of one sequence's rows."""

    def __init__(self, src: PromptKV, which: int):
        self.src, self.which = src, which

    def __getitem__(self, idx):
        l, i = int(idx[0]), int(idx[1])
        t = self.src.layer(l)[self.which]
        return bf16_bits(t[(i,) + tuple(idx[2:])])


class Case:
    """Seeded inputs on the GPU plus host copies for the oracle.

    `contexts` lists every sequence that takes part at some step (its prompt
    is in the cache from the start); a step runs the first `batch` of them.
    With lazy_kv the oracle's prompt rows and the slot-indexing check use
    regenerated layers instead of host copies of the whole cache."""

    def __init__(self, shape, contexts, steps, seed=1234, batch_cap=None, seq_cap=None, keep_f64=True,
                 engine_max_batch=None, lazy_kv=False):
        self.shape = shape
        self.contexts = list(contexts)
        self.b = len(contexts)
        self.batch_cap = batch_cap or self.b
        self.seq_cap = seq_cap or (max(contexts) + steps + 1)
        self.seed = seed
        self.lazy = lazy_kv
        dev = "cuda"
        self.w = make_weights(shape, seed, device=dev)
        self.K, self.V = make_kv_cache(shape, seed, self.contexts, self.batch_cap, self.seq_cap, device=dev)
        torch.cuda.synchronize()
        self.W = oracle.Weights(shape, {k: bf16_bits(v) for k, v in self.w.items()}, keep=keep_f64)
        if lazy_kv:
            self.prompt = PromptKV(shape, seed, self.contexts, self.batch_cap, self.seq_cap)
            self.kvs = oracle.KVState(shape, LazyBits(self.prompt, 0), LazyBits(self.prompt, 1), self.contexts)
        else:
            self.kvs = oracle.KVState(shape, bf16_bits(self.K), bf16_bits(self.V), self.contexts)
        self.engine = DecodeEngine(shape, self.w, max_batch=engine_max_batch or self.batch_cap,
                                   max_seq=self.seq_cap)
        self.tokens = draw_tokens(seed, self.b, shape.vocab)
        self.done = [0] * self.b      # steps each sequence has taken
        self.step_idx = 0

    def close(self):
        self.engine.close()


def _kv_index_lazy(case, b, pos):
    """Every layer: the cache differs from the regenerated prompt layer in
    exactly the rows the steps so far wrote (bit-exact slot indexing)."""
    sh = case.shape
    ok = True
    for l in range(sh.n_layers):
        k0, v0 = case.prompt.layer(l)
        ck = (case.K[l].view(torch.int16) != k0.view(torch.int16)).any(dim=-1)  # [B, nkv, S]
        cv = (case.V[l].view(torch.int16) != v0.view(torch.int16)).any(dim=-1)
        exp = torch.zeros_like(ck)
        for i in range(case.b):
            if case.done[i]:
                exp[i, :, case.contexts[i]:case.contexts[i] + case.done[i]] = True
        ok = ok and bool(torch.equal(ck, exp) and torch.equal(cv, exp))
        del ck, cv, exp
    return ok


def run_step(case: Case, check_kv_invariant=True, compare=True, batch=None):
    """One GPU step for the first `batch` sequences (default: all) + one
    oracle step; returns a dict of errors."""
    sh = case.shape
    b = case.b if batch is None else batch
    L, d, V = sh.n_layers, sh.hidden, sh.vocab
    pos = [case.contexts[i] + case.done[i] for i in range(b)]
    dev = "cuda"
    tok_t = torch.tensor(case.tokens[:b], dtype=torch.int32, device=dev)
    pos_t = torch.tensor(pos, dtype=torch.int32, device=dev)
    len_t = pos_t + 1
    logits = torch.full((b, V), float("nan"), dtype=torch.float32, device=dev)
    nxt = torch.full((b,), -1, dtype=torch.int32, device=dev)
    if check_kv_invariant and not case.lazy:
        K0 = case.K.view(torch.int16).clone()
        V0 = case.V.view(torch.int16).clone()
    case.engine.step(tok_t, pos_t, len_t, case.K, case.V, logits, nxt)
    torch.cuda.synchronize()
    status = case.engine.status()
    hidden = torch.empty((L + 1, b, d), dtype=torch.float32, device=dev)
    case.engine.copy_hidden(b, hidden)
    hmid = case.engine.state(STATE_HMID, b)
    torch.cuda.synchronize()
    for i in range(b):
        case.done[i] += 1
    out = {"status": status, "batch": b}
    # --- KV slot indexing, bit-exact
    if check_kv_invariant:
        if case.lazy:
            out["kv_index_ok"] = _kv_index_lazy(case, b, pos)
        else:
            ck = (case.K.view(torch.int16) != K0).any(dim=-1)  # [L, B, nkv, S]
            cv = (case.V.view(torch.int16) != V0).any(dim=-1)
            exp = torch.zeros_like(ck)
            for i in range(b):
                exp[:, i, :, pos[i]] = True
            out["kv_index_ok"] = bool(torch.equal(ck, exp) and torch.equal(cv, exp))
            del K0, V0, ck, cv, exp
    g_logits = logits.cpu().numpy().astype(np.float64)
    g_hidden = hidden.cpu().numpy().astype(np.float64)
    g_next = nxt.cpu().numpy()
    # --- tokens vs the GPU's own logits
    own = [int(np.flatnonzero(g_logits[i] == g_logits[i].max())[0]) for i in range(b)]
    out["tokens_self_ok"] = bool(all(int(g_next[i]) == own[i] for i in range(b)))
    out["finite"] = bool(np.all(np.isfinite(g_logits)) and np.all(np.isfinite(g_hidden)))
    if compare:
        t0 = time.perf_counter()
        ref = oracle.decode_step(sh, case.W, case.kvs, case.tokens[:b], pos, [p + 1 for p in pos])
        out["oracle_s"] = round(time.perf_counter() - t0, 1)
        h0_exact = np.array_equal(g_hidden[0], ref["hidden"][0])
        hid = [[rel_l2(g_hidden[l, i], ref["hidden"][l, i]) for i in range(b)] for l in range(1, L + 1)]
        hid_err = max(max(r) for r in hid)
        log_err = max(rel_l2(g_logits[i], ref["logits"][i]) for i in range(b))
        g_hmid = hmid.cpu().numpy().astype(np.float64)
        hmid_err = max((rel_l2(g_hmid[l, i], ref["h_mid"][l, i]) for l in range(L) for i in range(b)), default=0.0)
        # K/V rows written this step
        k_err = v_err = 0.0
        for l in range(L):
            kg = case.K[l, torch.arange(b), :, torch.tensor(pos), :].float().cpu().numpy()  # [b, nkv, hd]
            vg = case.V[l, torch.arange(b), :, torch.tensor(pos), :].float().cpu().numpy()
            for i in range(b):
                k_err = max(k_err, rel_l2(kg[i], ref["k_new"][l, i]))
                v_err = max(v_err, rel_l2(vg[i], ref["v_new"][l, i]))
        near_ties = 0
        tok_ok = True
        for i in range(b):
            r = ref["logits"][i]
            top2 = np.partition(r, -2)[-2:]
            gap = float(top2[1] - top2[0])
            maxerr = float(np.max(np.abs(g_logits[i] - r)))
            if gap > 2 * maxerr:
                tok_ok = tok_ok and int(g_next[i]) == ref["tokens"][i]
            else:
                near_ties += 1
        # log-probability the decoder assigns to the token it goes on with,
        # against the float64 forward pass (the pages' "mean log-probability
        # error"), per sequence
        lp_err = []
        for i in range(b):
            t = int(g_next[i])
            lg, lr = g_logits[i], ref["logits"][i]
            lp_g = lg[t] - (lg.max() + np.log(np.sum(np.exp(lg - lg.max()))))
            lp_r = lr[t] - (lr.max() + np.log(np.sum(np.exp(lr - lr.max()))))
            lp_err.append(abs(float(lp_g - lp_r)))
        out.update(h0_exact=bool(h0_exact), hidden_err=hid_err, hmid_err=hmid_err, logits_err=log_err, k_err=k_err,
                   v_err=v_err, tokens_oracle_ok=bool(tok_ok), near_ties=near_ties,
                   hidden_err_last_layer=max(hid[-1]), logprob_err=lp_err)
    case.tokens[:b] = [int(t) for t in g_next]
    case.step_idx += 1
    return out


def assert_step_ok(r, tol=TOL):
    assert r["status"] == 0, r
    assert r["finite"], r
    assert r.get("kv_index_ok", True), r
    assert r["tokens_self_ok"], r
    if "hidden_err" in r:
        assert r["h0_exact"], r
        assert r["hmid_err"] <= tol, r
        assert r["hidden_err"] <= tol, r
        assert r["logits_err"] <= tol, r
        assert r["k_err"] <= tol and r["v_err"] <= tol, r
        assert r["tokens_oracle_ok"], r
