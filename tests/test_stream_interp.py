"""Schedule fuzzing on the CPU: the per-CU instruction streams the library
builds, run by tests/stream_interp.py in random interleavings (each task phase
waiting on the data it polls on the device), must complete, write every output
once, consume every partial once, and give bit-identical results whatever the
order.  Their float64 results also match the oracle to rounding order (the
interpreter is a test of the schedule, not a reference for the GPU)."""
import numpy as np
import pytest

import oracle
from mkinputs import (TINY_LLAMA, TINY_QWEN, SMALL_MHA_H128, SMALL_WIDE_FFN, SMALL_LLAMA_H64, make_weights,
                      make_kv_cache, bf16_bits, draw_tokens)
from stream_interp import Interp

CASES = [
    (TINY_LLAMA, [5], 7, {}),
    (TINY_QWEN, [3, 40, 1, 77], 13, {}),
    (SMALL_MHA_H128, [64, 129, 1, 500, 33], 16, {}),
    (SMALL_LLAMA_H64, [17, 200, 33, 90, 1, 64, 150, 12, 77], 24, {}),
    (SMALL_WIDE_FFN, [9, 120, 31], 16, {"MK_KSPLIT_MIN_WINDOWS": "2"}),
    (SMALL_WIDE_FFN, [9, 120, 31, 4, 60, 2, 70, 11, 5], 32, {"MK_KSPLIT_MIN_WINDOWS": "2"}),
    (SMALL_LLAMA_H64, [300, 2, 45], 40, {"MK_GEMV_MODE": "2"}),
    # fewer CUs than K pieces (down projection: 3 pieces on 2 CUs): units dealt evenly
    (SMALL_WIDE_FFN, [9, 120, 31, 4, 60, 2, 70, 11, 5], 2, {"MK_KSPLIT_MIN_WINDOWS": "2"}),
    # K-split units dealt evenly over the CUs instead of piece by piece
    (SMALL_WIDE_FFN, [9, 120, 31, 4, 60, 2, 70, 11, 5], 13, {"MK_KSPLIT_MIN_WINDOWS": "2", "MK_KSPLIT_ALIGNED": "0"}),
]


@pytest.mark.parametrize("shape,ctx,n_cu,env", CASES,
                         ids=[f"{c[0].name}-b{len(c[1])}-cu{c[2]}{'-' + '-'.join(c[3]) if c[3] else ''}" for c in CASES])
def test_random_interleavings(monkeypatch, shape, ctx, n_cu, env):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    sh = shape
    seq_cap = max(ctx) + 2
    w = make_weights(sh, 5150, device="cpu")
    K, V = make_kv_cache(sh, 5150, ctx, len(ctx), seq_cap, device="cpu")
    bits = {k: bf16_bits(v) for k, v in w.items()}
    Wo = oracle.Weights(sh, bits)
    kb, vb = bf16_bits(K), bf16_bits(V)
    toks = draw_tokens(5150, len(ctx), sh.vocab)
    ref = oracle.decode_step(sh, Wo, oracle.KVState(sh, kb, vb, ctx), toks, ctx)
    Kf, Vf = oracle.bf16_to_f64(kb), oracle.bf16_to_f64(vb)
    results = []
    for seed in range(3):
        it = Interp(sh, oracle.Weights(sh, bits), Kf, Vf, toks, ctx, n_cu)
        results.append(it.run(np.random.default_rng(seed)))
        assert it.tokens_out == ref["tokens"] or np.isclose(
            np.sort(ref["logits"], -1)[:, -1], np.sort(ref["logits"], -1)[:, -2]).any()
    for other in results[1:]:
        for k in results[0]:
            assert np.array_equal(results[0][k], other[k]), f"{k} depends on the interleaving"
    buf = results[0]
    err = lambda g, r: np.linalg.norm(g - r) / np.linalg.norm(r)
    assert err(buf["hres"], ref["hidden"]) < 1e-12
    assert err(buf["hmid"], ref["h_mid"]) < 1e-12
    assert err(buf["logits"], ref["logits"]) < 1e-12
    assert err(buf["knew"], ref["k_new"]) < 1e-12 and err(buf["vnew"], ref["v_new"]) < 1e-12


def _wide_case(monkeypatch):
    monkeypatch.setenv("MK_KSPLIT_MIN_WINDOWS", "2")
    sh, ctx = SMALL_WIDE_FFN, [9, 120, 31]
    w = make_weights(sh, 5150, device="cpu")
    K, V = make_kv_cache(sh, 5150, ctx, len(ctx), max(ctx) + 2, device="cpu")
    bits = {k: bf16_bits(v) for k, v in w.items()}
    it = Interp(sh, oracle.Weights(sh, bits), oracle.bf16_to_f64(bf16_bits(K)), oracle.bf16_to_f64(bf16_bits(V)),
                draw_tokens(5150, len(ctx), sh.vocab), ctx, 16)
    return it


def test_dropped_task_is_a_deadlock(monkeypatch):
    # a K-split piece removed from one CU's stream: its finisher can never run
    it = _wide_case(monkeypatch)
    c = next(c for c in range(it.n_cu) if any(t["flags"] & 2 for t in it.streams[c]))
    k = next(k for k, t in enumerate(it.streams[c]) if t["flags"] & 2)
    del it.streams[c][k]
    it.prog = [it._program(cc) for cc in range(it.n_cu)]
    with pytest.raises(AssertionError):
        it.run(np.random.default_rng(0))


def test_missing_wait_is_caught(monkeypatch):
    # finish tasks that no longer wait for their pieces read a partial slot
    # before it is written in some interleaving
    it = _wide_case(monkeypatch)
    for c in range(it.n_cu):
        ph = 0
        for t in it.streams[c]:
            if t["type"] == 4:
                it.prog[c][ph] = (lambda: True, it.prog[c][ph][1])
            two = t["type"] == 3 or (t["type"] == 2 and t["nks"] > 1 and not t["flags"] & 2 and t["ks"] == 0)
            ph += 2 if two else 1
    with pytest.raises(AssertionError, match="read before written"):
        it.run(np.random.default_rng(0))
