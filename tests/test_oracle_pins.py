"""Pins for the float64 oracle, each against something other than the oracle
itself: closed forms, invariants, brute force in plain Python on tiny inputs,
and library routines (torch f64, Hugging Face transformers f64)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od
from mkinputs import (TINY_LLAMA, TINY_QWEN, SMALL_MHA_H128, make_weights, make_kv_cache,
                      bf16_bits, draw_tokens, BF16_NAN_SENTINEL)

RNG = np.random.default_rng(7)


# --------------------------------------------------------------------- bf16
def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x3E4C, 0x8000], dtype=np.uint16)
    got = oracle.bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0
    assert got[2] == 2.0 ** -133                 # smallest bf16 subnormal
    assert got[3] == math.inf
    assert got[4] == 0.19921875                  # 0x3E4C = 1.59375 * 2^-3
    assert got[5] == 0.0 and math.copysign(1, got[5]) < 0
    assert np.isnan(oracle.bf16_to_f64(np.array([BF16_NAN_SENTINEL], np.uint16)))[0]


def test_bf16_widening_matches_torch():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(bits), x.to(torch.float64).numpy())


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    for c in (0.0, 1e-3, 0.7, -3.0, 50.0):
        x = np.full(64, c)
        out = oracle.rms_norm(x, np.ones(64), 1e-5)
        assert np.allclose(out, c / math.sqrt(c * c + 1e-5), rtol=1e-14, atol=0)


def test_rmsnorm_output_rms_closed_form():
    x = RNG.standard_normal(97) * 0.3
    eps = 1e-2
    out = oracle.rms_norm(x, np.ones(97), eps)
    ms = np.mean(x * x)
    assert math.isclose(math.sqrt(np.mean(out * out)), math.sqrt(ms / (ms + eps)), rel_tol=1e-13)


def test_rmsnorm_matches_torch_library():
    x = RNG.standard_normal((5, 33))
    w = RNG.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(oracle.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------- RoPE
@pytest.mark.parametrize("hd", [2, 8, 64, 128])
def test_rope_preserves_norm(hd):
    x = RNG.standard_normal(hd)
    for p in (0, 1, 17, 4095, 8200):
        assert math.isclose(np.linalg.norm(oracle.rope(x, p, 1e4)), np.linalg.norm(x), rel_tol=1e-13)


def test_rope_identity_at_zero_and_composition():
    x = RNG.standard_normal(64)
    assert np.array_equal(oracle.rope(x, 0, 5e5), x)
    a, b = 37, 1200
    assert np.allclose(oracle.rope(oracle.rope(x, a, 5e5), b, 5e5), oracle.rope(x, a + b, 5e5),
                       rtol=1e-10, atol=1e-12)


def test_rope_relative_position_property():
    q, k = RNG.standard_normal(128), RNG.standard_normal(128)
    for m, n in ((5, 3), (1000, 10), (4096, 4000)):
        lhs = np.dot(oracle.rope(q, m, 1e6), oracle.rope(k, n, 1e6))
        rhs = np.dot(oracle.rope(q, m - n, 1e6), k)
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_hd2_is_complex_rotation():
    # hd = 2: a single frequency theta^0 = 1; rotation by angle p.
    x = np.array([0.3, -1.2])
    for p in (1, 2, 7, 100):
        z = complex(x[0], x[1]) * complex(math.cos(p), math.sin(p))
        assert np.allclose(oracle.rope(x, p, 1e4), [z.real, z.imag], rtol=1e-14)


def test_rope_pairs_rotate_half_not_interleaved():
    # a vector with only element 0 set rotates into element hd/2, not element 1
    x = np.zeros(8)
    x[0] = 1.0
    y = oracle.rope(x, 1, 1e4)
    assert y[1] == 0 and y[4] != 0 and math.isclose(y[4], math.sin(1.0))


def test_rope_matches_hf_llama():
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    from transformers import LlamaConfig
    hd, theta = 64, 5e5
    cfg = LlamaConfig(hidden_size=256, num_attention_heads=4, head_dim=hd, rope_theta=theta)
    emb = LlamaRotaryEmbedding(cfg)
    q = torch.randn(1, 4, 1, hd, dtype=torch.float64)
    k = torch.randn(1, 2, 1, hd, dtype=torch.float64)
    for pos in (0, 5, 3000):
        pid = torch.tensor([[pos]])
        cos, sin = emb(q, pid)
        # HF builds its table through float32 inv_freq; compare at that precision
        qr, kr = apply_rotary_pos_emb(q, k, cos.double(), sin.double())
        assert np.allclose(oracle.rope(q[0, :, 0].numpy(), pos, theta), qr[0, :, 0].numpy(),
                           rtol=0, atol=1e-4 * max(1, pos) ** 0.0 * 5)
        assert np.allclose(oracle.rope(k[0, :, 0].numpy(), pos, theta), kr[0, :, 0].numpy(),
                           rtol=0, atol=5e-4)


# ---------------------------------------------------------------- attention
def _brute_attention(q, K, V):
    """Plain-Python loops with math.fsum: softmax(q.K/sqrt(hd)) V for one head."""
    hd = len(q)
    z = [math.fsum(q[t] * K[j][t] for t in range(hd)) / math.sqrt(hd) for j in range(len(K))]
    m = max(z)
    e = [math.exp(v - m) for v in z]
    s = math.fsum(e)
    return [math.fsum(e[j] / s * V[j][t] for j in range(len(K))) for t in range(hd)]


def test_attention_brute_force_tiny():
    for s, hd, H in ((1, 4, 1), (3, 4, 2), (7, 8, 3), (13, 16, 4)):
        q = RNG.standard_normal((H, hd))
        K = RNG.standard_normal((s, hd))
        V = RNG.standard_normal((s, hd))
        got = oracle.attend(q, K, V)
        for h in range(H):
            ref = _brute_attention(q[h].tolist(), K.tolist(), V.tolist())
            assert np.allclose(got[h], ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    V = RNG.standard_normal((1, 16))
    assert np.allclose(oracle.attend(RNG.standard_normal((2, 16)), RNG.standard_normal((1, 16)), V), V)
    K = np.tile(RNG.standard_normal(16), (9, 1))
    V = RNG.standard_normal((9, 16))
    assert np.allclose(oracle.attend(RNG.standard_normal((3, 16)), K, V), V.mean(axis=0), rtol=1e-13)
    z = RNG.standard_normal((4, 50))
    a = oracle.softmax(z)
    assert np.allclose(a.sum(axis=-1), 1.0, rtol=1e-15)
    assert np.allclose(oracle.softmax(z + 123.0), a, rtol=1e-13)   # shift invariance


def test_attention_chunked_logsumexp_merge_equals_full():
    # split-KV decoding computes per-chunk (max, sum, weighted V) and merges;
    # the merge must equal the plain softmax for any chunking.
    q = RNG.standard_normal(32)
    K = RNG.standard_normal((100, 32))
    V = RNG.standard_normal((100, 32))
    full = oracle.attend(q[None], K, V)[0]
    for cuts in ([0, 100], [0, 1, 100], [0, 33, 34, 90, 100]):
        ms, ls, os_ = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            z = K[a:b] @ q / math.sqrt(32)
            m = z.max()
            e = np.exp(z - m)
            ms.append(m); ls.append(e.sum()); os_.append(e @ V[a:b])
        M = max(ms)
        num = sum(math.exp(m - M) * o for m, o in zip(ms, os_))
        den = sum(math.exp(m - M) * l for m, l in zip(ms, ls))
        assert np.allclose(num / den, full, rtol=1e-12)


def test_attention_gqa_matches_torch_sdpa():
    nq, nkv, s, hd = 8, 2, 11, 16
    q = torch.randn(1, nq, 1, hd, dtype=torch.float64)
    K = torch.randn(1, nkv, s, hd, dtype=torch.float64)
    V = torch.randn(1, nkv, s, hd, dtype=torch.float64)
    G = nq // nkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1))
    for h in range(nq):
        got = oracle.attend(q[0, h].numpy(), K[0, h // G].numpy(), V[0, h // G].numpy())
        assert np.allclose(got, ref[0, h].numpy(), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- SwiGLU etc
def test_silu_closed_form_and_library():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(oracle.silu(np.array([40.0]))[0], 40.0, rel_tol=1e-15)
    assert math.isclose(oracle.silu(np.array([1.0]))[0], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    z = RNG.standard_normal(100) * 5
    assert np.allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)


def test_greedy_token_lowest_index_wins_ties():
    assert oracle.greedy_token(np.array([1.0, 3.0, 2.0, 3.0])) == 1
    assert oracle.greedy_token(np.array([-5.0, -5.0])) == 0
    row = RNG.standard_normal(1000)
    assert oracle.greedy_token(row) == int(torch.argmax(torch.from_numpy(row)))


# ------------------------------------------------------------- whole step
def _setup(shape, contexts, seed=11, batch_cap=None, seq_cap=None):
    batch_cap = batch_cap or len(contexts)
    seq_cap = seq_cap or (max(contexts) + 8)
    w = make_weights(shape, seed)
    bits = {k: bf16_bits(v) for k, v in w.items()}
    K, V = make_kv_cache(shape, seed, contexts, batch_cap, seq_cap)
    return bits, bf16_bits(K), bf16_bits(V)


@pytest.mark.parametrize("shape", [TINY_LLAMA, TINY_QWEN, SMALL_MHA_H128.replace(n_layers=1)],
                         ids=lambda s: s.name)
def test_whole_step_matches_hf_transformers(shape):
    ctx = 9
    bits, kb, vb = _setup(shape, [ctx])
    W = oracle.Weights(shape, bits)
    kv = oracle.KVState(shape, kb, vb, [ctx])
    hf = __import__("hf_ref").HFRunner(shape, bits, kb, vb, row=0, context=ctx)
    tok = draw_tokens(3, 1, shape.vocab)[0]
    for step in range(3):
        r = oracle.decode_step(shape, W, kv, [tok], [ctx + step], [ctx + step + 1])
        hid, logits = hf.step(tok, ctx + step)
        for l in range(shape.n_layers + 1):
            err = np.linalg.norm(r["hidden"][l, 0] - hid[l]) / np.linalg.norm(hid[l])
            assert err < 1e-6, (step, l, err)
        err = np.linalg.norm(r["logits"][0] - logits) / np.linalg.norm(logits)
        assert err < 1e-6, (step, err)
        tok = r["tokens"][0]


def test_zero_layer_weights_leave_residual_unchanged():
    shape = TINY_LLAMA
    bits, kb, vb = _setup(shape, [5])
    for name in list(bits):
        if ".layers." in name and name.endswith("proj.weight"):
            bits[name] = np.zeros_like(bits[name])
    W = oracle.Weights(shape, bits)
    kv = oracle.KVState(shape, kb, vb, [5])
    r = oracle.decode_step(shape, W, kv, [17], [5])
    for l in range(1, shape.n_layers + 1):
        assert np.array_equal(r["hidden"][l], r["hidden"][0])


def test_zero_layers_gives_tied_embedding_logits():
    shape = TINY_LLAMA.replace(n_layers=0)
    bits, kb, vb = _setup(TINY_LLAMA, [3])
    bits = {k: v for k, v in bits.items() if ".layers." not in k}
    W = oracle.Weights(shape, bits)
    kv = oracle.KVState(shape, kb[:0], vb[:0], [3])
    t = 42
    r = oracle.decode_step(shape, W, kv, [t], [3])
    E = oracle.bf16_to_f64(bits["model.embed_tokens.weight"])
    x = E[t]
    ref = E @ (x / math.sqrt(np.mean(x * x) + shape.rms_eps))
    assert np.allclose(r["logits"][0], ref, rtol=1e-13)


def test_ragged_batch_equals_independent_runs_and_permutation():
    shape = TINY_QWEN
    ctx = [4, 11, 1, 7]
    bits, kb, vb = _setup(shape, ctx)
    toks = draw_tokens(5, 4, shape.vocab)
    W = oracle.Weights(shape, bits)
    batch = oracle.decode_step(shape, W, oracle.KVState(shape, kb, vb, ctx), toks, ctx)
    for i in range(4):
        single = oracle.decode_step(shape, W, oracle.KVState(shape, kb[:, i:i + 1], vb[:, i:i + 1], [ctx[i]]),
                                    [toks[i]], [ctx[i]])
        assert np.allclose(batch["logits"][i], single["logits"][0], rtol=1e-12, atol=1e-12)
        assert np.allclose(batch["hidden"][:, i], single["hidden"][:, 0], rtol=1e-12, atol=1e-12)
    perm = [2, 0, 3, 1]
    pb = oracle.decode_step(shape, W, oracle.KVState(shape, kb[:, perm], vb[:, perm], [ctx[p] for p in perm]),
                            [toks[p] for p in perm], [ctx[p] for p in perm])
    assert np.allclose(pb["logits"], batch["logits"][perm], rtol=1e-12, atol=1e-12)


def test_oracle_never_reads_past_sequence_length():
    # every slot at or beyond a sequence's context holds NaN: any read past
    # seq_len would poison the outputs.
    shape = TINY_LLAMA
    ctx = [3, 6]
    bits, kb, vb = _setup(shape, ctx, seq_cap=16)
    W = oracle.Weights(shape, bits)
    kv = oracle.KVState(shape, kb, vb, ctx)
    toks = [1, 2]
    for step in range(4):
        r = oracle.decode_step(shape, W, kv, toks, [c + step for c in ctx])
        assert np.all(np.isfinite(r["logits"])) and np.all(np.isfinite(r["hidden"]))
        toks = r["tokens"]


def test_broadcast_position_bug_is_detectable():
    # The pages warn that equal-length prompts hide a kernel that broadcasts one
    # sequence's position across a ragged batch.  Plant that bug in the oracle
    # (use sequence 0's position for everyone) and check ragged outputs change.
    shape = TINY_LLAMA
    ctx = [5, 9]
    bits, kb, vb = _setup(shape, ctx, seq_cap=16)
    W = oracle.Weights(shape, bits)
    good = oracle.decode_step(shape, W, oracle.KVState(shape, kb, vb, ctx), [7, 8], ctx)
    kv = oracle.KVState(shape, kb, vb, ctx)
    bad_logits = []
    for i in range(2):  # emulate: sequence 1 run at sequence 0's position
        x = W.rows("model.embed_tokens.weight", np.array([[7, 8][i]]))
        for l in range(shape.n_layers):
            x, *_ = oracle.layer_forward(shape, W, l, x, [ctx[0]], lambda j, l=l: kv.rows(l, i, ctx[0]))
        bad_logits.append(oracle.lm_head(shape, W, x)[0])
    assert np.allclose(bad_logits[0], good["logits"][0])
    assert not np.allclose(bad_logits[1], good["logits"][1], rtol=1e-3)
