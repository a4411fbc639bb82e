"""Float64 CPU oracle for one auto-regressive decode step.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the graft entry
point and the CPU-baseline leg of the benchmark may import or run anything in
this package.  It shares no code with the GPU path; both only consume the same
seeded input bits (bf16 weights, bf16 prompt KV, int32 tokens/positions).

What it computes is the plain definition of the decode step as the
ForgeMegakernel paper summary describes it ("2.1 The decode step"): per layer
an RMSNorm, the Q/K/V projections, RoPE, attention of the new token over every
cached position of its own sequence, the output projection, a second RMSNorm
and a SwiGLU MLP, each sublayer added to the residual stream; then a final
RMSNorm and the LM head.  Everything is float64 ("4.2 The mid-state test
oracle": mid-states are checked against float64 references); bf16 inputs are
widened exactly.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * RoPE uses the rotate-half pairing (element j with j + hd/2) and
    frequencies theta^(-2j/hd), no frequency scaling;
  * Qwen3-style QK-norm is an RMSNorm over each head's hd values, applied to q
    and k before RoPE; the cache holds k after norm and RoPE and v raw;
  * attention scale 1/sqrt(hd), no bias, softcap, window or sinks; query head
    h reads KV head h // (n_q / n_kv);
  * the token at position p is written to cache slot p and attends to slots
    0..p, so seq_len = p + 1;
  * greedy decoding picks the lowest index among equal maxima.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# element-wise building blocks
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * j / head_dim)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of vectors x[..., hd] at integer position pos."""
    hd = x.shape[-1]
    half = hd // 2
    ang = pos * rope_frequencies(hd, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Softmax attention of query heads q[H, hd] over rows K[s, hd], V[s, hd]."""
    hd = q.shape[-1]
    z = (q @ K.T) / math.sqrt(hd)
    return softmax(z) @ V


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def greedy_token(logits_row: np.ndarray) -> int:
    """Index of the largest logit; the lowest index wins a tie."""
    m = np.max(logits_row)
    return int(np.flatnonzero(logits_row == m)[0])


# ---------------------------------------------------------------------------
# weights and KV state
# ---------------------------------------------------------------------------

class Weights:
    """bf16 weight bits by Hugging Face name, widened to float64 on use.

    `keep` caches the widened arrays (fine for small models); otherwise every
    use widens again, which bounds memory for large ones.
    """

    def __init__(self, shape, bits: dict, keep: bool = True):
        self.shape = shape
        self.bits = bits
        self.keep = keep
        self._f64 = {}
        self.bytes_read = 0   # bf16 bytes of every weight the oracle reads

    def get(self, name: str) -> np.ndarray:
        arr = self._f64.get(name)
        if arr is None:
            arr = bf16_to_f64(self.bits[name])
            if self.keep:
                self._f64[name] = arr
        return arr

    def read(self, name: str) -> np.ndarray:
        arr = self.get(name)
        self.bytes_read += 2 * arr.size
        return arr

    def rows(self, name: str, idx) -> np.ndarray:
        """Gather rows of a matrix (the embedding lookup)."""
        sub = bf16_to_f64(self.bits[name][np.asarray(idx)])
        self.bytes_read += 2 * sub.size
        return sub

    def lm_head_name(self) -> str:
        return "model.embed_tokens.weight" if self.shape.tied_embeddings else "lm_head.weight"


class KVState:
    """The oracle's view of the KV cache.

    Prompt rows come from the bf16 cache bits, layout
    [L][batch_cap][n_kv][seq_cap][hd]; rows the oracle appends itself are kept
    in float64, per (layer, sequence row), so the oracle never reads back
    anything the GPU wrote.
    """

    def __init__(self, shape, k_bits, v_bits, contexts):
        self.shape = shape
        self.k_bits = k_bits
        self.v_bits = v_bits
        self.ctx = list(contexts)
        L = shape.n_layers
        self.app_k = [[[] for _ in range(len(self.ctx))] for _ in range(L)]
        self.app_v = [[[] for _ in range(len(self.ctx))] for _ in range(L)]
        self.n_app = [0] * len(self.ctx)
        self.stats = {"kv_bytes": 0}

    def add_sequence(self, context: int):
        self.ctx.append(context)
        self.n_app.append(0)
        for l in range(self.shape.n_layers):
            self.app_k[l].append([])
            self.app_v[l].append([])

    def length(self, i: int) -> int:
        return self.ctx[i] + self.n_app[i]

    def rows(self, l: int, i: int, upto: int):
        """K, V rows [0, upto) of sequence i at layer l: arrays [n_kv, upto, hd]."""
        c = min(self.ctx[i], upto)
        Kp = bf16_to_f64(self.k_bits[l, i, :, :c, :])
        Vp = bf16_to_f64(self.v_bits[l, i, :, :c, :])
        n_app = upto - c
        if n_app > 0:
            Ka = np.stack(self.app_k[l][i][:n_app], axis=1)
            Va = np.stack(self.app_v[l][i][:n_app], axis=1)
            Kp = np.concatenate([Kp, Ka], axis=1)
            Vp = np.concatenate([Vp, Va], axis=1)
        return Kp, Vp

    def append(self, l: int, i: int, k: np.ndarray, v: np.ndarray):
        self.app_k[l][i].append(k)
        self.app_v[l][i].append(v)


# ---------------------------------------------------------------------------
# the decode step
# ---------------------------------------------------------------------------

def layer_forward(shape, W: Weights, l: int, x: np.ndarray, positions, kv_rows, stats=None):
    """One decoder layer for a batch.

    x: residual stream [b, d] float64.  positions[i] is sequence i's decode
    position p_i; it attends to its own cached rows 0..p_i-1 (from
    kv_rows(i) -> (K[n_kv, p_i, hd], V[...])) plus the row it writes now.
    Returns the new residual, the mid-layer residual (after attention), and
    the K/V rows written (after QK-norm and RoPE for k).  If given,
    stats["kv_bytes"] grows by the bf16 size of every K and V row attended.
    """
    b, d = x.shape
    hd, nq, nkv, G = shape.head_dim, shape.n_q_heads, shape.n_kv_heads, shape.group
    eps = shape.rms_eps
    p = f"model.layers.{l}."
    u = rms_norm(x, W.read(p + "input_layernorm.weight"), eps)
    q = u @ W.read(p + "self_attn.q_proj.weight").T        # nn.Linear: y = W x
    k = u @ W.read(p + "self_attn.k_proj.weight").T
    v = u @ W.read(p + "self_attn.v_proj.weight").T
    q = q.reshape(b, nq, hd)
    k = k.reshape(b, nkv, hd)
    v = v.reshape(b, nkv, hd)
    if shape.qk_norm:
        q = rms_norm(q, W.read(p + "self_attn.q_norm.weight"), eps)
        k = rms_norm(k, W.read(p + "self_attn.k_norm.weight"), eps)
    o = np.empty((b, nq, hd))
    k_rot = np.empty_like(k)
    for i in range(b):
        pi = int(positions[i])
        qi = rope(q[i], pi, shape.rope_theta)
        k_rot[i] = rope(k[i], pi, shape.rope_theta)
        Kc, Vc = kv_rows(i)
        for g in range(nkv):
            Kg = np.concatenate([Kc[g, :pi], k_rot[i, g][None]], axis=0)
            Vg = np.concatenate([Vc[g, :pi], v[i, g][None]], axis=0)
            if stats is not None:
                stats["kv_bytes"] = stats.get("kv_bytes", 0) + 2 * (Kg.size + Vg.size)
            o[i, g * G:(g + 1) * G] = attend(qi[g * G:(g + 1) * G], Kg, Vg)
    h_mid = x + o.reshape(b, nq * hd) @ W.read(p + "self_attn.o_proj.weight").T
    u2 = rms_norm(h_mid, W.read(p + "post_attention_layernorm.weight"), eps)
    gate = u2 @ W.read(p + "mlp.gate_proj.weight").T
    up = u2 @ W.read(p + "mlp.up_proj.weight").T
    h_out = h_mid + (silu(gate) * up) @ W.read(p + "mlp.down_proj.weight").T
    return h_out, h_mid, k_rot, v


def lm_head(shape, W: Weights, h: np.ndarray) -> np.ndarray:
    u = rms_norm(h, W.read("model.norm.weight"), shape.rms_eps)
    return u @ W.read(W.lm_head_name()).T


def decode_step(shape, W: Weights, kv: KVState, tokens, positions, seq_lens=None) -> dict:
    """One greedy decode step for the batch of sequences 0..b-1.

    Sequence i feeds token tokens[i] at position positions[i] and, after the
    step, has seq_lens[i] = positions[i] + 1 attended rows.  The K/V rows the
    step produces are appended to `kv` (float64).  Returns every mid-state:
    hidden[l] for l = 0..L (the residual stream entering layer l; hidden[L]
    leaves the last layer), h_mid[l], k_new[l], v_new[l], logits and tokens.
    """
    b = len(tokens)
    positions = [int(p) for p in positions]
    if seq_lens is not None:
        for p, s in zip(positions, seq_lens):
            if int(s) != p + 1:
                raise ValueError("seq_len must equal position + 1")
    for i in range(b):
        if kv.length(i) != positions[i]:
            raise ValueError(f"sequence {i}: cache holds {kv.length(i)} rows, position {positions[i]}")
    x = W.rows("model.embed_tokens.weight", np.asarray(tokens, dtype=np.int64))
    hidden = [x]
    h_mids, k_new, v_new = [], [], []
    for l in range(shape.n_layers):
        x, hm, kr, vr = layer_forward(
            shape, W, l, x, positions,
            lambda i, l=l: kv.rows(l, i, positions[i]), stats=kv.stats)
        for i in range(b):
            kv.append(l, i, kr[i], vr[i])
        hidden.append(x)
        h_mids.append(hm)
        k_new.append(kr)
        v_new.append(vr)
    for i in range(b):
        kv.n_app[i] += 1
    logits = lm_head(shape, W, x)
    toks = [greedy_token(logits[i]) for i in range(b)]
    hd, nkv = shape.head_dim, shape.n_kv_heads

    def stack(xs, tail):
        return np.stack(xs) if xs else np.zeros((0,) + tail)
    return {"hidden": np.stack(hidden), "h_mid": stack(h_mids, (b, shape.hidden)),
            "k_new": stack(k_new, (b, nkv, hd)), "v_new": stack(v_new, (b, nkv, hd)),
            "logits": logits, "tokens": toks}
