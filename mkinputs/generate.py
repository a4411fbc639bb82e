"""Seeded synthetic inputs: random-init bf16 weights, a prefilled KV cache,
prompt contexts and first tokens.

This module draws random numbers and lays them out; it holds none of the
decode-step arithmetic.  The float64 oracle and the GPU path both consume the
*bits* it produces (the oracle after copying them to the host).

Recipe (one independent torch.Generator per named tensor, seeded from the
workload seed and the CRC32 of the tensor's name, so any tensor can be
regenerated alone):
  * linear and embedding weights: N(0, 1) drawn in float32, times 0.02
    (float32, round-to-nearest-even), then rounded to bf16 (RNE);
  * RMSNorm weights (layer norms, final norm, per-head QK norms): exactly 1.0;
  * prompt KV: N(0, 1) in float32 rounded to bf16 at every position below a
    sequence's context; every other slot holds the bf16 NaN sentinel 0x7FC0,
    so a read past a sequence's length poisons its outputs;
  * contexts: integers uniform in [lo, hi], both ends inclusive;
  * first tokens: integers uniform in [0, vocab).

Bit patterns differ between the CPU and GPU generators of torch; a test
generates on one device and hands the same tensors to both sides.
"""
from __future__ import annotations

import zlib

import torch

from .configs import ModelShape

BF16_NAN_SENTINEL = 0x7FC0
WEIGHT_STD = 0.02


def _generator(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def weight_specs(shape: ModelShape):
    """(name, tensor shape, kind) for every weight tensor, Hugging Face names.

    kind is "linear" (random) or "norm" (ones).  Linear weights are stored
    [out, in] row-major as torch.nn.Linear does.
    """
    d, hd, I, V = shape.hidden, shape.head_dim, shape.intermediate, shape.vocab
    out = [("model.embed_tokens.weight", (V, d), "linear")]
    for l in range(shape.n_layers):
        p = f"model.layers.{l}."
        out += [
            (p + "input_layernorm.weight", (d,), "norm"),
            (p + "self_attn.q_proj.weight", (shape.q_dim, d), "linear"),
            (p + "self_attn.k_proj.weight", (shape.kv_dim, d), "linear"),
            (p + "self_attn.v_proj.weight", (shape.kv_dim, d), "linear"),
            (p + "self_attn.o_proj.weight", (d, shape.q_dim), "linear"),
        ]
        if shape.qk_norm:
            out += [(p + "self_attn.q_norm.weight", (hd,), "norm"),
                    (p + "self_attn.k_norm.weight", (hd,), "norm")]
        out += [
            (p + "post_attention_layernorm.weight", (d,), "norm"),
            (p + "mlp.gate_proj.weight", (I, d), "linear"),
            (p + "mlp.up_proj.weight", (I, d), "linear"),
            (p + "mlp.down_proj.weight", (d, I), "linear"),
        ]
    out.append(("model.norm.weight", (d,), "norm"))
    if not shape.tied_embeddings:
        out.append(("lm_head.weight", (V, d), "linear"))
    return out


def make_tensor(seed: int, name: str, shp, kind: str, device="cpu") -> torch.Tensor:
    if kind == "norm":
        return torch.ones(shp, dtype=torch.bfloat16, device=device)
    g = _generator(seed, name, device)
    x = torch.randn(shp, generator=g, dtype=torch.float32, device=device)
    x.mul_(WEIGHT_STD)
    return x.to(torch.bfloat16)


def make_weights(shape: ModelShape, seed: int, device="cpu", names=None) -> dict:
    """All weights (or only `names`) as bf16 tensors on `device`."""
    out = {}
    for name, shp, kind in weight_specs(shape):
        if names is not None and name not in names:
            continue
        out[name] = make_tensor(seed, name, shp, kind, device)
    return out


def lm_head_name(shape: ModelShape) -> str:
    return "model.embed_tokens.weight" if shape.tied_embeddings else "lm_head.weight"


def draw_contexts(seed: int, n: int, lo: int, hi: int, tag: str = "ctx") -> list:
    g = _generator(seed, tag, "cpu")
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g)]


def draw_tokens(seed: int, n: int, vocab: int, tag: str = "tok0") -> list:
    g = _generator(seed, tag, "cpu")
    return [int(v) for v in torch.randint(0, vocab, (n,), generator=g)]


def kv_capacity(max_context: int, steps: int, align: int = 256) -> int:
    need = max_context + steps
    return ((need + align - 1) // align) * align


def make_kv_layer(shape: ModelShape, seed: int, contexts, batch_cap: int, seq_cap: int, layer: int,
                  device="cpu"):
    """Layer `layer` of the K and V caches: bf16 [batch_cap][n_kv][seq_cap][head_dim].

    The same bits make_kv_cache stores for that layer (one generator per
    layer and tensor), so any layer can be regenerated alone: positions <
    contexts[i] of row i are N(0,1) in bf16, every other slot the NaN
    sentinel."""
    nkv, hd = shape.n_kv_heads, shape.head_dim
    pos = torch.arange(seq_cap, device=device)
    ctx = torch.zeros(batch_cap, dtype=torch.long, device=device)
    ctx[: len(contexts)] = torch.tensor(list(contexts), dtype=torch.long, device=device)
    valid = (pos[None, :] < ctx[:, None])[:, None, :, None]  # [B,1,S,1]
    nan = torch.tensor(BF16_NAN_SENTINEL, dtype=torch.int16, device=device).view(torch.bfloat16)
    out = []
    for tag in ("k", "v"):
        g = _generator(seed, f"kv.{layer}.{tag}", device)
        x = torch.randn((batch_cap, nkv, seq_cap, hd), generator=g,
                        dtype=torch.float32, device=device).to(torch.bfloat16)
        out.append(torch.where(valid, x, nan))
        del x
    return out[0], out[1]


def make_kv_cache(shape: ModelShape, seed: int, contexts, batch_cap: int, seq_cap: int,
                  device="cpu"):
    """K and V caches, bf16, layout [L][batch_cap][n_kv][seq_cap][head_dim].

    Row i holds sequence i.  Positions < contexts[i] are N(0,1) in bf16 (taken
    as keys that are already rotated); all other slots hold the NaN sentinel.
    Rows i >= len(contexts) are all sentinel.
    """
    L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    K = torch.empty((L, batch_cap, nkv, seq_cap, hd), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    for l in range(L):
        K[l], V[l] = make_kv_layer(shape, seed, contexts, batch_cap, seq_cap, l, device)
    return K, V


def make_paged_kv(shape: ModelShape, seed: int, contexts, batch_cap: int, seq_cap: int, block: int,
                  device="cpu", permute: bool = True):
    """The rows of make_kv_cache in paged pools: K, V bf16
    [L][n_blocks][n_kv][block][head_dim] with n_blocks = batch_cap * seq_cap /
    block, and the int32 block table [batch_cap][seq_cap / block] (entry j of
    row i: the pool block holding positions j*block .. of sequence i).  Block
    ids are a seeded permutation (a sequence's blocks scattered over the
    pool), or in order when `permute` is false."""
    if seq_cap % block:
        raise ValueError(f"block {block} must divide the capacity {seq_cap}")
    L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    nb = seq_cap // block
    n_blocks = batch_cap * nb
    g = _generator(seed, "kv.block_table", "cpu")
    perm = torch.randperm(n_blocks, generator=g) if permute else torch.arange(n_blocks)
    table = perm.view(batch_cap, nb).to(torch.int32).to(device)
    dst = perm.to(device)
    Kp = torch.empty((L, n_blocks, nkv, block, hd), dtype=torch.bfloat16, device=device)
    Vp = torch.empty_like(Kp)
    for l in range(L):
        k, v = make_kv_layer(shape, seed, contexts, batch_cap, seq_cap, l, device)
        for src, pool in ((k, Kp), (v, Vp)):
            blocks = src.view(batch_cap, nkv, nb, block, hd).permute(0, 2, 1, 3, 4).reshape(n_blocks, nkv, block, hd)
            pool[l].index_copy_(0, dst, blocks)
        del k, v
    return Kp, Vp, table


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bits (copies off the device)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
