"""Hugging Face transformers as an independent library pin for the oracle.

Builds a float64 LlamaForCausalLM / Qwen3ForCausalLM holding exactly the bf16
weights the oracle sees, prefills its cache with the same prompt K/V rows and
steps it with the same tokens and positions.  Used only by CPU tests.
"""
from __future__ import annotations

import numpy as np
import torch


def _bits_to_f64_torch(bits: np.ndarray) -> torch.Tensor:
    # torch's own bf16 -> f64 widening (independent of the oracle's helper)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64)


def build_model(shape, weight_bits: dict):
    from transformers import LlamaConfig, LlamaForCausalLM, Qwen3Config, Qwen3ForCausalLM
    common = dict(vocab_size=shape.vocab, hidden_size=shape.hidden,
                  intermediate_size=shape.intermediate, num_hidden_layers=shape.n_layers,
                  num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
                  head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
                  rope_theta=shape.rope_theta, tie_word_embeddings=shape.tied_embeddings,
                  attention_bias=False, max_position_embeddings=1 << 16)
    if shape.qk_norm:
        cfg = Qwen3Config(**common)
        cls = Qwen3ForCausalLM
    else:
        cfg = LlamaConfig(mlp_bias=False, **common)
        cls = LlamaForCausalLM
    cfg._attn_implementation = "eager"
    model = cls(cfg).to(torch.float64).eval()
    sd = {}
    for name, bits in weight_bits.items():
        sd[name] = _bits_to_f64_torch(bits)
    if shape.tied_embeddings:
        sd["lm_head.weight"] = sd["model.embed_tokens.weight"]
    missing, unexpected = model.load_state_dict(sd, strict=False)
    missing = [m for m in missing if "rotary" not in m]
    assert not missing and not unexpected, (missing, unexpected)
    return model, cfg


class HFRunner:
    """One sequence (batch 1) stepped through the HF model."""

    def __init__(self, shape, weight_bits, k_bits, v_bits, row: int, context: int):
        from transformers import DynamicCache
        self.model, self.cfg = build_model(shape, weight_bits)
        self.cache = DynamicCache(config=self.cfg)
        for l in range(shape.n_layers):
            k = _bits_to_f64_torch(k_bits[l, row, :, :context, :])[None]
            v = _bits_to_f64_torch(v_bits[l, row, :, :context, :])[None]
            self.cache.update(k, v, l)
        self.shape = shape

    @torch.no_grad()
    def step(self, token: int, position: int):
        outs = []
        hooks = [layer.register_forward_hook(
            lambda m, i, o: outs.append((o[0] if isinstance(o, tuple) else o)[0, -1].clone()))
            for layer in self.model.model.layers]
        try:
            res = self.model(input_ids=torch.tensor([[token]]),
                             position_ids=torch.tensor([[position]]),
                             past_key_values=self.cache, use_cache=True)
        finally:
            for h in hooks:
                h.remove()
        emb = self.model.model.embed_tokens.weight[token]
        hidden = torch.stack([emb] + outs).numpy()
        return hidden, res.logits[0, -1].numpy()
