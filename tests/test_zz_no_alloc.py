"""The allocation-free step (mk_decode_step_static) through the C ABI: two
calls in a row, the second with a smaller batch, must give the same logits,
greedy tokens and KV-cache bytes as mk_decode_step on the same inputs (the
same kernel and schedules run on scratch in the library's static array
instead of the handle's workspace).  A handle whose scratch exceeds the
static array is rejected before anything is enqueued."""
import ctypes

import pytest
import torch

from decode_megakernel_amd.binding import DecodeEngine, MKError
from gpu_harness import log
from mkinputs import SMALL_LLAMA_H64, SMALL_MHA_H128, ModelShape, make_weights, make_kv_cache

pytestmark = pytest.mark.gpu


def _run(eng, sh, K, V, calls, static):
    out = []
    for toks, pos in calls:
        b = len(toks)
        dev = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
        logits = torch.full((b, sh.vocab), float("nan"), dtype=torch.float32, device="cuda")
        nxt = torch.full((b,), -1, dtype=torch.int32, device="cuda")
        eng.step(dev(toks), dev(pos), dev([p + 1 for p in pos]), K, V, logits, nxt, static=static)
        torch.cuda.synchronize()
        assert eng.status() == 0
        out.append((logits, nxt, K.clone(), V.clone()))
    return out


@pytest.mark.parametrize("shape,ctx", [(SMALL_LLAMA_H64, [40, 3, 17, 60, 9]),
                                       (SMALL_MHA_H128, [5, 300, 77, 100, 2, 64, 129, 211, 3, 12, 1, 40, 77, 5, 31, 8])],
                         ids=["valu-b5-b3", "mfma-b16-b9"])
def test_static_step_matches_workspace_step(shape, ctx):
    sh = shape
    w = make_weights(sh, 61, device="cuda")
    K, V = make_kv_cache(sh, 61, ctx, len(ctx), 320, device="cuda")
    K0, V0 = K.clone(), V.clone()
    b2 = len(ctx) // 2 + 1
    calls = [(list(range(3, 3 + len(ctx))), ctx), (list(range(7, 7 + b2)), [c + 1 for c in ctx[:b2]])]
    eng = DecodeEngine(sh, w, max_batch=len(ctx), max_seq=320)
    try:
        ref = _run(eng, sh, K, V, calls, static=False)
        K.copy_(K0)
        V.copy_(V0)
        got = _run(eng, sh, K, V, calls, static=True)
        for k, ((lr, nr, kr, vr), (lg, ng, kg, vg)) in enumerate(zip(ref, got)):
            log(f"call {k} (batch {len(calls[k][0])}): logits equal {torch.equal(lr, lg)}, tokens {ng.tolist()}")
            assert torch.equal(lr, lg) and torch.equal(nr, ng)
            assert torch.equal(kr.view(torch.int16), kg.view(torch.int16))
            assert torch.equal(vr.view(torch.int16), vg.view(torch.int16))
    finally:
        eng.close()


def test_static_step_rejects_scratch_beyond_the_array():
    # 64 layers of one aliased layer's weights: the per-layer activations of
    # 16 sequences at hidden 2048 / intermediate 8192 exceed the 64 MiB array
    sh = ModelShape("wide-64-layers", 1, 2048, 16, 4, 128, 8192, 1000, True, False, 1e4, 1e-5)
    w = make_weights(sh, 3, device="cuda")
    deep = sh.replace(n_layers=64)
    wd = {}
    for name, t in w.items():
        if ".layers.0." in name:
            for l in range(64):
                wd[name.replace(".layers.0.", f".layers.{l}.")] = t
        else:
            wd[name] = t
    K, V = make_kv_cache(sh, 3, [4], 16, 16, device="cuda")
    eng = DecodeEngine(deep, wd, max_batch=16, max_seq=16)
    try:
        dev = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
        logits = torch.empty((1, sh.vocab), dtype=torch.float32, device="cuda")
        Kd = K.expand(64, *K.shape[1:])  # never read: the call is rejected before any launch
        with pytest.raises(MKError) as e:
            eng.step(dev([1]), dev([4]), dev([5]), Kd, Kd, logits, static=True)
        log(f"rejected: {e.value}")
        assert e.value.code == -6
    finally:
        eng.close()
