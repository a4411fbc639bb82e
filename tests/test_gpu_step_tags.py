"""Step tags of the hand-off buffers, through the C ABI.

Activations handed between compute units carry a per-sequence step tag in
their lowest mantissa bit, flipped by the host each step a sequence takes
part in; consumers poll until the tag matches and use the value with the bit
cleared.  These cases check that results do not depend on the tag history:
a sequence that sat out some steps (its rows hold words of an older step), a
batch that shrinks and grows again, and mk_reset (which clears the buffers
and the host-side tags) all give bit-identical logits and tokens for the same
inputs."""
import pytest
import torch

from decode_megakernel_amd.binding import DecodeEngine
from gpu_harness import log
from mkinputs import TINY_QWEN, make_weights, make_kv_cache

pytestmark = pytest.mark.gpu


def _step(eng, sh, K, V, toks, pos):
    b = len(toks)
    logits = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(b, dtype=torch.int32, device="cuda")
    dev = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    eng.step(dev(toks), dev(pos), dev([p + 1 for p in pos]), K, V, logits, nxt)
    torch.cuda.synchronize()
    assert eng.status() == 0
    return logits, nxt


def test_results_do_not_depend_on_tag_history():
    sh = TINY_QWEN
    ctx = [5, 9, 7]
    w = make_weights(sh, 91, device="cuda")
    K, V = make_kv_cache(sh, 91, ctx, len(ctx), 64, device="cuda")
    K0, V0 = K.clone(), V.clone()
    toks = [3, 11, 17]
    eng = DecodeEngine(sh, w, max_batch=len(ctx), max_seq=64)
    try:
        ref_logits, ref_next = _step(eng, sh, K, V, toks, ctx)
        # the batch shrinks for two steps (sequence 0 alone, with its own
        # schedule), then grows back: rows 1 and 2 hold words of an older step
        for _ in range(2):
            K.copy_(K0)
            V.copy_(V0)
            _, n1 = _step(eng, sh, K, V, toks[:1], ctx[:1])
            log(f"batch 1 step: token {int(n1[0])}")
        K.copy_(K0)
        V.copy_(V0)
        logits, nxt = _step(eng, sh, K, V, toks, ctx)
        assert torch.equal(logits, ref_logits) and torch.equal(nxt, ref_next)
        # mk_reset clears the tagged buffers and the host tags
        eng.reset()
        K.copy_(K0)
        V.copy_(V0)
        logits, nxt = _step(eng, sh, K, V, toks, ctx)
        log(f"after reset: tokens {nxt.tolist()} reference {ref_next.tolist()}")
        assert torch.equal(logits, ref_logits) and torch.equal(nxt, ref_next)
    finally:
        eng.close()
