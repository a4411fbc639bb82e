"""Input validation inside the step kernel, through the C ABI.

Out-of-range step inputs never make the kernel read or write out of bounds:
the kernel clamps them, raises a status bit that mk_get_status reports (and
clears), and otherwise computes as if given the clamped value.  Each case is
forced from the host; every launch runs to completion."""
import numpy as np
import pytest
import torch

from decode_megakernel_amd.binding import DecodeEngine
from gpu_harness import log
from mkinputs import TINY_QWEN, make_weights, make_kv_cache

pytestmark = pytest.mark.gpu

STATUS_BAD_TOKEN, STATUS_BAD_POSITION, STATUS_BAD_SEQLEN = 1, 2, 4


def _setup(ctx, seq_cap=64):
    sh = TINY_QWEN
    w = make_weights(sh, 77, device="cuda")
    K, V = make_kv_cache(sh, 77, ctx, len(ctx), seq_cap, device="cuda")
    eng = DecodeEngine(sh, w, max_batch=len(ctx), max_seq=seq_cap)
    return sh, w, K, V, eng


def _step(eng, sh, K, V, toks, pos, lens):
    b = len(toks)
    logits = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(b, dtype=torch.int32, device="cuda")
    eng.step(torch.tensor(toks, dtype=torch.int32, device="cuda"), torch.tensor(pos, dtype=torch.int32, device="cuda"),
             torch.tensor(lens, dtype=torch.int32, device="cuda"), K, V, logits, nxt)
    torch.cuda.synchronize()
    return logits, nxt, eng.status()


def test_bad_token_is_clamped_and_reported():
    ctx = [5, 9]
    sh, w, K, V, eng = _setup(ctx)
    try:
        K0, V0 = K.clone(), V.clone()
        ref_logits, ref_next, st = _step(eng, sh, K, V, [3, sh.vocab - 1], ctx, [c + 1 for c in ctx])
        log(f"reference status {st}")
        assert st == 0
        K.copy_(K0)
        V.copy_(V0)
        logits, nxt, st = _step(eng, sh, K, V, [3, sh.vocab + 17], ctx, [c + 1 for c in ctx])
        log(f"bad token status {st}")
        assert st == STATUS_BAD_TOKEN
        assert torch.equal(logits, ref_logits) and torch.equal(nxt, ref_next)
        assert eng.status() == 0  # reading the status cleared it
        logits, nxt, st = _step(eng, sh, K, V, [-4, 3], [c + 1 for c in ctx], [c + 2 for c in ctx])
        assert st == STATUS_BAD_TOKEN
    finally:
        eng.close()


def test_bad_position_is_clamped_and_reported():
    ctx = [5, 9]
    seq_cap = 64
    sh, w, K, V, eng = _setup(ctx, seq_cap)
    try:
        logits, nxt, st = _step(eng, sh, K, V, [1, 2], [5, seq_cap + 40], [6, seq_cap + 41])
        log(f"bad position status {st}")
        assert st & STATUS_BAD_POSITION
        assert bool(torch.isfinite(logits[0]).all())
        # the clamped sequence wrote its row at the last slot, nothing past it
        assert K.shape[3] == seq_cap
    finally:
        eng.close()


def test_seq_len_mismatch_is_reported():
    ctx = [5, 9]
    sh, w, K, V, eng = _setup(ctx)
    try:
        K0, V0 = K.clone(), V.clone()
        ref_logits, _, st = _step(eng, sh, K, V, [1, 2], ctx, [c + 1 for c in ctx])
        assert st == 0
        K.copy_(K0)
        V.copy_(V0)
        logits, _, st = _step(eng, sh, K, V, [1, 2], ctx, [ctx[0] + 1, ctx[1] + 3])
        log(f"seq_len mismatch status {st}")
        assert st == STATUS_BAD_SEQLEN
        # the step attends to positions 0..p, whatever seq_len says
        assert torch.equal(logits, ref_logits)
    finally:
        eng.close()
