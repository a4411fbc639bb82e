"""Boundary behaviour of the C ABI on the GPU.

  * a wait that exceeds the spin limit raises MK_STATUS_TIMEOUT, and the bit
    stays reported on every later mk_get_status (the kernel's abort flag makes
    later steps give up their waits too) until mk_reset clears it.  The
    timeout is forced from the host: a handle created with
    MK_SPIN_TIMEOUT_MS=0 gives up every wait at its first failed poll, so every
    launch still exits normally;
  * the mid-state dump receives exactly the residual stream mk_copy_hidden
    returns, inside the same launch, and stops when switched off;
  * cooperative and plain launches give bit-identical results;
  * a batch size that changes from step to step (a sequence joining) needs no
    schedule build at step time: the second size's first step is bit-identical
    to the same step on a handle that ran that size before."""
import os

import pytest
import torch

from decode_megakernel_amd.binding import DecodeEngine, STATUS_TIMEOUT
from gpu_harness import log
from mkinputs import TINY_QWEN, SMALL_LLAMA_H64, make_weights, make_kv_cache

pytestmark = pytest.mark.gpu


def _inputs(sh, ctx, seed, seq_cap=64):
    w = make_weights(sh, seed, device="cuda")
    K, V = make_kv_cache(sh, seed, ctx, len(ctx), seq_cap, device="cuda")
    return w, K, V


def _step(eng, sh, K, V, toks, pos, batch=None):
    b = len(toks) if batch is None else batch
    dev = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    logits = torch.full((b, sh.vocab), float("nan"), dtype=torch.float32, device="cuda")
    nxt = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    eng.step(dev(toks[:b]), dev(pos[:b]), dev([p + 1 for p in pos[:b]]), K, V, logits, nxt)
    torch.cuda.synchronize()
    return logits, nxt


def test_forced_timeout_stays_reported_until_reset(monkeypatch):
    sh = TINY_QWEN
    ctx = [5, 9]
    w, K, V = _inputs(sh, ctx, 31)
    monkeypatch.setenv("MK_SPIN_TIMEOUT_MS", "0")
    eng = DecodeEngine(sh, w, max_batch=2, max_seq=64)
    monkeypatch.delenv("MK_SPIN_TIMEOUT_MS")
    try:
        log("forced timeout: step 1")
        _step(eng, sh, K, V, [1, 2], ctx)
        s1 = eng.status()
        log(f"  status {s1}")
        assert s1 & STATUS_TIMEOUT
        # reading the status does not clear a timeout
        assert eng.status() & STATUS_TIMEOUT
        log("forced timeout: step 2")
        _step(eng, sh, K, V, [1, 2], ctx)
        assert eng.status() & STATUS_TIMEOUT
        eng.reset()
        s3 = eng.status()
        log(f"  after reset: status {s3}")
        assert s3 == 0
    finally:
        eng.close()


def test_midstate_dump_matches_copy_hidden():
    sh = SMALL_LLAMA_H64
    ctx = [40, 3, 17]
    w, K, V = _inputs(sh, ctx, 41)
    eng = DecodeEngine(sh, w, max_batch=4, max_seq=64)
    try:
        dump = torch.full((sh.n_layers + 1, 4, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
        eng.set_midstate_dump(dump)
        _step(eng, sh, K, V, [7, 8, 9], ctx)
        assert eng.status() == 0
        hid = torch.empty((sh.n_layers + 1, 3, sh.hidden), dtype=torch.float32, device="cuda")
        eng.copy_hidden(3, hid)
        torch.cuda.synchronize()
        log(f"dump vs copy_hidden: equal={torch.equal(dump[:, :3], hid)}")
        assert torch.equal(dump[:, :3], hid)
        assert bool(torch.isnan(dump[:, 3]).all())  # row 3 took no part
        # switched off: the buffer keeps the last step's values
        eng.set_midstate_dump(None)
        before = dump.clone()
        _step(eng, sh, K, V, [7, 8, 9], [c + 1 for c in ctx])
        assert eng.status() == 0
        assert torch.equal(dump.view(torch.int32), before.view(torch.int32))
    finally:
        eng.close()


def test_cooperative_and_plain_launches_agree(monkeypatch):
    sh = SMALL_LLAMA_H64
    ctx = [40, 3, 17, 60, 9, 1, 33, 20, 5]
    w, K, V = _inputs(sh, ctx, 43, seq_cap=96)
    K0, V0 = K.clone(), V.clone()
    out = []
    for coop in ("1", "0"):
        monkeypatch.setenv("MK_COOP", coop)
        eng = DecodeEngine(sh, w, max_batch=9, max_seq=96)
        monkeypatch.delenv("MK_COOP")
        try:
            K.copy_(K0)
            V.copy_(V0)
            res = []
            for b in (8, 9):   # VALU and MFMA schedules
                lg, nx = _step(eng, sh, K, V, list(range(1, 10)), ctx, batch=b)
                assert eng.status() == 0
                res.append((lg, nx, K.clone(), V.clone()))
            out.append(res)
        finally:
            eng.close()
    for (la, na, ka, va), (lb, nb, kb, vb) in zip(*out):
        assert torch.equal(la, lb) and torch.equal(na, nb)
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16))
    log("cooperative and plain launches bit-identical at batch 8 and 9")


def test_batch_change_needs_no_step_time_build():
    sh = TINY_QWEN
    ctx = [5, 9, 7, 11]
    w, K, V = _inputs(sh, ctx, 47)
    K0, V0 = K.clone(), V.clone()
    toks = [3, 5, 7, 9]
    e1 = DecodeEngine(sh, w, max_batch=4, max_seq=64)
    e2 = DecodeEngine(sh, w, max_batch=4, max_seq=64)
    try:
        # e1: batch 3 first, then batch 4; e2: batch 4 straight away
        _step(e1, sh, K, V, toks, ctx, batch=3)
        K.copy_(K0)
        V.copy_(V0)
        l1, n1 = _step(e1, sh, K, V, toks, ctx, batch=4)
        K.copy_(K0)
        V.copy_(V0)
        l2, n2 = _step(e2, sh, K, V, toks, ctx, batch=4)
        assert e1.status() == 0 and e2.status() == 0
        assert torch.equal(l1, l2) and torch.equal(n1, n2)
    finally:
        e1.close()
        e2.close()
