"""Paged KV cache through the C ABI (mk_decode_step_paged).

  * On pools whose blocks are a random permutation of a contiguous cache's
    rows (unused blocks hold the NaN sentinel), every step is bit-identical to
    mk_decode_step on the contiguous cache -- logits, tokens, and the written
    rows land in the blocks the table names -- and matches the float64 oracle
    run on the gathered contiguous copy.  Chunks of cached rows cross block
    boundaries (ragged lengths, 64-row blocks).
  * Continuous batching: sequences leave and join between steps by rewriting
    block-table rows; each sequence is checked against its own oracle state.
  * A block-table entry outside the pool is clamped and raises
    MK_STATUS_BAD_BLOCK (every access stays inside the pool).
  * At the benchmark's full sizes (Llama-3-8B b8 -> b9 and Llama-2-13B b16,
    whose contiguous runs are compared with the oracle at every mid-state in
    test_gpu_workloads), pools of 256-position blocks in seeded permuted
    order give steps bit-identical to the contiguous cache, the ninth
    sequence's join included."""
import numpy as np
import pytest
import torch

import oracle
from decode_megakernel_amd.binding import DecodeEngine, STATUS_BAD_BLOCK
from gpu_harness import log, rel_l2, TOL
from mkinputs import (SMALL_QWEN_H128, SMALL_MHA_H128, SMALL_MHA_H64, SMALL_LLAMA_H64, WORKLOADS, make_weights,
                      make_kv_cache, make_paged_kv, bf16_bits, draw_tokens, draw_contexts, kv_capacity, BF16_NAN_SENTINEL)

pytestmark = pytest.mark.gpu


def _sentinel_like(shape):
    return torch.full(shape, BF16_NAN_SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def to_paged(K, bs, extra, gen):
    """Contiguous [L][B][nkv][S][hd] -> pool [L][B*S/bs + extra][nkv][bs][hd] and
    block table [B][S/bs] (a random permutation of the pool's blocks)."""
    L, B, nkv, S, hd = K.shape
    nb = S // bs
    total = B * nb + extra
    perm = torch.randperm(total, generator=gen)[: B * nb].reshape(B, nb)
    pool = _sentinel_like((L, total, nkv, bs, hd))
    for i in range(B):
        for j in range(nb):
            pool[:, int(perm[i, j])] = K[:, i, :, j * bs:(j + 1) * bs]
    return pool, perm.to(torch.int32).cuda().contiguous()


def from_paged(pool, bt, S):
    L, total, nkv, bs, hd = pool.shape
    B, nb = bt.shape
    out = _sentinel_like((L, B, nkv, S, hd))
    btc = bt.cpu()
    for i in range(B):
        for j in range(nb):
            out[:, i, :, j * bs:(j + 1) * bs] = pool[:, int(btc[i, j])]
    return out


def _ints(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("shape,ctx,bs", [(SMALL_QWEN_H128, [5, 300, 64, 127, 1, 191], 64),
                                          (SMALL_MHA_H128, [63, 64, 65, 250, 3], 64),
                                          (SMALL_MHA_H64, [100, 7, 129, 256], 128),
                                          (SMALL_LLAMA_H64, [17, 200, 33, 90, 1, 64, 150, 12, 77], 64)],
                         ids=["qwen-h128-b6", "mha-h128-b5", "mha-h64-b4", "llama-h64-b9"])
def test_paged_matches_contiguous_and_oracle(shape, ctx, bs):
    sh = shape
    b, steps = len(ctx), 3
    S = ((max(ctx) + steps + bs - 1) // bs) * bs
    w = make_weights(sh, 71, device="cuda")
    K, V = make_kv_cache(sh, 71, ctx, b, S, device="cuda")
    gen = torch.Generator().manual_seed(9)
    Kp, bt = to_paged(K, bs, 5, gen)
    gen = torch.Generator().manual_seed(9)
    Vp, bt2 = to_paged(V, bs, 5, gen)
    assert torch.equal(bt, bt2)
    W = oracle.Weights(sh, {k: bf16_bits(v) for k, v in w.items()})
    kvs = oracle.KVState(sh, bf16_bits(K), bf16_bits(V), ctx)
    e_c = DecodeEngine(sh, w, max_batch=b, max_seq=S)
    e_p = DecodeEngine(sh, w, max_batch=b, max_seq=S)
    toks = draw_tokens(71, b, sh.vocab)
    try:
        for s in range(steps):
            pos = [c + s for c in ctx]
            lc = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
            lp = torch.empty_like(lc)
            nc = torch.empty(b, dtype=torch.int32, device="cuda")
            np_ = torch.empty_like(nc)
            e_c.step(_ints(toks), _ints(pos), _ints([p + 1 for p in pos]), K, V, lc, nc)
            e_p.step_paged(_ints(toks), _ints(pos), _ints([p + 1 for p in pos]), Kp, Vp, bt, lp, np_)
            torch.cuda.synchronize()
            assert e_c.status() == 0 and e_p.status() == 0
            same = torch.equal(lc, lp) and torch.equal(nc, np_)
            kv_same = (torch.equal(from_paged(Kp, bt, S).view(torch.int16), K.view(torch.int16)) and
                       torch.equal(from_paged(Vp, bt, S).view(torch.int16), V.view(torch.int16)))
            ref = oracle.decode_step(sh, W, kvs, toks, pos, [p + 1 for p in pos])
            g = lp.cpu().numpy().astype(np.float64)
            err = max(rel_l2(g[i], ref["logits"][i]) for i in range(b))
            log(f"{sh.name} step {s}: paged == contiguous {same}, caches equal {kv_same}, logits rel L2 {err:.2e}")
            assert same and kv_same
            assert err <= TOL
            toks = [int(t) for t in np_.cpu()]
    finally:
        e_c.close()
        e_p.close()


def test_continuous_batching_join_and_leave():
    sh = SMALL_QWEN_H128
    bs = 64
    seqs = {"A": 70, "B": 200, "C": 5, "D": 129}   # prompt lengths
    nb = 5                                          # logical blocks per sequence (320 positions)
    # every sequence's prompt generated as its own contiguous row, then scattered into one shared pool
    w = make_weights(sh, 81, device="cuda")
    names = list(seqs)
    K, V = make_kv_cache(sh, 81, [seqs[n] for n in names], len(names), nb * bs, device="cuda")
    gen = torch.Generator().manual_seed(4)
    Kp, bt_all = to_paged(K, bs, 3, gen)
    gen = torch.Generator().manual_seed(4)
    Vp, _ = to_paged(V, bs, 3, gen)
    W = oracle.Weights(sh, {k: bf16_bits(v) for k, v in w.items()})
    states = {n: oracle.KVState(sh, bf16_bits(K[:, i:i + 1]), bf16_bits(V[:, i:i + 1]), [seqs[n]])
              for i, n in enumerate(names)}
    tok = dict(zip(names, draw_tokens(81, len(names), sh.vocab)))
    length = dict(seqs)
    eng = DecodeEngine(sh, w, max_batch=4, max_seq=nb * bs)
    # (active sequences per step): B leaves after step 1, D joins at step 2
    schedule = [["A", "B", "C"], ["A", "B", "C"], ["A", "C", "D"], ["C", "D", "A"]]
    try:
        for s, active in enumerate(schedule):
            b = len(active)
            rows = torch.stack([bt_all[names.index(n)] for n in active]).contiguous()
            pos = [length[n] for n in active]
            logits = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
            nxt = torch.empty(b, dtype=torch.int32, device="cuda")
            eng.step_paged(_ints([tok[n] for n in active]), _ints(pos), _ints([p + 1 for p in pos]), Kp, Vp, rows,
                           logits, nxt)
            torch.cuda.synchronize()
            assert eng.status() == 0
            g = logits.cpu().numpy().astype(np.float64)
            errs = []
            for j, n in enumerate(active):
                ref = oracle.decode_step(sh, W, states[n], [tok[n]], [length[n]], [length[n] + 1])
                errs.append(rel_l2(g[j], ref["logits"][0]))
                # the new rows of every layer sit in the block the table names
                blk = int(bt_all[names.index(n), length[n] // bs])
                for l in range(sh.n_layers):
                    row = Kp[l, blk, :, length[n] % bs, :].float().cpu().numpy()
                    assert rel_l2(row, ref["k_new"][l, 0]) <= TOL
                length[n] += 1
                tok[n] = int(nxt[j])
            log(f"step {s} active {active}: logits rel L2 {max(errs):.2e}")
            assert max(errs) <= TOL
    finally:
        eng.close()


def test_bad_block_is_clamped_and_reported():
    sh = SMALL_QWEN_H128
    bs, ctx = 64, [70, 10]
    w = make_weights(sh, 91, device="cuda")
    K, V = make_kv_cache(sh, 91, ctx, 2, 2 * bs, device="cuda")
    gen = torch.Generator().manual_seed(2)
    Kp, bt = to_paged(K, bs, 0, gen)
    gen = torch.Generator().manual_seed(2)
    Vp, _ = to_paged(V, bs, 0, gen)
    bad = bt.clone()
    bad[0, 1] = Kp.shape[1] + 7   # outside the pool
    eng = DecodeEngine(sh, w, max_batch=2, max_seq=2 * bs)
    try:
        logits = torch.empty((2, sh.vocab), dtype=torch.float32, device="cuda")
        eng.step_paged(_ints([1, 2]), _ints(ctx), _ints([c + 1 for c in ctx]), Kp, Vp, bad, logits)
        torch.cuda.synchronize()
        st = eng.status()
        log(f"bad block: status {st}")
        assert st & STATUS_BAD_BLOCK
        assert bool(torch.isfinite(logits[1]).all())
    finally:
        eng.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["llama3-8b-b8to9", "llama2-13b-b16"])
def test_paged_full_size_matches_contiguous(key):
    wl = WORKLOADS[key]
    sh = wl.shape
    steps = 2  # per phase
    ctx = draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)
    cap = kv_capacity(max(ctx) + 1, steps * len(wl.phases))
    log(f"case {key} paged 256 vs contiguous, contexts {ctx}, capacity {cap}")
    w = make_weights(sh, wl.seed, device="cuda")
    K, V = make_kv_cache(sh, wl.seed, ctx, wl.batch_cap, cap, device="cuda")
    Kp, Vp, bt = make_paged_kv(sh, wl.seed, ctx, wl.batch_cap, cap, 256, device="cuda", permute=True)
    e_c = DecodeEngine(sh, w, max_batch=wl.batch_cap, max_seq=cap)
    e_p = DecodeEngine(sh, w, max_batch=wl.batch_cap, max_seq=cap)
    toks = draw_tokens(wl.seed, wl.batch_cap, sh.vocab)
    done = [0] * wl.batch_cap
    try:
        for ph in wl.phases:
            b = ph.batch
            for s in range(steps):
                pos = [ctx[i] + done[i] for i in range(b)]
                lc = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
                lp = torch.empty_like(lc)
                nc = torch.empty(b, dtype=torch.int32, device="cuda")
                np_ = torch.empty_like(nc)
                lens = [p + 1 for p in pos]
                e_c.step(_ints(toks[:b]), _ints(pos), _ints(lens), K, V, lc, nc)
                e_p.step_paged(_ints(toks[:b]), _ints(pos), _ints(lens), Kp, Vp, bt, lp, np_)
                torch.cuda.synchronize()
                assert e_c.status() == 0 and e_p.status() == 0
                same = torch.equal(lc, lp) and torch.equal(nc, np_)
                # this step's new rows: where the table puts them, equal to the contiguous cache's
                rows_same = True
                for i in range(b):
                    blk, off = int(bt[i, pos[i] // 256]), pos[i] % 256
                    rows_same = rows_same and torch.equal(Kp[:, blk, :, off].view(torch.int16),
                                                          K[:, i, :, pos[i]].view(torch.int16))
                    rows_same = rows_same and torch.equal(Vp[:, blk, :, off].view(torch.int16),
                                                          V[:, i, :, pos[i]].view(torch.int16))
                log(f"  {key} batch {b} step {s}: logits and tokens identical {same}, new rows identical {rows_same}")
                assert same and rows_same
                for i in range(b):
                    done[i] += 1
                toks[:b] = [int(t) for t in np_.cpu()]
    finally:
        e_c.close()
        e_p.close()
        del K, V, Kp, Vp, w
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
