"""Benchmark of the decode-step megakernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]

A step is one greedy decode step of the whole model (one megakernel launch)
for the workload's batch, with weights, KV cache and step inputs already
resident in HBM.  Steps chain on the device: step s reads the tokens step s-1
wrote and the next position of every sequence, exactly as a decode loop does.
Prints one JSON line.  `value` is decode tokens/s; `mbu` and the roofline
block use the algorithmic byte count B(b, S) of each step (every weight, the
LM head, the gathered embedding rows, and the K/V rows attended) against the
8 TB/s HBM peak.  The float64 oracle is timed on a bounded sample of the same
workload on the host CPU as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
DEFAULT_WORKLOAD = "llama2-13b-b16"
# workloads measured beside the headline: (workload, phases timed)
PER_CONFIG = ["llama3.2-1b-b8", "llama3-8b-b1", "llama3-8b-b8to9"]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_api.cpp", "mk_plan.cpp", "mk_internal.h"):
        with open(os.path.join(ROOT, "decode_megakernel_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--per-config-steps", type=int, default=10)
    ap.add_argument("--no-per-op", action="store_true",
                    help="skip the per-operation baseline beside the per-config workloads")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="run every workload on a paged KV cache of BLOCK-position blocks (blocks of each "
                         "sequence scattered over the pool; no CPU or per-operation baselines)")
    ap.add_argument("--paged-order", choices=("permuted", "sequential"), default="permuted",
                    help="block ids of the paged pools: a seeded permutation, or each sequence's blocks in order")
    ap.add_argument("--cold", action="store_true",
                    help="rewrite a 2 GiB buffer before every timed step (outside its events) so that no "
                         "weight or KV byte is served from the 256 MB memory-side cache or the L2s")
    ap.add_argument("--context-sweep", action="store_true",
                    help="Qwen3-8B-shaped model at batch 1 and 8 over contexts 64-4096, with and without "
                         "context routing (mk_set_context_bound); prints one JSON line and exits")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device copy (for scaling profiler byte counters) and exit")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 1 << 28  # 1 GiB of float32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "launches": 3}))


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Run:
    """A workload's weights, KV cache (every sequence's prompt in place from
    the start) and engine on the GPU; phases run back to back on the same
    engine and cache, so a sequence that joins finds the others mid-run."""

    def __init__(self, wl, steps_per_phase, paged=0, paged_order="permuted"):
        import torch
        from mkinputs import make_weights, make_kv_cache, make_paged_kv, draw_contexts, draw_tokens, kv_capacity
        from decode_megakernel_amd.binding import DecodeEngine
        self.wl, self.shape = wl, wl.shape
        self.ctx = draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)
        total = steps_per_phase * len(wl.phases)
        self.seq_cap = kv_capacity(max(self.ctx) + 1, total)
        self.weights = make_weights(self.shape, wl.seed, device="cuda")
        # paged: the same rows in pools of `paged`-position blocks, each
        # sequence's blocks scattered over the pool by a seeded permutation
        self.paged = paged
        if paged:
            self.K = self.V = None
            self.Kp, self.Vp, self.btab = make_paged_kv(self.shape, wl.seed, self.ctx, wl.batch_cap, self.seq_cap,
                                                        paged, device="cuda", permute=paged_order == "permuted")
        else:
            self.K, self.V = make_kv_cache(self.shape, wl.seed, self.ctx, wl.batch_cap, self.seq_cap,
                                           device="cuda")
        self.first_tok = torch.tensor(draw_tokens(wl.seed, wl.batch_cap, self.shape.vocab), dtype=torch.int32,
                                      device="cuda")
        self.tok = torch.zeros((2, wl.batch_cap), dtype=torch.int32, device="cuda")
        self.tok[0] = self.first_tok
        self.logits = torch.empty((wl.batch_cap, self.shape.vocab), dtype=torch.float32, device="cuda")
        self.done = [0] * wl.batch_cap
        self.s = 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.eng = DecodeEngine(self.shape, self.weights, max_batch=wl.batch_cap, max_seq=self.seq_cap)
        self.create_ms = (time.perf_counter() - t0) * 1e3

    def phase(self, b, warmup, steps, scrub=None):
        """warmup + steps chained decode steps at batch b; per-step kernel time
        from HIP events on the launch stream, wall time of the timed steps.
        `scrub`: a device buffer rewritten before every timed step, outside its
        events, so each step starts with cold caches (the wall time then
        includes the scrubs)."""
        import torch
        from decode_megakernel_amd.bytes_model import step_bytes
        stream = torch.cuda.current_stream()
        # sequences taking their first step feed their own first token
        for i in range(b):
            if self.done[i] == 0:
                self.tok[self.s % 2, i] = self.first_tok[i]
        n = warmup + steps
        pos = torch.tensor([[self.ctx[i] + self.done[i] + k for i in range(b)] for k in range(n)], dtype=torch.int32,
                           device="cuda")
        lens = pos + 1
        s0 = self.s

        def step(k):
            s = s0 + k
            if self.paged:
                self.eng.step_paged(self.tok[s % 2, :b], pos[k], lens[k], self.Kp, self.Vp, self.btab,
                                    self.logits[:b], self.tok[(s + 1) % 2, :b], stream=stream, batch=b)
            else:
                self.eng.step(self.tok[s % 2, :b], pos[k], lens[k], self.K, self.V, self.logits[:b],
                              self.tok[(s + 1) % 2, :b], stream=stream, batch=b)

        for k in range(warmup):
            step(k)
        torch.cuda.synchronize()
        st = self.eng.status()
        if st:
            raise RuntimeError(f"device status {st:#x} during warmup")
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            if scrub is not None:
                scrub.add_(1)
            starts[k].record(stream)
            step(warmup + k)
            ends[k].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = self.eng.status()
        if st:
            raise RuntimeError(f"device status {st:#x} during the timed steps")
        per = [starts[k].elapsed_time(ends[k]) * 1e-3 for k in range(steps)]
        nbytes = [step_bytes(self.shape, [self.ctx[i] + self.done[i] + warmup + k + 1 for i in range(b)])
                  for k in range(steps)]
        ctx_first = [self.ctx[i] + self.done[i] + warmup for i in range(b)]
        for i in range(b):
            self.done[i] += n
        self.s += n
        return {"batch": b, "per_step_s": per, "bytes": nbytes, "wall_s": wall, "steps": steps,
                "context_at_first_timed_step": ctx_first}

    def close(self):
        import torch
        self.eng.close()
        del self.weights, self.K, self.V
        if self.paged:
            del self.Kp, self.Vp, self.btab
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


class PerOpEngine:
    """The same decode step as one library call per operation (PyTorch on
    ROCm: hipBLASLt GEMMs, elementwise, reduction and softmax kernels), on the
    same weights and KV cache -- the per-operation engine the megakernel is
    measured against, never used by the library.  Residual and attention in
    fp32, GEMMs in bf16; every sequence's attention is its own set of calls."""

    def __init__(self, run):
        import torch
        sh = run.shape
        self.run, self.sh = run, sh
        self.w = run.weights
        j = torch.arange(sh.head_dim // 2, dtype=torch.float64)
        self.freq = (sh.rope_theta ** (-2.0 * j / sh.head_dim)).to("cuda")

    def _norm(self, x, w):
        import torch
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.sh.rms_eps) * w.float()

    def _rope(self, x, pos):
        import torch
        ang = pos[:, None].double() * self.freq[None, :]
        c, s = ang.cos().float()[:, None, :], ang.sin().float()[:, None, :]
        h = x.shape[-1] // 2
        a, b = x[..., :h], x[..., h:]
        return torch.cat([a * c - b * s, b * c + a * s], -1)

    def step(self, tokens, positions, host_positions):
        import torch
        import torch.nn.functional as F
        sh, w, run = self.sh, self.w, self.run
        b, hd, nkv, G = tokens.numel(), sh.head_dim, sh.n_kv_heads, sh.group
        pos = positions.long()
        x = w["model.embed_tokens.weight"][tokens.long()].float()
        for l in range(sh.n_layers):
            p = f"model.layers.{l}."
            u = self._norm(x, w[p + "input_layernorm.weight"]).bfloat16()
            q = F.linear(u, w[p + "self_attn.q_proj.weight"]).float().view(b, sh.n_q_heads, hd)
            k = F.linear(u, w[p + "self_attn.k_proj.weight"]).float().view(b, nkv, hd)
            v = F.linear(u, w[p + "self_attn.v_proj.weight"]).float().view(b, nkv, hd)
            if sh.qk_norm:
                q = self._norm(q, w[p + "self_attn.q_norm.weight"])
                k = self._norm(k, w[p + "self_attn.k_norm.weight"])
            q, k = self._rope(q, pos), self._rope(k, pos)
            ar = torch.arange(b, device="cuda")
            run.K[l, ar, :, pos] = k.bfloat16()
            run.V[l, ar, :, pos] = v.bfloat16()
            outs = []
            for i in range(b):
                n = host_positions[i] + 1
                Ki = run.K[l, i, :, :n].float()                     # [nkv, n, hd]
                Vi = run.V[l, i, :, :n].float()
                qi = q[i].view(nkv, G, hd)
                sc = torch.matmul(qi, Ki.transpose(1, 2).contiguous()) / hd ** 0.5
                outs.append(torch.matmul(torch.softmax(sc, -1), Vi).reshape(-1))
            o = torch.stack(outs).bfloat16()
            x = x + F.linear(o, w[p + "self_attn.o_proj.weight"]).float()
            u2 = self._norm(x, w[p + "post_attention_layernorm.weight"]).bfloat16()
            a = F.silu(F.linear(u2, w[p + "mlp.gate_proj.weight"]).float()) * F.linear(u2, w[p + "mlp.up_proj.weight"]).float()
            x = x + F.linear(a.bfloat16(), w[p + "mlp.down_proj.weight"]).float()
        from mkinputs import lm_head_name
        logits = F.linear(self._norm(x, w["model.norm.weight"]).bfloat16(), w[lm_head_name(sh)]).float()
        return torch.argmax(logits, -1).to(torch.int32)


def per_op_baseline(run, b, warmup, steps):
    """Time the per-operation engine on the run's weights and cache (positions
    past the megakernel's, so the same cached rows are attended) and count its
    kernel launches per step."""
    import torch
    from decode_megakernel_amd.bytes_model import step_bytes, HBM_PEAK_BYTES_PER_S
    eng = PerOpEngine(run)
    base = [run.ctx[i] + run.done[i] for i in range(b)]
    tok = run.first_tok[:b].clone()
    seq_cap = run.K.shape[3]
    n = warmup + steps
    if max(base) + n >= seq_cap:
        base = [run.ctx[i] for i in range(b)]
    hpos = [[c + k for c in base] for k in range(n)]
    pos = [torch.tensor(hp, dtype=torch.int32, device="cuda") for hp in hpos]
    for k in range(warmup):
        tok = eng.step(tok, pos[k], hpos[k])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        tok = eng.step(tok, pos[warmup + k], hpos[warmup + k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches = None
    try:
        from torch.profiler import profile, ProfilerActivity
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            eng.step(tok, pos[-1], hpos[-1])
            torch.cuda.synchronize()
        launches = int(sum(e.count for e in prof.key_averages() if e.device_type is not None and
                           str(e.device_type).endswith("CUDA")))
    except Exception:
        launches = None
    nbytes = sum(step_bytes(run.shape, [pp + 1 for pp in hpos[warmup + k]]) for k in range(steps)) / steps
    ms = wall / steps * 1e3
    return {"kind": "one library call per operation (PyTorch-ROCm: hipBLASLt GEMMs, elementwise, softmax)",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(b * steps / wall, 2),
            "mbu": round(nbytes / (wall / steps) / HBM_PEAK_BYTES_PER_S, 4), "kernel_launches_per_step": launches,
            "steps": steps}


def context_sweep(steps=10, warmup=4):
    """The pages' context-length sweep (Qwen3-8B shape, contexts 64-4096):
    kernel ms and MBU per (batch, context), with the step routed to its
    context bucket (mk_set_context_bound) and without."""
    import torch
    from mkinputs import QWEN3_8B, make_weights, make_kv_cache, draw_tokens
    from decode_megakernel_amd.binding import DecodeEngine
    from decode_megakernel_amd.bytes_model import step_bytes, HBM_PEAK_BYTES_PER_S
    sh = QWEN3_8B
    w = make_weights(sh, 2001, device="cuda")
    rows = []
    for b in (1, 8):
        for S in (64, 128, 256, 512, 1024, 2048, 4096):
            ctx = [S] * b
            cap = S + 2 * (warmup + steps) + 1
            K, V = make_kv_cache(sh, 2001, ctx, b, cap, device="cuda")
            rec = {"batch": b, "context": S}
            for routed in (False, True):
                eng = DecodeEngine(sh, w, max_batch=b, max_seq=cap)
                if routed:
                    eng.set_context_bound(S + warmup + steps + 1)
                tok = torch.tensor(draw_tokens(1, b, sh.vocab), dtype=torch.int32, device="cuda")
                logits = torch.empty((b, sh.vocab), dtype=torch.float32, device="cuda")
                times, nbytes = [], []
                for k in range(warmup + steps):
                    pos = torch.tensor([c + k for c in ctx], dtype=torch.int32, device="cuda")
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    eng.step(tok, pos, pos + 1, K, V, logits, tok)
                    e1.record()
                    torch.cuda.synchronize()
                    if k >= warmup:
                        times.append(e0.elapsed_time(e1) * 1e-3)
                        nbytes.append(step_bytes(sh, [c + k + 1 for c in ctx]))
                if eng.status():
                    raise RuntimeError("device status during the context sweep")
                eng.close()
                key = "routed" if routed else "default"
                rec[key + "_ms"] = round(sum(times) / len(times) * 1e3, 4)
                rec[key + "_mbu"] = round(sum(nbytes) / sum(times) / HBM_PEAK_BYTES_PER_S, 4)
            rows.append(rec)
            print("# " + json.dumps(rec), file=sys.stderr, flush=True)
            del K, V
            torch.cuda.empty_cache()
    print(json.dumps({"context_sweep": "qwen3-8b (36 layers, hidden 4096, 32/8 heads, head_dim 128, QK-norm, untied)",
                      "rows": rows}), flush=True)


def summarize(ph):
    from decode_megakernel_amd.bytes_model import HBM_PEAK_BYTES_PER_S
    ks = sum(ph["per_step_s"])
    achieved = sum(ph["bytes"]) / ks
    srt = sorted(ph["per_step_s"])
    return {"batch": ph["batch"], "kernel_ms_mean": round(ks / ph["steps"] * 1e3, 4),
            "kernel_ms_median": round(srt[len(srt) // 2] * 1e3, 4),
            "tokens_per_s": round(ph["batch"] * ph["steps"] / ph["wall_s"], 2),
            "algorithmic_bytes_per_step": int(sum(ph["bytes"]) / ph["steps"]),
            "achieved_GBps": round(achieved / 1e9, 1), "mbu": round(achieved / HBM_PEAK_BYTES_PER_S, 4)}


def cpu_baseline(run, b, ctx, host_sample_layers=None):
    """The float64 oracle, as it stands, timed on the host for a bounded sample
    of the same workload: one full decode step for models up to ~1B
    parameters, otherwise a few layers plus the LM head scaled to all layers."""
    import numpy as np
    import oracle
    from mkinputs import bf16_bits
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    shape = run.shape
    L = shape.n_layers
    n_params_layer = (shape.hidden * (shape.q_dim + 2 * shape.kv_dim) + shape.q_dim * shape.hidden +
                      3 * shape.hidden * shape.intermediate)
    nl = L if n_params_layer * L <= 1.2e9 else (host_sample_layers or 2)
    names = [n for n in run.weights if ".layers." not in n or int(n.split(".")[2]) < nl]
    bits = {n: bf16_bits(run.weights[n]) for n in names}
    # the sample's prompt rows: every position below each sequence's context
    cmax = max(ctx)
    kbits = bf16_bits(run.K[:nl, :b, :, :cmax])
    vbits = bf16_bits(run.V[:nl, :b, :, :cmax])
    sub = shape.replace(n_layers=nl)
    W = oracle.Weights(sub, bits, keep=False)
    kv = oracle.KVState(sub, kbits, vbits, ctx)
    toks = [int(t) for t in run.first_tok[:b].cpu()]
    pos = ctx
    # repeat the sampled step until about 10 s of CPU work (at most 30 s)
    t_layers = t_head = 0.0
    reps = 0
    while reps == 0 or (t_layers + t_head < 10.0 and reps < 200):
        t0 = time.perf_counter()
        x = W.rows("model.embed_tokens.weight", np.asarray(toks))
        for l in range(nl):
            x, *_ = oracle.layer_forward(sub, W, l, x, pos, lambda i, l=l: kv.rows(l, i, pos[i]))
        t1 = time.perf_counter()
        oracle.lm_head(sub, W, x)
        t2 = time.perf_counter()
        t_layers += t1 - t0
        t_head += t2 - t1
        reps += 1
        if t_layers + t_head > 30.0:
            break
    step_s = (t_layers * (L / nl) + t_head) / reps
    sample = (f"{reps} repetitions of one full float64 oracle decode step (batch {b})" if nl == L else
              f"{reps} repetitions of {nl} of {L} layers plus the LM head of one float64 oracle decode step "
              f"(batch {b}), layer time scaled to {L} layers")
    return {"value": b / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "sample": sample,
            "host_cpu": host_cpu_model(), "host_logical_cpus": os.cpu_count(),
            "cores_note": "cores = threads of the BLAS pool the float64 oracle ran on",
            "seconds_measured": round(t_layers + t_head, 3), "repetitions": reps}


def traffic_from_profile(workload):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("kernel_sha") != kernel_sha():
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe()
        return
    if args.context_sweep:
        context_sweep()
        return
    from mkinputs import WORKLOADS
    from decode_megakernel_amd.bytes_model import HBM_PEAK_BYTES_PER_S
    wl = WORKLOADS[args.workload]
    n = args.warmup + args.steps
    # the headline: the workload's last phase after its earlier ones (a batch
    # that grows runs its first phase untimed, warmup only)
    if args.paged:
        args.no_cpu_baseline = args.no_per_op = True
    run = Run(wl, n, args.paged, args.paged_order)
    scrub = torch.zeros(1 << 29, dtype=torch.float32, device="cuda") if args.cold else None
    for p in wl.phases[:-1]:
        run.phase(p.batch, args.warmup, 1)
    ph = run.phase(wl.phases[-1].batch, args.warmup, args.steps, scrub)
    del scrub
    b = ph["batch"]
    head = summarize(ph)
    kernel_s = sum(ph["per_step_s"])
    achieved = sum(ph["bytes"]) / kernel_s
    cpu = None if args.no_cpu_baseline else cpu_baseline(run, b, [run.ctx[i] for i in range(b)])
    create_ms = run.create_ms
    run.close()
    del run
    per_config = {}
    if not args.no_per_config:
        k = args.per_config_steps
        for key in PER_CONFIG:
            if key == wl.key:
                continue
            w2 = WORKLOADS[key]
            r2 = Run(w2, args.warmup + k, args.paged, args.paged_order)
            rec = {"note": w2.note, "phases": []}
            for p in w2.phases:
                rec["phases"].append(summarize(r2.phase(p.batch, args.warmup, k)))
            if len(rec["phases"]) == 2:
                rec["mbu_ratio_last_to_first"] = round(rec["phases"][1]["mbu"] / rec["phases"][0]["mbu"], 4)
            if not args.no_per_op:
                po = per_op_baseline(r2, w2.phases[-1].batch, 2, 3)
                po["megakernel_speedup"] = round(po["ms_per_step"] / rec["phases"][-1]["kernel_ms_mean"], 3)
                rec["per_op_baseline"] = po
            r2.close()
            del r2
            per_config[key] = rec
            print(f"# per-config {key}: " + json.dumps(rec["phases"]), file=sys.stderr, flush=True)
    line = {
        "metric": "decode tokens/sec and MBU (% of 8 TB/s HBM peak) per decode step, 1 MI355X",
        "value": round(b * args.steps / ph["wall_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ph["wall_s"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init bf16 weights N(0,0.02), N(0,1) prompt KV, uniform first tokens",
        "config": {"workload": wl.key, "shape": wl.shape.name, "batch": b,
                   "kv_cache": f"paged, {args.paged}-position blocks, {args.paged_order}" if args.paged else "contiguous",
                   "caches": "cold (2 GiB rewritten before every timed step)" if args.cold else "warm",
                   "context_at_first_timed_step": ph["context_at_first_timed_step"], "note": wl.note},
        "mbu": round(achieved / HBM_PEAK_BYTES_PER_S, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK_BYTES_PER_S / 1e9,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_BYTES_PER_S, 4),
                     "traffic": traffic_from_profile(wl.key),
                     "kernel": "mk_step_kernel",
                     "algorithmic_bytes_per_step": head["algorithmic_bytes_per_step"],
                     "kernel_ms_mean": head["kernel_ms_mean"], "kernel_ms_median": head["kernel_ms_median"],
                     "kernel_ms_min": round(min(ph["per_step_s"]) * 1e3, 4)},
        "cpu_baseline": cpu,
        "per_config": per_config,
        "create_ms_including_all_schedules": round(create_ms, 1),
        "kernel_sha": kernel_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
