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
DEFAULT_WORKLOAD = "qwen3-0.6b-b1"


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_api.cpp", "mk_plan.cpp", "mk_internal.h"):
        with open(os.path.join(ROOT, "decode_megakernel_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--phase", type=int, default=-1, help="phase index (default: the last phase)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def setup(wl, phase_idx, steps_total):
    """Weights, KV cache and per-step input buffers on the GPU."""
    import torch
    from mkinputs import make_weights, make_kv_cache, draw_contexts, draw_tokens, kv_capacity
    shape = wl.shape
    phase = wl.phases[phase_idx]
    b = phase.batch
    ctx = draw_contexts(wl.seed, wl.batch_cap, wl.ctx_lo, wl.ctx_hi)
    # earlier phases advance their sequences before this phase starts
    start = [0] * wl.batch_cap
    for p in wl.phases[:phase_idx]:
        for i in range(p.batch):
            start[i] += p.steps
    ctx_now = [ctx[i] + start[i] for i in range(b)]
    seq_cap = kv_capacity(max(ctx_now) + 1, steps_total)
    weights = make_weights(shape, wl.seed, device="cuda")
    K, V = make_kv_cache(shape, wl.seed, ctx_now, wl.batch_cap, seq_cap, device="cuda")
    toks = draw_tokens(wl.seed, b, shape.vocab)
    pos = torch.tensor([[c + s for c in ctx_now] for s in range(steps_total)], dtype=torch.int32, device="cuda")
    lens = pos + 1
    tok = torch.zeros((2, b), dtype=torch.int32, device="cuda")
    tok[0] = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty((b, shape.vocab), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return dict(shape=shape, b=b, ctx=ctx_now, seq_cap=seq_cap, weights=weights, K=K, V=V, pos=pos, lens=lens,
                tok=tok, logits=logits)


def cpu_baseline(wl, S, host_sample_layers=None):
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
    shape = S["shape"]
    b = S["b"]
    L = shape.n_layers
    n_params_layer = (shape.hidden * (shape.q_dim + 2 * shape.kv_dim) + shape.q_dim * shape.hidden +
                      3 * shape.hidden * shape.intermediate)
    nl = L if n_params_layer * L <= 1.2e9 else (host_sample_layers or 2)
    names = [n for n in S["weights"] if ".layers." not in n or int(n.split(".")[2]) < nl]
    bits = {n: bf16_bits(S["weights"][n]) for n in names}
    kbits = bf16_bits(S["K"][:nl])
    vbits = bf16_bits(S["V"][:nl])
    sub = shape.replace(n_layers=nl)
    W = oracle.Weights(sub, bits, keep=False)
    kv = oracle.KVState(sub, kbits, vbits, S["ctx"])
    toks = [int(t) for t in S["tok"][0].cpu()]
    pos = S["ctx"]
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
    from mkinputs import WORKLOADS
    from decode_megakernel_amd.binding import DecodeEngine
    from decode_megakernel_amd.bytes_model import step_bytes, HBM_PEAK_BYTES_PER_S
    wl = WORKLOADS[args.workload]
    phase_idx = args.phase if args.phase >= 0 else len(wl.phases) - 1
    total = args.warmup + args.steps
    S = setup(wl, phase_idx, total)
    shape, b = S["shape"], S["b"]
    eng = DecodeEngine(shape, S["weights"], max_batch=wl.batch_cap, max_seq=S["seq_cap"])
    stream = torch.cuda.current_stream()

    def step(s):
        eng.step(S["tok"][s % 2], S["pos"][s], S["lens"][s], S["K"], S["V"], S["logits"], S["tok"][(s + 1) % 2],
                 stream=stream)

    t_first = time.perf_counter()
    step(0)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t_first) * 1e3
    for s in range(1, args.warmup):
        step(s)
    torch.cuda.synchronize()
    status = eng.status()
    if status:
        raise RuntimeError(f"device status {status:#x} during warmup")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        step(args.warmup + k)
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status = eng.status()
    if status:
        raise RuntimeError(f"device status {status:#x} during the timed steps")
    per = [starts[k].elapsed_time(ends[k]) * 1e-3 for k in range(args.steps)]
    kernel_s = sum(per)
    total_bytes = sum(step_bytes(shape, [c + args.warmup + k + 1 for c in S["ctx"]]) for k in range(args.steps))
    achieved = total_bytes / kernel_s
    tokens_per_s = b * args.steps / wall
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, S)
    per_sorted = sorted(per)
    line = {
        "metric": "decode tokens/sec and MBU (% of 8 TB/s HBM peak) per decode step, 1 MI355X",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init bf16 weights N(0,0.02), N(0,1) prompt KV, uniform first tokens",
        "config": {"workload": wl.key, "shape": shape.name, "batch": b, "context_at_first_timed_step": S["ctx"],
                   "note": wl.note},
        "mbu": round(achieved / HBM_PEAK_BYTES_PER_S, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK_BYTES_PER_S / 1e9,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_BYTES_PER_S, 4),
                     "traffic": traffic_from_profile(wl.key),
                     "algorithmic_bytes_per_step": int(total_bytes / args.steps),
                     "kernel_ms_mean": round(kernel_s / args.steps * 1e3, 4),
                     "kernel_ms_median": round(per_sorted[len(per) // 2] * 1e3, 4),
                     "kernel_ms_min": round(per_sorted[0] * 1e3, 4)},
        "cpu_baseline": cpu,
        "first_step_ms_including_schedule_build": round(first_ms, 2),
        "kernel_sha": kernel_sha(),
    }
    eng.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
