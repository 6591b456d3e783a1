#!/usr/bin/env python
"""Decode-step throughput of the Gemma-4-E2B-shaped decoder on one MI355X.

One "step" is one greedy decode step of the whole path (embedding and
per-layer inputs, 35 layers, tied lm_head, argmax) for every sequence of the
batch.  Default workload: E2B shape, bf16 weights (random init N(0, 0.02),
seed 0), batch 1, a 128-token random prompt, then 512 greedy steps (KV length
129..640).  The prompt is prefilled before timing; warm-up steps are run and
then the positions and tokens are reset, so the timed steps cover exactly
positions 128..128+K-1.  Each step is one replay of a HIP graph captured by
the library (one graph launch per step; tokens and positions advance on the
device).

Prints one JSON line on stdout (progress goes to stderr):
  value      tok/s = batch * K / (timed seconds)
  roofline   the kernel kind with the largest share of step time, timed with
             HIP events in an eager pass over the same positions:
             algorithmic bytes per launch / mean launch duration vs 8 TB/s
  step_roofline  algorithmic bytes of the whole step (weights streamed once +
             unique K/V read + K/V write + gathers) / step time vs 8 TB/s
  cpu_baseline   the fp64 oracle on this host's cores, teacher-forced on the
             GPU's tokens, over a bounded sample of the same workload
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "decode tok/s at batch 1 and 64 (E2B shape, bf16 & W4A16); % of HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg, quant, batch, positions):
    """Algorithmic bytes of one decode step at the given positions (per sequence
    the position of its new token).  Weights: every linear, the tied lm_head
    and the norm gains are read once per step; the per-layer table is gathered
    (one row per token).  K/V: unique bytes of the caches read (sharing layers
    read their source's cache, counted once) plus the new token's K/V write."""
    import synth
    L, H, P, V = cfg["num_hidden_layers"], cfg["hidden_size"], cfg["hidden_size_per_layer_input"], cfg["vocab_size"]
    lin = gain = 0
    for s in synth.tensor_specs(cfg, kv_all_layers=False):
        n = 1
        for d in s.shape:
            n *= d
        if s.kind == "linear":
            lin += n // 2 + 2 * (n // 32) if quant == "w4a16" else 2 * n
        elif s.kind in ("gain", "scalar"):
            gain += 2 * n
    weights = lin + 2 * V * H + gain
    first = L - cfg["num_kv_shared_layers"]
    src_layers = [l for l in range(first)]
    kv_read = 0
    for p in positions:
        T = p + 1
        for l in src_layers:
            hd = synth.layer_head_dim(cfg, l)
            t = T if synth.layer_is_full(cfg, l) else min(T, cfg["sliding_window"])
            kv_read += 2 * 2 * hd * t
    kv_write = 2 * 2 * sum(synth.layer_head_dim(cfg, l) for l in src_layers)
    gathers = 2 * H + 2 * L * P
    per_step = weights + (kv_read / len(positions)) * batch + batch * (kv_write + gathers)
    return per_step, weights


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--quant", choices=["bf16", "w4a16"], default="bf16")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=128)
    ap.add_argument("--eager", action="store_true", help="launch kernels per step instead of a graph")
    ap.add_argument("--cpu-steps", type=int, default=24, help="oracle decode steps timed (0: skip)")
    ap.add_argument("--profile-steps", type=int, default=32)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sequences shard across GPUs with no per-step exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    cfg = synth.get_config("e2b")
    B, P, K, W = args.batch, args.prompt, args.steps, args.warmup
    V = cfg["vocab_size"]
    t0 = time.time()
    w = synth.generate(cfg, args.quant, seed=0)
    log(f"weights generated in {time.time() - t0:.1f}s")
    max_ctx = P + max(K, W)
    eng = Engine(cfg, args.quant, w, max_batch=B, max_ctx=max_ctx, max_rows=min(128, max(B, P)))
    dev = eng.device
    log(f"engine loaded ({eng.model.arena_bytes() / 1e9:.3f} GB arena) in {time.time() - t0:.1f}s")
    stream = torch.cuda.Stream(dev)
    prompts = [synth.tokens(P, 1 + b, V) for b in range(B)]
    with torch.cuda.stream(stream):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        for b in range(B):
            eng.prefill(b, torch.from_numpy(prompts[b]).to(dev), 0, tok[b:b + 1])
        eng.check()
        tok0 = tok.clone()
        pos = torch.full((B,), P, dtype=torch.int32, device=dev)
        graph = None if args.eager else eng.capture(tok, pos, tok, advance=True)

        def run(n):
            for _ in range(n):
                if graph is not None:
                    graph.replay()
                else:
                    eng.decode_step(tok, pos, tok)
                    pos.add_(1)

        run(W)
        stream.synchronize()
        pos.fill_(P)
        tok.copy_(tok0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(K)
        e1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        ms = e0.elapsed_time(e1)
    log(f"timed {K} steps: {ms:.2f} ms")
    value = B * K / (ms / 1e3)
    positions = list(range(P, P + K))
    sb, wbytes = step_bytes(cfg, args.quant, B, positions)
    ms_step = ms / K

    # per-kernel timing (eager, events around each launch of one kind)
    kinds = ["gate_up", "down", "lm_head", "qkv", "o"]
    prof = {}
    gpu_tokens = []
    with torch.cuda.stream(stream):
        for i, kind in enumerate(kinds):
            pos.fill_(P)
            tok.copy_(tok0)
            eng.profile_begin(kind)
            for s in range(args.profile_steps):
                eng.decode_step(tok, pos, tok)
                pos.add_(1)
                if i == 0 and s < args.cpu_steps:
                    gpu_tokens.append(tok.cpu().numpy().copy())
            n, tms, tby = eng.profile_read()
            prof[kind] = dict(launches=n, ms=tms / max(n, 1), bytes=tby / max(n, 1),
                              share=tms / (args.profile_steps * ms_step) if n else 0.0)
    dom = max(prof, key=lambda k: prof[k]["ms"] * prof[k]["launches"])
    d = prof[dom]
    achieved = d["bytes"] / (d["ms"] / 1e3)
    log("kernel kinds: " + ", ".join(f"{k}: {v['ms'] * 1e3:.1f} us x{v['launches'] // args.profile_steps}"
                                     f" = {v['bytes'] / (v['ms'] / 1e3) / 1e9:.0f} GB/s"
                                     for k, v in prof.items()))

    cpu = None
    if args.cpu_steps > 0:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        orc = oracle.Oracle(cfg, args.quant, w, 1, max_ctx)
        tpf = time.time()
        orc.prefill(0, prompts[0], logits=False)
        log(f"oracle prefill of {P} tokens: {time.time() - tpf:.1f}s")
        feed = [int(tok0[0].item())] + [int(t[0]) for t in gpu_tokens[:args.cpu_steps - 1]]
        tc = time.time()
        for i, t in enumerate(feed):
            orc.step(0, t, P + i)
        dt = time.time() - tc
        cpu = {"value": round(len(feed) / dt, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
               "sample": f"sequence 0: {len(feed)} teacher-forced decode steps at positions "
                         f"{P}..{P + len(feed) - 1} after an untimed {P}-token prefill, fp64"}
        orc.close()

    wl = (f"E2B shape ({cfg['num_hidden_layers']} layers, hidden {cfg['hidden_size']}, vocab {V}), "
          f"{args.quant} weights, batch {B}, {P}-token random prompt then {K} greedy decode steps "
          f"(KV length {P + 1}..{P + K})")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tok/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.quant, "data": "synthetic",
        "config": {"workload": wl, "quant": args.quant, "batch": B, "prompt": P, "decode_steps": K,
                   "graph": graph is not None},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": None, "bytes_per_launch": int(d["bytes"]),
                     "mean_launch_us": round(d["ms"] * 1e3, 2)},
        "step_roofline": {"bytes_per_step": int(sb), "weight_bytes": int(wbytes),
                          "achieved": round(sb / (ms_step / 1e3) / 1e9, 1), "peak": HBM_PEAK / 1e9,
                          "unit": "GB/s", "frac": round(sb / (ms_step / 1e3) / HBM_PEAK, 4)},
        "kernel_kinds": {k: {"mean_us": round(v["ms"] * 1e3, 2), "per_step": v["launches"] // args.profile_steps,
                             "GBps": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1) if v["ms"] else None}
                         for k, v in prof.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
