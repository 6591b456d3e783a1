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
  value      tok/s = batch * K / (timed seconds) of the headline workload
  roofline   the kernel kind with the largest share of step time: algorithmic
             bytes per launch / mean launch duration (HIP events around each
             launch of that kind on its stream, eager steps queued behind a
             spin kernel so the host never starves the GPU) vs 8 TB/s;
             traffic = HBM bytes per launch from the committed PMC profile of
             the same kernels (null if the kernel source changed since)
  step_roofline  algorithmic bytes of the whole step (weights streamed once +
             unique K/V read + K/V write + gathers) / step time vs 8 TB/s
  cpu_baseline   the fp64 oracle on this host's cores, teacher-forced on the
             GPU's tokens, over a bounded sample of the same workload
  also       the same measurement for W4A16 and for batch 64 (unless --no-aux)

--long: the long-context workload instead (W4A16, batch 1 or 8 via --batch,
context grown 500 -> 8,000 by 500-token prefill chunks, 64 timed decode
steps at each length, decoded positions rolled back before the next chunk).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "decode tok/s at batch 1 and 64 (E2B shape, bf16 & W4A16); % of HBM roofline"
KINDS = ["gate_up", "down", "lm_head", "qkv", "o"]
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernels_sha():
    h = hashlib.sha1()
    for f in ("kernels.hip", "dev_common.h", "e2b_internal.h"):
        with open(os.path.join(ROOT, "w4a16_weight_streaming_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


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
    kv_read = 0
    for p in positions:
        T = p + 1
        for l in range(first):
            hd = synth.layer_head_dim(cfg, l)
            t = T if synth.layer_is_full(cfg, l) else min(T, cfg["sliding_window"])
            kv_read += 2 * 2 * hd * t
    kv_write = 2 * 2 * sum(synth.layer_head_dim(cfg, l) for l in range(first))
    gathers = 2 * H + 2 * L * P
    per_step = weights + (kv_read / len(positions)) * batch + batch * (kv_write + gathers)
    return per_step, weights


def pmc_traffic(kernel_symbol):
    """HBM bytes per launch of a kernel from the committed PMC profile, or None
    if there is none or the kernel sources changed since it was taken."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernels_sha") != kernels_sha():
        return None
    k = d.get("kernels", {}).get(kernel_symbol)
    if not k:
        return None
    return k["fetch_bytes"] * d["fetch_factor"] + k["write_bytes"] * d["write_factor"]


# kernel symbol (as rocprof names it) of each kind, by quant and batch path
# (one row: o is one K slice per head, the sliding layers' 256 named here)
def kernel_symbol(kind, quant, batch):
    tag = {"qkv": 1, "o": 2, "gate_up": 3, "down": 4, "lm_head": 8}[kind]
    if batch == 1:
        wq = 0 if kind == "lm_head" else int(quant == "w4a16")
        ks = {"o": 256, "down": 2048}.get(kind, 1536)
        if ks == 1536:
            u = (3 if kind == "gate_up" else 2) if wq else 4
        else:
            u = 2 if ks == 2048 else 4
        return f"void e2b::k_gemv<{wq}, {ks}, {u}, {tag}>"
    return None


def spin(torch, ms):
    """Keep the GPU busy for ~ms so the host can queue a whole eager step."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 2.4e6))


def measure(cfg, quant, B, P, K, W, prof_steps, eager=False, cpu_steps=0, label=""):
    import numpy as np
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    V = cfg["vocab_size"]
    t0 = time.time()
    w = synth.generate(cfg, quant, seed=0)
    max_ctx = P + max(K, W, prof_steps)
    eng = Engine(cfg, quant, w, max_batch=B, max_ctx=max_ctx, max_rows=min(128, max(B, P)))
    dev = eng.device
    log(f"[{label}] engine loaded ({eng.model.arena_bytes() / 1e9:.3f} GB arena) in {time.time() - t0:.1f}s")
    stream = torch.cuda.Stream(dev)
    prompts = [synth.tokens(P, 1 + b, V) for b in range(B)]
    with torch.cuda.stream(stream):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        for b in range(B):
            eng.prefill(b, torch.from_numpy(prompts[b]).to(dev), 0, tok[b:b + 1])
        eng.check()
        tok0 = tok.clone()
        pos = torch.full((B,), P, dtype=torch.int32, device=dev)
        graph = None if eager else eng.capture(tok, pos, tok, advance=True)

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
    log(f"[{label}] timed {K} steps: {ms:.2f} ms")
    ms_step = ms / K
    sb, wbytes = step_bytes(cfg, quant, B, list(range(P, P + K)))

    # per-kernel timing: eager steps at the same positions, each queued behind
    # a spin kernel; each launch of one kind records its own start and end.
    prof, gpu_tokens = {}, []
    kinds = KINDS
    with torch.cuda.stream(stream):
        for i, kind in enumerate(kinds if prof_steps else []):
            pos.fill_(P)
            tok.copy_(tok0)
            eng.profile_begin(kind)
            for s in range(prof_steps):
                spin(torch, 10)
                eng.decode_step(tok, pos, tok)
                pos.add_(1)
                if i == 0 and s < cpu_steps:
                    gpu_tokens.append(tok.cpu().numpy().copy())
            n, tms, tby = eng.profile_read()
            prof[kind] = dict(launches=n, ms=tms / max(n, 1), bytes=tby / max(n, 1))
    res = {"value": B * K / (ms / 1e3), "ms_per_step": ms_step, "step_bytes": sb, "weight_bytes": wbytes,
           "kinds": prof, "graph": graph is not None}
    if prof:
        log(f"[{label}] kernel kinds: " + ", ".join(
            f"{k}: {v['ms'] * 1e3:.1f} us x{v['launches'] // prof_steps} = {v['bytes'] / (v['ms'] / 1e3) / 1e9:.0f} GB/s"
            for k, v in prof.items()))

    if cpu_steps > 0:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        orc = oracle.Oracle(cfg, quant, w, 1, max_ctx)
        tpf = time.time()
        orc.prefill(0, prompts[0], logits=False)
        log(f"[{label}] oracle prefill of {P} tokens: {time.time() - tpf:.1f}s")
        feed = [int(tok0[0].item())] + [int(t[0]) for t in gpu_tokens[:cpu_steps - 1]]
        tc = time.time()
        for i, t in enumerate(feed):
            orc.step(0, t, P + i)
        dt = time.time() - tc
        res["cpu_baseline"] = {
            "value": round(len(feed) / dt, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"sequence 0: {len(feed)} teacher-forced decode steps at positions "
                      f"{P}..{P + len(feed) - 1} after an untimed {P}-token prefill, fp64"}
        orc.close()
    del eng, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def roofline_of(res, quant, B):
    prof = res["kinds"]
    dom = max(prof, key=lambda k: prof[k]["ms"] * prof[k]["launches"])
    d = prof[dom]
    achieved = d["bytes"] / (d["ms"] / 1e3)
    sym = kernel_symbol(dom, quant, B)
    traffic = pmc_traffic(sym) if sym else None
    return {"bound": "hbm", "kernel": dom, "symbol": sym, "achieved": round(achieved / 1e9, 1),
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
            "traffic": None if traffic is None else int(traffic),
            "bytes_per_launch": int(d["bytes"]), "mean_launch_us": round(d["ms"] * 1e3, 2)}


def step_roofline(res):
    ms = res["ms_per_step"]
    return {"bytes_per_step": int(res["step_bytes"]), "weight_bytes": int(res["weight_bytes"]),
            "achieved": round(res["step_bytes"] / (ms / 1e3) / 1e9, 1), "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": round(res["step_bytes"] / (ms / 1e3) / HBM_PEAK, 4)}


def long_context(args):
    """Context 500 -> 8,000 in 500-token prefill chunks; 64 timed decode steps
    per length, then the decoded positions are rolled back."""
    import numpy as np
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    cfg = synth.get_config("e2b")
    quant, B, chunk, steps, top = args.quant, args.batch, 500, 64, 8000
    V = cfg["vocab_size"]
    w = synth.generate(cfg, quant, seed=0)
    eng = Engine(cfg, quant, w, max_batch=B, max_ctx=top + steps, max_rows=128)
    dev = eng.device
    stream = torch.cuda.Stream(dev)
    rows = []
    with torch.cuda.stream(stream):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        pos = torch.zeros(B, dtype=torch.int32, device=dev)
        graph = eng.capture(tok, pos, tok, advance=True)
        for c in range(top // chunk):
            L0 = c * chunk
            for b in range(B):
                t = synth.tokens(chunk, 1 + b, V, stream=f"chunk{c}")
                eng.prefill(b, torch.from_numpy(t).to(dev), L0, tok[b:b + 1])
            eng.check()
            L = L0 + chunk
            tok_ctx = tok.clone()
            for _ in range(2):  # warm-up replays, then roll back
                pos.fill_(L)
                tok.copy_(tok_ctx)
                graph.replay()
            pos.fill_(L)
            tok.copy_(tok_ctx)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            eng.check()
            ms = e0.elapsed_time(e1) / steps
            sb, _ = step_bytes(cfg, quant, B, list(range(L, L + steps)))
            rows.append({"context": L, "tok_s": round(B / (ms / 1e3), 2), "ms_per_step": round(ms, 4),
                         "step_bytes": int(sb), "frac": round(sb / (ms / 1e3) / HBM_PEAK, 4)})
            log(f"context {L}: {rows[-1]['tok_s']} tok/s, {ms:.3f} ms/step")
            tok.copy_(tok_ctx)
    mean = sum(r["tok_s"] for r in rows) / len(rows)
    ms_mean = sum(r["ms_per_step"] for r in rows) / len(rows)
    out = {"metric": METRIC, "value": round(mean, 2), "unit": "tok/s", "n_gpus": 1,
           "steps": steps * len(rows), "warmup": 2 * len(rows), "ms_per_step": round(ms_mean, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": quant,
           "data": "synthetic",
           "config": {"workload": f"E2B shape, {quant} weights, long-context decode: batch {B}, context "
                                  f"grown 500 -> 8,000 by 500-token random prefill chunks, {steps} greedy "
                                  f"decode steps timed at each length (mean over lengths)",
                      "quant": quant, "batch": B},
           "per_length": rows}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--quant", choices=["bf16", "w4a16"], default=None,
                    help="weights (default bf16; w4a16 with --long)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=128)
    ap.add_argument("--eager", action="store_true", help="launch kernels per step instead of a graph")
    ap.add_argument("--cpu-steps", type=int, default=24, help="oracle decode steps timed (0: skip)")
    ap.add_argument("--profile-steps", type=int, default=32)
    ap.add_argument("--no-aux", action="store_true", help="skip the W4A16 / batch-64 measurements")
    ap.add_argument("--long", action="store_true", help="long-context workload (see above)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device copy (reference kernel for PMC byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sequences shard across GPUs with no per-step exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written by one elementwise kernel")
        del src, dst
    if args.quant is None:
        args.quant = "w4a16" if args.long else "bf16"
    if args.long:
        long_context(args)
        return

    cfg = synth.get_config("e2b")
    B, P, K, W = args.batch, args.prompt, args.steps, args.warmup
    head = measure(cfg, args.quant, B, P, K, W, args.profile_steps, args.eager, args.cpu_steps,
                   f"{args.quant} B={B}")
    also = []
    if not args.no_aux:
        for q, b in (("w4a16", 1), ("bf16", 64), ("w4a16", 64)):
            if (q, b) == (args.quant, B):
                continue
            r = measure(cfg, q, b, P, K, W, 8, False, 0, f"{q} B={b}")
            also.append({"quant": q, "batch": b, "tok_s": round(r["value"], 2),
                         "ms_per_step": round(r["ms_per_step"], 4), "step_roofline": step_roofline(r),
                         "roofline": roofline_of(r, q, b)})
    wl = (f"E2B shape ({cfg['num_hidden_layers']} layers, hidden {cfg['hidden_size']}, vocab "
          f"{cfg['vocab_size']}), {args.quant} weights, batch {B}, {P}-token random prompt then {K} greedy "
          f"decode steps (KV length {P + 1}..{P + K})")
    out = {
        "metric": METRIC, "value": round(head["value"], 2), "unit": "tok/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(head["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.quant, "data": "synthetic",
        "config": {"workload": wl, "quant": args.quant, "batch": B, "prompt": P, "decode_steps": K,
                   "graph": head["graph"]},
        "roofline": roofline_of(head, args.quant, B) if head["kinds"] else None,
        "step_roofline": step_roofline(head),
        "kernel_kinds": {k: {"mean_us": round(v["ms"] * 1e3, 2), "per_step": v["launches"] // max(args.profile_steps, 1),
                             "GBps": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1) if v["ms"] else None}
                         for k, v in head["kinds"].items()},
        "cpu_baseline": head.get("cpu_baseline"),
        "also": also,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
