#!/usr/bin/env python
"""Decode-step throughput of the Gemma-4-E2B-shaped decoder on one MI355X.

One "step" is one greedy decode step of the whole path (embedding and
per-layer inputs, 35 layers, tied lm_head, argmax) for every sequence of the
batch.  Default workload: E2B shape, bf16 weights (random init N(0, 0.02),
seed 0), batch 1, a 128-token random prompt, then K greedy steps (KV length
129..128+K).  The prompt is prefilled before timing; warm-up steps are run and
then the positions and tokens are reset, so every timed loop covers exactly
positions 128..128+K-1.  Each step is one replay of a HIP graph captured by the
library (one graph launch per step; tokens and positions advance on the
device).  The loop of K steps is timed --repeats times (HIP events on the
stream, synchronised on both sides); value is the median.

Prints one JSON line on stdout (progress goes to stderr):
  value      tok/s = batch * K / (median timed seconds) of the headline workload
  repeats    every repeat's loop time, median and interquartile range
  roofline   the dominant kernel (the kind with the largest share of step
             time): algorithmic bytes per launch / mean launch duration (the
             dispatch's own timestamps, eager steps queued behind a spin
             kernel) vs 8 TB/s, and vs the calibrated streaming read;
             traffic = HBM bytes per launch from the committed PMC profile of
             the same kernels (null if the kernel sources changed since)
  step_roofline  algorithmic bytes of the whole step (weights streamed once +
             unique K/V read + K/V write + gathers) / step time, vs 8 TB/s and
             vs the calibrated streaming read
  calibration    a plain streaming reduction over 4 GiB: the read bandwidth
             this device sustains (best of 5)
  kernel_kinds   per-launch time and achieved GB/s of every profiled kind
             (attention: unique and logical K/V bytes)
  prefill    the 128-token prompt through e2b_prefill (one 128-row pass,
             through the first greedy token): ms, = time to first token on
             the device (median of 5 at batch 1; each sequence once at 64)
  cpu_baseline   the fp64 oracle on this host's cores (and on one core),
             teacher-forced on the GPU's tokens, over a bounded sample
  also       W4A16 B=1 (bf16 and int4 vocabulary tables), bf16 and W4A16
             B=64, serving uneven requests (continuous vs lockstep
             batching), and the long-context workload (W4A16, bf16 and int8
             caches, B=1 and 8, contexts 500 / 4,000 / 8,000, with each
             500-token chunk's prefill and the prefill of the whole context so
             far) unless --no-aux (--no-long: without serving and long context)

--long: the long-context workload alone (W4A16, batch 1 or 8 via --batch,
context grown 500 -> 8,000 by 500-token prefill chunks, 64 timed decode
steps at each length, decoded positions rolled back before the next chunk).
"""
import argparse
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "decode tok/s at batch 1 and 64 (E2B shape, bf16 & W4A16); % of HBM roofline"
KINDS = ["gate_up", "down", "lm_head", "qkv", "o", "attn"]
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
TAGS = {"qkv": 1, "o": 2, "gate_up": 3, "down": 4, "lm_head": 8}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg, quant, batch, positions, embed_quant="bf16", kv_quant="bf16"):
    """Algorithmic bytes of one decode step at the given positions (per sequence
    the position of its new token).  Weights: every linear, the tied lm_head
    and the norm gains are read once per step; the per-layer table is gathered
    (one row per token).  K/V: unique bytes of the caches read (sharing layers
    read their source's cache, counted once) plus the new token's K/V write.
    embed_quant "w4a16": the vocabulary tables (lm_head, gathers) are int4
    codes plus a bf16 scale per 32."""
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
    def table(n):   # bytes of n vocabulary-table values
        return n // 2 + 2 * (n // 32) if embed_quant == "w4a16" else 2 * n
    weights = lin + table(V * H) + gain
    kv_read = sum(kv_bytes(cfg, p, True, kv_quant) for p in positions) / len(positions)
    first = L - cfg["num_kv_shared_layers"]
    kv_write = 2 * sum(row_bytes(synth.layer_head_dim(cfg, l), kv_quant) for l in range(first))
    gathers = table(H) + table(L * P)
    per_step = weights + kv_read * batch + batch * (kv_write + gathers)
    return per_step, weights


def row_bytes(hd, kv_quant):
    """Bytes of one cached K or V row: bf16, or int8 codes plus an fp32 scale."""
    return hd + 4 if kv_quant == "int8" else 2 * hd


def kv_bytes(cfg, pos, unique, kv_quant="bf16"):
    """K/V bytes one sequence's attention reads at position pos: every layer
    that owns K/V (unique) or every layer (logical: sharing layers re-read
    their source's cache)."""
    import synth
    L = cfg["num_hidden_layers"]
    first = L - cfg["num_kv_shared_layers"]
    T, tot = pos + 1, 0
    for l in range(first if unique else L):
        hd = synth.layer_head_dim(cfg, l)
        t = T if synth.layer_is_full(cfg, l) else min(T, cfg["sliding_window"])
        tot += 2 * row_bytes(hd, kv_quant) * t
    return tot


def pmc_traffic(pattern):
    """HBM bytes per launch (dispatch-weighted mean over the kernels whose
    symbol matches `pattern`) from the committed PMC profile, or None if there
    is none or the kernel sources changed since it was taken."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    from w4a16_weight_streaming_amd.pmc import kernels_sha
    if d.get("kernels_sha") != kernels_sha():
        return None
    rx = re.compile(pattern)
    hits = [k for name, k in d.get("kernels", {}).items() if rx.fullmatch(name)]
    n = sum(k["dispatches"] for k in hits)
    if not n:
        return None
    return sum((k["fetch_bytes"] * d["fetch_factor"] + k["write_bytes"] * d["write_factor"]) * k["dispatches"]
               for k in hits) / n


def kernel_pattern(kind, quant, batch, embed_quant="bf16"):
    """Regular expression of the kernel symbols (as rocprof names them) that
    run this kind at this batch: the one-row matvec, or the matrix-core
    product with its m-tiles per block."""
    if kind not in TAGS:
        return None
    tag = TAGS[kind]
    wq = int((embed_quant if kind == "lm_head" else quant) == "w4a16")
    if batch == 1:
        return rf"void e2b::k_gemv<{wq}, \d+, \d+, {tag}>"
    mt = 1 if batch <= 16 else (2 if batch <= 32 else 4)
    if kind == "gate_up" or (kind in ("qkv", "o") and not wq):  # (at most 2 m-tiles, W4A16 1)
        mt = min(mt, 1 if wq else 2)
    if wq and kind in ("qkv", "o", "down"):
        mt = 1
    return rf"void e2b::k_gemm<{wq}, \d+, {mt}, \d+, {tag}, \d+>"


def spin(torch, ms):
    """Keep the GPU busy for ~ms so the host can queue a whole eager step."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 2.4e6))


def calibrate(torch):
    """Best of 5 streaming reductions over 4 GiB (the read bandwidth a plain
    stream sustains on this device), bytes/s."""
    from w4a16_weight_streaming_amd import binding
    L = binding.load_library()
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(L.e2b_stream_reduce_blocks(), dtype=torch.float32, device="cuda:0")
    binding.stream_reduce(buf, out)
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.stream_reduce(buf, out)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, buf.numel() * 4 / (e0.elapsed_time(e1) / 1e3))
    total = float(out.double().sum())
    assert abs(total - buf.numel()) < 1e-3 * buf.numel(), total   # the read covered every word
    del buf, out
    torch.cuda.empty_cache()
    log(f"calibration: streaming reduction over 4 GiB at {best / 1e9:.0f} GB/s")
    return best


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def quantiles(xs):
    q = statistics.quantiles(xs, n=4) if len(xs) >= 2 else [xs[0]] * 3
    return q[0], statistics.median(xs), q[2]


def measure(cfg, quant, B, P, K, W, prof_steps, repeats, eager=False, cpu_steps=0, label="",
            embed_quant="bf16"):
    import numpy as np
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    V = cfg["vocab_size"]
    t0 = time.time()
    w = synth.generate(cfg, quant, seed=0, embed_quant=embed_quant)
    max_ctx = P + max(K, W, prof_steps) + 8
    eng = Engine(cfg, quant, w, max_batch=B, max_ctx=max_ctx, max_rows=min(128, max(B, P)))
    dev = eng.device
    log(f"[{label}] engine loaded ({eng.model.arena_bytes() / 1e9:.3f} GB arena) in {time.time() - t0:.1f}s")
    stream = torch.cuda.Stream(dev)
    prompts = [synth.tokens(P, 1 + b, V) for b in range(B)]
    with torch.cuda.stream(stream):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        pdev = [torch.from_numpy(p).to(dev) for p in prompts]
        eng.prefill(0, pdev[0], 0, tok[0:1])       # untimed first pass
        stream.synchronize()
        # prefill = time to first token on the device: the prompt's passes
        # through the first greedy token (a lone sequence is prefilled 5 times
        # over the same positions; each of B sequences once)
        pre_ms = []
        for b in ([0] * 5 if B == 1 else range(B)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            eng.prefill(b, pdev[b], 0, tok[b:b + 1])
            e1.record(stream)
            e1.synchronize()
            pre_ms.append(e0.elapsed_time(e1))
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
        loops = []
        for _ in range(repeats):
            pos.fill_(P)
            tok.copy_(tok0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(K)
            e1.record(stream)
            torch.cuda.synchronize()
            loops.append(e0.elapsed_time(e1))
        eng.check()
    q1, ms, q3 = quantiles(loops)
    log(f"[{label}] {repeats} x {K} steps: median {ms:.2f} ms (IQR {q1:.2f}-{q3:.2f}); "
        f"prefill {statistics.median(pre_ms):.2f} ms")
    ms_step = ms / K
    sb, wbytes = step_bytes(cfg, quant, B, list(range(P, P + K)), embed_quant)

    # per-kernel timing: eager steps at the same positions, each queued behind
    # a spin kernel; each launch of one kind records its own start and end
    prof, gpu_tokens = {}, []
    with torch.cuda.stream(stream):
        for i, kind in enumerate(KINDS if prof_steps else []):
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
            d = dict(launches=n, ms=tms / max(n, 1), bytes=tby / max(n, 1))
            if kind == "attn":   # K/V bytes from the positions the steps covered
                per = [B * kv_bytes(cfg, P + s, u) for s in range(prof_steps) for u in (True, False)]
                d["bytes"] = sum(per[0::2]) / max(n, 1)          # unique, per launch
                d["logical_bytes"] = sum(per[1::2]) / max(n, 1)
            prof[kind] = d
    res = {"value": B * K / (ms / 1e3), "ms_per_step": ms_step, "step_bytes": sb, "weight_bytes": wbytes,
           "kinds": prof, "graph": graph is not None,
           "repeats": {"n": repeats, "loop_ms": [round(x, 3) for x in loops], "median_ms": round(ms, 3),
                       "iqr_ms": [round(q1, 3), round(q3, 3)]},
           "prefill": {"tokens": P, "rows_per_pass": min(128, P), "ms_median": round(statistics.median(pre_ms), 3),
                       "ms_iqr": [round(x, 3) for x in quantiles(pre_ms)[::2]],
                       "ms_min": round(min(pre_ms), 3), "timings": len(pre_ms), "sequences": B,
                       "ttft_ms": round(statistics.median(pre_ms), 3),
                       "ttft": "device time from the first prefill kernel to the first greedy token, "
                               "prompt resident in HBM"}}
    if prof:
        log(f"[{label}] kernel kinds: " + ", ".join(
            f"{k}: {v['ms'] * 1e3:.1f} us x{v['launches'] // prof_steps} = {v['bytes'] / (v['ms'] / 1e3) / 1e9:.0f} GB/s"
            for k, v in prof.items()))

    if cpu_steps > 0:
        import oracle
        threads = oracle.get_threads()
        orc = oracle.Oracle(cfg, quant, w, 1, max_ctx)
        tpf = time.time()
        orc.prefill(0, prompts[0], logits=False)
        log(f"[{label}] oracle prefill of {P} tokens: {time.time() - tpf:.1f}s")
        feed = [int(tok0[0].item())] + [int(t[0]) for t in gpu_tokens[:cpu_steps - 1]]
        tc = time.time()
        for i, t in enumerate(feed):
            orc.step(0, t, P + i)
        dt = time.time() - tc
        # one core: a few further steps on the same cache
        one = min(4, len(feed))
        oracle.set_threads(1)
        t1 = time.time()
        for i in range(one):
            orc.step(0, feed[i], P + len(feed) + i)
        dt1 = time.time() - t1
        oracle.set_threads(threads)
        log(f"[{label}] oracle: {len(feed) / dt:.2f} tok/s on {threads} threads, {one / dt1:.3f} on 1")
        res["cpu_baseline"] = {
            "value": round(len(feed) / dt, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "precision": "fp64",
            "value_1_core": round(one / dt1, 4),
            "sample": f"sequence 0: {len(feed)} teacher-forced decode steps at positions "
                      f"{P}..{P + len(feed) - 1} after an untimed {P}-token prefill, fp64, on {threads} "
                      f"threads; then {one} steps at positions {P + len(feed)}.. on 1 thread"}
        orc.close()
    del eng, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def roofline_of(res, quant, B, calib, embed_quant="bf16"):
    prof = {k: v for k, v in res["kinds"].items()}
    dom = max(prof, key=lambda k: prof[k]["ms"] * prof[k]["launches"])
    d = prof[dom]
    achieved = d["bytes"] / (d["ms"] / 1e3)
    pat = kernel_pattern(dom, quant, B, embed_quant)
    traffic = pmc_traffic(pat) if pat else None
    return {"scope": "dominant kernel", "bound": "hbm", "kernel": dom, "symbols": pat,
            "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK, 4),
            "frac_calibrated": round(achieved / calib, 4) if calib else None,
            "traffic": None if traffic is None else int(traffic),
            "bytes_per_launch": int(d["bytes"]), "mean_launch_us": round(d["ms"] * 1e3, 2)}


def step_roofline(res, calib):
    ms = res["ms_per_step"]
    a = res["step_bytes"] / (ms / 1e3)
    return {"bytes_per_step": int(res["step_bytes"]), "weight_bytes": int(res["weight_bytes"]),
            "achieved": round(a / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(a / HBM_PEAK, 4), "frac_calibrated": round(a / calib, 4) if calib else None}


def kinds_summary(res, steps):
    out = {}
    for k, v in res["kinds"].items():
        e = {"mean_us": round(v["ms"] * 1e3, 2), "per_step": v["launches"] // max(steps, 1),
             "GBps": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1) if v["ms"] else None}
        if "logical_bytes" in v and v["ms"]:
            e["GBps_logical"] = round(v["logical_bytes"] / (v["ms"] / 1e3) / 1e9, 1)
        out[k] = e
    return out


def long_context(quant, B, lengths=None, steps=64, chunk=500, top=8000, kv_quant="bf16"):
    """Context 500 -> 8,000 in 500-token prefill chunks; `steps` timed decode
    steps at each measured length, then the decoded positions are rolled back.
    Returns per-length rows (tok/s, step fraction, prefill ms of the chunk)."""
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    cfg = synth.get_config("e2b")
    V = cfg["vocab_size"]
    w = synth.generate(cfg, quant, seed=0)
    eng = Engine(cfg, quant, w, max_batch=B, max_ctx=top + steps, max_rows=128, kv_quant=kv_quant)
    dev = eng.device
    stream = torch.cuda.Stream(dev)
    rows = []
    cum_ms = 0.0  # prefill of the context so far, per sequence (time to first token of that prompt)
    with torch.cuda.stream(stream):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        pos = torch.zeros(B, dtype=torch.int32, device=dev)
        graph = eng.capture(tok, pos, tok, advance=True)
        for c in range(top // chunk):
            L0 = c * chunk
            L = L0 + chunk
            chunks = [torch.from_numpy(synth.tokens(chunk, 1 + b, V, stream=f"chunk{c}")).to(dev)
                      for b in range(B)]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for b in range(B):
                eng.prefill(b, chunks[b], L0, tok[b:b + 1])
            e1.record(stream)
            eng.check()
            pre_ms = e0.elapsed_time(e1) / B
            cum_ms += pre_ms
            if lengths is not None and L not in lengths:
                continue
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
            sb, _ = step_bytes(cfg, quant, B, list(range(L, L + steps)), kv_quant=kv_quant)
            rows.append({"context": L, "tok_s": round(B / (ms / 1e3), 2), "ms_per_step": round(ms, 4),
                         "step_bytes": int(sb), "frac": round(sb / (ms / 1e3) / HBM_PEAK, 4),
                         "prefill_chunk_ms": round(pre_ms, 3), "prefill_to_here_ms": round(cum_ms, 2)})
            log(f"[long {quant} {kv_quant} cache B={B}] context {L}: {rows[-1]['tok_s']} tok/s, {ms:.3f} ms/step, "
                f"{chunk}-token chunk prefill {pre_ms:.2f} ms per sequence")
            tok.copy_(tok_ctx)
    graph.close()
    del eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rows


def serve_uneven(quant="w4a16", n_req=32, slots=16, prompt=128, lo=16, hi=512, seed=5):
    """Continuous batching over the paged cache against lockstep batches, on
    requests of uneven output length (uniform in [lo, hi]), each a `prompt`-
    token random prompt: useful tokens per second of wall time (prefills
    included), eager decode steps in both modes.  Lockstep runs `slots`
    requests at a time until the longest finishes (finished rows keep
    decoding, their tokens not counted); continuous batching admits a request
    as soon as a slot and its pages free up and moves the last live slot into
    a finished one (no K/V copied)."""
    import numpy as np
    import torch

    import synth
    from w4a16_weight_streaming_amd import Engine

    cfg = synth.get_config("e2b")
    V = cfg["vocab_size"]
    w = synth.generate(cfg, quant, seed=0)
    rng = np.random.default_rng(seed)
    olen = [int(x) for x in rng.integers(lo, hi + 1, size=n_req)]
    prompts = [torch.from_numpy(synth.tokens(prompt, 200 + i, V)) for i in range(n_req)]
    useful = sum(olen)
    max_ctx = prompt + hi
    per_req = (max_ctx + 127) // 128
    out = {"requests": n_req, "slots": slots, "prompt": prompt, "output_lengths": [lo, hi],
           "useful_tokens": useful}
    for mode in ("lockstep", "continuous"):
        paged = mode == "continuous"
        eng = Engine(cfg, quant, w, max_batch=slots, max_ctx=max_ctx, max_rows=128,
                     n_pages=slots * per_req if paged else 0)
        dev = eng.device
        ps = [p.to(dev) for p in prompts]
        stream = torch.cuda.Stream(dev)
        steps = 0
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            t0 = time.time()
            if not paged:
                for b0 in range(0, n_req, slots):
                    grp = list(range(b0, min(n_req, b0 + slots)))
                    tok = torch.zeros(len(grp), dtype=torch.int32, device=dev)
                    for j, i in enumerate(grp):
                        eng.prefill(j, ps[i], 0, tok[j:j + 1])
                    pos = torch.full((len(grp),), prompt, dtype=torch.int32, device=dev)
                    for _ in range(max(olen[i] for i in grp)):
                        eng.decode_step(tok, pos, tok)
                        pos.add_(1)
                        steps += 1
            else:
                pending, live = list(range(n_req)), []   # live: [request, steps left]
                tok = torch.zeros(slots, dtype=torch.int32, device=dev)
                pos = torch.zeros(slots, dtype=torch.int32, device=dev)
                while pending or live:
                    while pending and len(live) < slots and eng.pages_free() >= per_req:
                        i = pending.pop(0)
                        b = len(live)
                        eng.reserve(b, prompt + olen[i])
                        eng.prefill(b, ps[i], 0, tok[b:b + 1])
                        pos[b] = prompt
                        live.append([i, olen[i]])
                    B = len(live)
                    eng.decode_step(tok[:B], pos[:B], tok[:B])
                    pos[:B] += 1
                    steps += 1
                    for b in reversed(range(B)):
                        live[b][1] -= 1
                        if live[b][1] == 0:
                            eng.release(b)
                            last = len(live) - 1
                            if b != last:
                                eng.move(last, b)
                                tok[b] = tok[last]
                                pos[b] = pos[last]
                                live[b] = live[last]
                            live.pop()
            torch.cuda.synchronize()
            dt = time.time() - t0
            eng.check()
        out[mode] = {"seconds": round(dt, 3), "decode_steps": steps, "useful_tok_s": round(useful / dt, 1)}
        log(f"[serve {quant}] {mode}: {useful} useful tokens in {dt:.2f} s ({steps} steps), "
            f"{useful / dt:.0f} tok/s")
        del eng
        torch.cuda.empty_cache()
    out["speedup"] = round(out["continuous"]["useful_tok_s"] / out["lockstep"]["useful_tok_s"], 3)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--repeats", type=int, default=5, help="timed loops of K steps (median reported)")
    ap.add_argument("--quant", choices=["bf16", "w4a16"], default=None,
                    help="weights (default bf16; w4a16 with --long)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=128)
    ap.add_argument("--eager", action="store_true", help="launch kernels per step instead of a graph")
    ap.add_argument("--cpu-steps", type=int, default=24, help="oracle decode steps timed (0: skip)")
    ap.add_argument("--profile-steps", type=int, default=32)
    ap.add_argument("--no-aux", action="store_true", help="skip the W4A16 / batch-64 / long-context lines")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context lines")
    ap.add_argument("--long", action="store_true", help="long-context workload alone (see above)")
    ap.add_argument("--kv", choices=["bf16", "int8"], default="bf16", help="K/V cache format (--long)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device copy (reference kernel for PMC byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(sequences shard across GPUs with no per-step exchange).",
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
        rows = long_context(args.quant, args.batch, kv_quant=args.kv)
        cfg = synth.get_config("e2b")
        mean = sum(r["tok_s"] for r in rows) / len(rows)
        ms_mean = sum(r["ms_per_step"] for r in rows) / len(rows)
        out = {"metric": METRIC, "value": round(mean, 2), "unit": "tok/s", "n_gpus": 1,
               "steps": 64 * len(rows), "warmup": 2 * len(rows), "ms_per_step": round(ms_mean, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.quant,
               "data": "synthetic",
               "config": {"workload": f"E2B shape, {args.quant} weights, {args.kv} K/V cache, long-context decode: batch "
                                      f"{args.batch}, context grown 500 -> 8,000 by 500-token random "
                                      f"prefill chunks, 64 greedy decode steps timed at each length "
                                      f"(mean over lengths)", "quant": args.quant, "batch": args.batch},
               "per_length": rows}
        print(json.dumps(out), flush=True)
        return

    calib = calibrate(torch)
    cfg = synth.get_config("e2b")
    B, P, K, W, R = args.batch, args.prompt, args.steps, args.warmup, max(1, args.repeats)
    head = measure(cfg, args.quant, B, P, K, W, args.profile_steps, R, args.eager, args.cpu_steps,
                   f"{args.quant} B={B}")
    also = []
    if not args.no_aux:
        for q, b, eq in (("w4a16", 1, "bf16"), ("w4a16", 1, "w4a16"), ("bf16", 64, "bf16"),
                         ("w4a16", 64, "bf16"), ("w4a16", 64, "w4a16")):
            if (q, b, eq) == (args.quant, B, "bf16"):
                continue
            lab = f"{q}{' + int4 vocabulary tables' if eq == 'w4a16' else ''} B={b}"
            r = measure(cfg, q, b, P, K, W, 8, R, False, 0, lab, eq)
            also.append({"quant": q, "embed_quant": eq, "batch": b, "tok_s": round(r["value"], 2),
                         "ms_per_step": round(r["ms_per_step"], 4), "repeats": r["repeats"],
                         "step_roofline": step_roofline(r, calib), "roofline": roofline_of(r, q, b, calib, eq),
                         "kernel_kinds": kinds_summary(r, 8), "prefill": r["prefill"]})
        if not args.no_long:
            sv = serve_uneven()
            also.append(dict(workload="serving uneven requests: continuous batching over the paged K/V cache "
                                      "(128-position pages) vs lockstep batches, E2B W4A16", **sv))
            for b, kq in ((1, "bf16"), (8, "bf16"), (1, "int8"), (8, "int8")):
                rows = long_context("w4a16", b, lengths=(500, 4000, 8000), kv_quant=kq)
                also.append({"workload": f"long context, w4a16, {kq} K/V cache, batch {b}: context grown by "
                                         f"500-token prefill chunks, 64 graph-replayed steps timed at each "
                                         f"listed length", "quant": "w4a16", "kv_quant": kq, "batch": b,
                             "per_length": rows})
    wl = (f"E2B shape ({cfg['num_hidden_layers']} layers, hidden {cfg['hidden_size']}, vocab "
          f"{cfg['vocab_size']}), {args.quant} weights, batch {B}, {P}-token random prompt then {K} greedy "
          f"decode steps (KV length {P + 1}..{P + K})")
    out = {
        "metric": METRIC, "value": round(head["value"], 2), "unit": "tok/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(head["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.quant, "data": "synthetic",
        "config": {"workload": wl, "quant": args.quant, "batch": B, "prompt": P, "decode_steps": K,
                   "graph": head["graph"]},
        "repeats": head["repeats"],
        "roofline": roofline_of(head, args.quant, B, calib) if head["kinds"] else None,
        "step_roofline": step_roofline(head, calib),
        "calibration": {"method": "streaming reduction over 4 GiB (e2b_stream_reduce), best of 5",
                        "read_GBps": round(calib / 1e9, 1)},
        "kernel_kinds": kinds_summary(head, args.profile_steps),
        "prefill": head["prefill"],
        "cpu_baseline": head.get("cpu_baseline"),
        "also": also,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
