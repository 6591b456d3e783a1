"""HBM traffic per kernel launch from two rocprofv3 counter runs.

Usage (after two runs of the same command, one with `--pmc FETCH_SIZE`, one
with `--pmc WRITE_SIZE`, both with `--output-format csv`, the command running
`bench.py --copy-calibration` so that a 1 GiB elementwise copy is among the
dispatches):

    python -m w4a16_weight_streaming_amd.pmc FETCH_DIR WRITE_DIR OUT.json

or, for any other counters (one or more `--pmc` runs):

    python -m w4a16_weight_streaming_amd.pmc --counters PATTERN DIR [DIR ...]

which prints, as a markdown table, the mean per-dispatch value of every
counter found under the DIRs for each kernel whose name contains PATTERN
(`--ratios` instead of `--counters`: the shares formed from the SQ counters
of the two passes the shader-counter profile takes: waiting, VALU-active and
LDS bank-conflict shares and the MFMA-busy ratio); or, for a `--kernel-trace`
run of the decode loop,

    python -m w4a16_weight_streaming_amd.pmc --steps N DIR

which splits the trace into decode steps (each ends with the argmax's final
kernel) and tabulates the last N: kernels per step, their summed durations
and the step's span on the GPU clock, and each kernel's share.

Both FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by what it
reads for the reference copy (1 GiB read, 1 GiB written), so the factors
absorb any unit or sampling convention of the counters.  OUT.json records the
mean per-dispatch values of every kernel of this library, the two factors,
and a hash of the kernel sources, so that a reader can tell when the profile
no longer describes the current kernels.
"""
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

GIB = float(1 << 30)
HERE = os.path.dirname(os.path.abspath(__file__))


KERNEL_SOURCES = ("kernels.hip", "attn_prefill.hip", "gemm_impl.h", "gemm_bf16.hip", "gemm_w4.hip", "dev_common.h",
                  "e2b_internal.h")


def kernels_sha():
    """Hash of every device source, to tell whether a profile still describes
    the current kernels."""
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_counter(d, counter):
    """{kernel name: [per-dispatch value (KiB)]} for one counter run."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = defaultdict(lambda: defaultdict(float))  # kernel -> dispatch -> value
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name", "").strip() != counter:
                    continue
                name = row["Kernel_Name"].strip()
                disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                per[name][disp] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def short(name):
    return name.split("(")[0].strip()


def main(fetch_dir, write_dir, out):
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "neg" in k.lower() and "e2b::" not in k]
    if not copy:
        raise SystemExit("reference copy kernel not found (run bench.py with --copy-calibration)")
    big = lambda d, k: max(d.get(k, [0.0]))
    ck = max(copy, key=lambda k: big(fetch, k))
    f_copy, w_copy = big(fetch, ck) * 1024.0, big(write, ck) * 1024.0
    res = {"kernels_sha": kernels_sha(), "reference_kernel": short(ck),
           "reference_fetch_kib": f_copy / 1024.0, "reference_write_kib": w_copy / 1024.0,
           "fetch_factor": GIB / f_copy, "write_factor": GIB / w_copy, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if "e2b::" not in k:
            continue
        fv, wv = fetch.get(k, []), write.get(k, [])
        res["kernels"][short(k)] = {
            "dispatches": max(len(fv), len(wv)),
            "fetch_bytes": 1024.0 * sum(fv) / max(len(fv), 1),
            "write_bytes": 1024.0 * sum(wv) / max(len(wv), 1)}
    with open(out, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    print(f"reference {short(ck)}: fetch {f_copy / GIB:.4f} GiB, write {w_copy / GIB:.4f} GiB "
          f"for 1 GiB each; {len(res['kernels'])} kernels -> {out}")


def counter_means(pattern, dirs):
    """{kernel: (dispatches, {counter: mean per-dispatch value})} for the
    kernels whose name contains `pattern`."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))  # kernel -> counter -> dispatch
    for d in dirs:
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    name = row["Kernel_Name"].strip()
                    if pattern not in name:
                        continue
                    disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                    per[short(name)][row["Counter_Name"].strip()][disp] += float(row["Counter_Value"])
    return {k: (max(len(v) for v in c.values()), {n: sum(v.values()) / len(v) for n, v in c.items()})
            for k, c in per.items()}


def ratios_table(pattern, dirs):
    """Markdown table of the shares the SQ counters give per kernel: cycles
    waiting on a dependency and VALU-active cycles (of the wave cycles), LDS
    bank-conflict cycles (of the LDS-active cycles), MFMA-busy cycles over
    busy-CU cycles (two units: compare between kernels), and the instruction
    counts; heaviest kernels (dispatches x wave cycles) first."""
    m = counter_means(pattern, dirs)
    g = lambda c, n: c.get(n, 0.0)
    lines = ["| kernel | dispatches | wait / wave cycles | VALU active / wave cycles | LDS bank-conflict / "
             "LDS-active cycles | MFMA-busy / busy-CU cycles | VALU insts | MFMA insts | LDS insts |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k, (n, c) in sorted(m.items(), key=lambda kv: -kv[1][0] * g(kv[1][1], "SQ_WAVE_CYCLES")):
        wc = g(c, "SQ_WAVE_CYCLES") or 1.0
        lds = g(c, "SQ_LDS_IDX_ACTIVE")
        lines.append(f"| `{k}` | {n} | {g(c, 'SQ_WAIT_INST_ANY') / wc:.2f} | {g(c, 'SQ_ACTIVE_INST_VALU') / wc:.2f} | "
                     f"{(g(c, 'SQ_LDS_BANK_CONFLICT') / lds if lds else 0.0):.2f} | "
                     f"{g(c, 'SQ_VALU_MFMA_BUSY_CYCLES') / (g(c, 'SQ_BUSY_CU_CYCLES') or 1.0):.2f} | "
                     f"{g(c, 'SQ_INSTS_VALU'):.3g} | {g(c, 'SQ_INSTS_MFMA'):.3g} | {g(c, 'SQ_INSTS_LDS'):.3g} |")
    return "\n".join(lines)


def counters_table(pattern, dirs):
    """Markdown table: mean per-dispatch value of each counter, per kernel
    whose name contains `pattern`."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))  # kernel -> counter -> dispatch
    for d in dirs:
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    name = row["Kernel_Name"].strip()
                    if pattern not in name:
                        continue
                    disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                    per[short(name)][row["Counter_Name"].strip()][disp] += float(row["Counter_Value"])
    names = sorted({c for k in per.values() for c in k})
    lines = ["| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---:|" + "---:|" * len(names)]
    for k in sorted(per):
        n = max(len(v) for v in per[k].values())
        cells = []
        for c in names:
            v = per[k].get(c, {})
            cells.append(f"{sum(v.values()) / len(v):.4g}" if v else "")
        lines.append(f"| `{k}` | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def step_chain(trace_dir, last):
    """Markdown summary of the last `last` decode steps of a kernel trace: a
    step is the run of dispatches that ends with `k_argmax_final`."""
    rows = []
    for fn in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"].strip()))
    rows.sort()
    ends = [i for i, r in enumerate(rows) if "k_argmax_final" in r[2]]
    steps = [rows[a + 1:b + 1] for a, b in zip(ends[:-1], ends[1:])][-last:]
    if not steps:
        raise SystemExit("no decode steps in the trace")
    med = lambda xs: sorted(xs)[len(xs) // 2]
    n = [len(s) for s in steps]
    busy = [sum(e - b for b, e, _ in s) / 1e3 for s in steps]
    span = [(s[-1][1] - s[0][0]) / 1e3 for s in steps]
    per = defaultdict(list)
    for s in steps:
        for b, e, k in s:
            per[short(k)].append((e - b) / 1e3)
    lines = [f"{len(steps)} steps: median {med(n)} kernels per step (min {min(n)}, max {max(n)}); "
             f"summed kernel time {med(busy):.1f} us, span from the first kernel's start to the last "
             f"kernel's end {med(span):.1f} us (median), so {med(span) - med(busy):.1f} us "
             f"({(med(span) - med(busy)) / max(med(n) - 1, 1):.2f} us per boundary) lie between kernels.",
             "", "| kernel | per step | mean us | us per step | share of kernel time |",
             "|---|---:|---:|---:|---:|"]
    tot = sum(sum(v) for v in per.values())
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v) / len(steps):.1f} | {sum(v) / len(v):.2f} | "
                     f"{sum(v) / len(steps):.1f} | {100 * sum(v) / tot:.1f}% |")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "--steps":
        print(step_chain(sys.argv[3], int(sys.argv[2])))
    elif len(sys.argv) >= 4 and sys.argv[1] == "--counters":
        print(counters_table(sys.argv[2], sys.argv[3:]))
    elif len(sys.argv) >= 4 and sys.argv[1] == "--ratios":
        print(ratios_table(sys.argv[2], sys.argv[3:]))
    elif len(sys.argv) == 4:
        main(*sys.argv[1:])
    else:
        raise SystemExit(__doc__)
