"""Host-side checks of the measurement tooling (no GPU): the byte model the
bench's roofline fractions divide by, pinned to closed forms of the E2B shape;
the PMC traffic scaling against a reference copy; the decode-step table of a
kernel trace; and the kernel symbols the bench looks up."""
import csv
import json
import os
import re

import pytest

import bench
import synth
from w4a16_weight_streaming_amd import pmc

E2B = synth.get_config("e2b")


def test_weight_bytes_per_step_closed_form():
    """Every linear once, the tied lm_head once, the norm gains; the per-layer
    table is gathered, not streamed.  Linear parameters of the E2B shape:
    q + o 264,241,152; k + v (15 source layers) 14,155,776; MLP
    1,557,135,360; PLE gate + projection 27,525,120; per-layer model
    projection 13,762,560 (1,876,819,968 in all); embedding 402,653,184."""
    lin = 264_241_152 + 14_155_776 + 1_557_135_360 + 27_525_120 + 13_762_560
    assert lin == 1_876_819_968
    emb = 262_144 * 1_536
    _, w_bf16 = bench.step_bytes(E2B, "bf16", 1, [128])
    _, w_w4 = bench.step_bytes(E2B, "w4a16", 1, [128])
    gains = w_bf16 - 2 * (lin + emb)
    assert 0 < gains < 1_000_000          # norm gains and layer scalars: < 0.02%
    assert w_bf16 == 4_559_518_278
    # W4A16: 4 bits per weight plus one bf16 scale per 32 (= 9/16 byte)
    assert w_w4 == lin * 9 // 16 + 2 * emb + gains
    assert w_w4 == 1_861_589_574


@pytest.mark.parametrize("T", [1, 129, 512, 513, 640, 8000])
def test_unique_kv_bytes_closed_form(T):
    """Unique K/V read per sequence at T attended positions: 12 sliding source
    layers (hd 256, window 512) and 3 full ones (hd 512), K and V, bf16:
    12 * 2 * 256 * 2 * min(T, 512) + 3 * 2 * 512 * 2 * T; logical (all 35
    layers re-reading their source): 28 sliding and 7 full."""
    assert bench.kv_bytes(E2B, T - 1, True) == 12_288 * min(T, 512) + 6_144 * T
    assert bench.kv_bytes(E2B, T - 1, False) == 28_672 * min(T, 512) + 14_336 * T
    # int8 rows: hd codes plus one fp32 scale
    assert bench.kv_bytes(E2B, T - 1, True, "int8") == (12 * 2 * 260 * min(T, 512)
                                                         + 3 * 2 * 516 * T)


def test_step_bytes_adds_kv_and_writes_per_sequence():
    one, w = bench.step_bytes(E2B, "bf16", 1, [200])
    four, w4 = bench.step_bytes(E2B, "bf16", 4, [200])
    assert w == w4
    per_seq = one - w
    assert four - w == 4 * per_seq
    # per sequence: the unique K/V read, the new token's K/V (18,432 B) and the gathers
    gathers = 2 * 1_536 + 2 * 35 * 256
    assert per_seq == bench.kv_bytes(E2B, 200, True) + 18_432 + gathers


def test_kernel_patterns():
    pat = {(k, q, b): bench.kernel_pattern(k, q, b) for k in ("gate_up", "down", "lm_head")
           for q in ("bf16", "w4a16") for b in (1, 8, 64)}
    assert re.fullmatch(pat[("gate_up", "bf16", 1)], "void e2b::k_gemv<0, 1536, 4, 3>")
    assert re.fullmatch(pat[("gate_up", "w4a16", 1)], "void e2b::k_gemv<1, 1536, 3, 3>")
    # the batched gate/up carries the GeGLU epilogue: bf16 <= 2 m-tiles, W4A16 1
    assert re.fullmatch(pat[("gate_up", "bf16", 64)], "void e2b::k_gemm<0, 2, 2, 0, 3, 1>")
    assert re.fullmatch(pat[("gate_up", "w4a16", 64)], "void e2b::k_gemm<1, 2, 1, 0, 3, 1>")
    assert re.fullmatch(pat[("down", "bf16", 64)], "void e2b::k_gemm<0, 2, 4, 0, 4, 1>")
    assert re.fullmatch(pat[("down", "w4a16", 8)], "void e2b::k_gemm<1, 2, 1, 0, 4, 1>")
    # W4A16 q/k/v, O and down in 16-row blocks; bf16 q/k/v and O above 32 rows in 32-row blocks
    assert re.fullmatch(pat[("down", "w4a16", 64)], "void e2b::k_gemm<1, 2, 1, 0, 4, 1>")
    assert re.fullmatch(bench.kernel_pattern("qkv", "w4a16", 64), "void e2b::k_gemm<1, 2, 1, 0, 1, 1>")
    assert re.fullmatch(bench.kernel_pattern("o", "bf16", 64), "void e2b::k_gemm<0, 2, 2, 0, 2, 1>")
    assert not re.fullmatch(pat[("down", "bf16", 64)], "void e2b::k_gemm<0, 2, 1, 0, 4, 1>")
    # the lm_head follows the vocabulary table's format, not the linears'
    assert re.fullmatch(bench.kernel_pattern("lm_head", "w4a16", 1), "void e2b::k_gemv<0, 1536, 4, 8>")
    assert re.fullmatch(bench.kernel_pattern("lm_head", "w4a16", 1, "w4a16"), "void e2b::k_gemv<1, 1536, 4, 8>")
    assert bench.kernel_pattern("attn", "bf16", 1) is None


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i, name, counter, v])


def test_pmc_traffic_scaled_by_the_reference_copy(tmp_path):
    """Counters in KiB per dispatch, scaled so that the 1 GiB reference copy
    reads and writes exactly 1 GiB; a kernel's figure is its dispatch mean."""
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)"
    k = "void e2b::k_gemv<0, 1536, 4, 3>(e2b::Lin, int, e2b::Prologue, e2b::Epilogue)"
    # the counter reports half of what is read (as FETCH_SIZE does here)
    fetch = [(copy, 524_288.0), (k, 29_000.0), (k, 31_000.0)]
    write = [(copy, 1_048_576.0), (k, 150.0), (k, 160.0)]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    out = str(tmp_path / "t.json")
    pmc.main(str(tmp_path / "f"), str(tmp_path / "w"), out)
    d = json.load(open(out))
    assert d["fetch_factor"] == pytest.approx(2.0)
    assert d["write_factor"] == pytest.approx(1.0)
    e = d["kernels"]["void e2b::k_gemv<0, 1536, 4, 3>"]
    assert e["dispatches"] == 2
    assert e["fetch_bytes"] * d["fetch_factor"] == pytest.approx(30_000.0 * 1024 * 2)
    assert e["write_bytes"] * d["write_factor"] == pytest.approx(155.0 * 1024)
    assert d["kernels_sha"] == pmc.kernels_sha()


def test_step_chain_table(tmp_path):
    """A step is the run of dispatches ending with the argmax's final kernel;
    the table covers the last N steps."""
    rows, t = [], 0
    def k(name, dur, gap=1000):
        nonlocal t
        t += gap
        rows.append((name, t, t + dur))
        t += dur
    k("e2b::k_embed<0>(...)", 50_000)                 # before the first step: dropped
    k("e2b::k_argmax_final(...)", 4_000)
    for s in range(3):
        k("void e2b::k_gemv<0, 1536, 4, 3>(...)", 10_000 + 1_000 * s)
        k("void e2b::k_attn_dec<256, 0>(...)", 8_000, gap=500)
        k("e2b::k_argmax_final(...)", 4_000, gap=500)
    d = tmp_path / "tr"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, a, b in rows:
            w.writerow([name, a, b])
    out = pmc.step_chain(str(d), 2)
    first = out.splitlines()[0]
    assert first.startswith("2 steps: median 3 kernels per step")
    # the last two steps: 11 + 8 + 4 and 12 + 8 + 4 us of kernels; median (upper) 24
    assert "summed kernel time 24.0 us" in first
    # span: first kernel's start to the last kernel's end = 12 + 0.5 + 8 + 0.5 + 4 = 25 us,
    # 1 us of it in the two gaps
    assert "25.0 us (median)" in first and "1.0 us (0.50 us per boundary)" in first
    assert "| `void e2b::k_gemv<0, 1536, 4, 3>` | 1.0 | 11.50 | 11.5 |" in out


def test_sq_ratios_table(tmp_path):
    """The shares of the shader-counter profile: waiting and VALU-active over
    wave cycles, bank conflicts over LDS-active cycles, MFMA-busy over
    busy-CU cycles; per-dispatch means first (two dispatches here)."""
    k = "void e2b::k_gemm<0, 2, 2, 0, 3, 1>(e2b::Lin, int, e2b::GemmA, int, e2b::Epilogue)"
    vals = {"SQ_WAVE_CYCLES": (1000.0, 3000.0), "SQ_WAIT_INST_ANY": (300.0, 500.0),
            "SQ_ACTIVE_INST_VALU": (100.0, 300.0), "SQ_LDS_IDX_ACTIVE": (50.0, 150.0),
            "SQ_LDS_BANK_CONFLICT": (20.0, 20.0), "SQ_BUSY_CU_CYCLES": (400.0, 400.0),
            "SQ_VALU_MFMA_BUSY_CYCLES": (200.0, 600.0), "SQ_INSTS_VALU": (10.0, 30.0),
            "SQ_INSTS_MFMA": (4.0, 4.0), "SQ_INSTS_LDS": (6.0, 8.0)}
    d = tmp_path / "sq"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, (a, b) in vals.items():
            w.writerow([1, k, name, a])
            w.writerow([2, k, name, b])
    row = pmc.ratios_table("e2b::k_", [str(d)]).splitlines()[2]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[0] == "`void e2b::k_gemm<0, 2, 2, 0, 3, 1>`" and cells[1] == "2"
    # means: wave 2000, wait 400, valu 200, lds-active 100, conflicts 20, busy-CU 400, MFMA 400
    assert cells[2:6] == ["0.20", "0.10", "0.20", "1.00"]
    assert cells[6:] == ["20", "4", "7"]
