"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

The oracle stores K/V rounded to bf16, as the cache the pages describe does
(the GPU path stores bf16 K/V too); everything else in it is fp64.

Tolerances (fixed by the workload definition, not tuned):
  * int4 unpack (one-hot columns), the embedding gathers, K/V-share identity:
    bit-exact;
  * logits: max |GPU - oracle| <= 2e-2 (bf16) / 3e-2 (W4A16) of max |oracle logit|;
  * greedy token: bit-exact argmax (lowest index on ties) of the GPU's own fp32
    logits, and equal to the oracle's wherever the oracle's top-2 gap exceeds
    1e-2.  Teacher-forced: the oracle replays the GPU's tokens, so one flip
    cannot cascade.  Over the 512-step workloads the greedy tokens agree with
    the oracle's on at least 99% of the steps.  As an extra check, a token
    that differs must still be a valid argmax of the oracle's logits within
    the measured error e = max |GPU - oracle|: oracle[gpu token] >=
    max(oracle) - 2e.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "w4a16": 3e-2}
# The E2B bf16 workload's own logits move by this fraction of max |logit| when
# every cached K/V element changes by 3e-6 relative before its bf16 rounding
# (test_workload_conditioning.py::test_e2b_bf16_cache_rounding_sensitivity):
# two logits closer than twice that can trade places in any implementation
# that is not bit-identical to the fp64 oracle.  (The W4A16 workload moves by
# ~1e-5 under the same change: its rule stays the fixed 1e-2 gap.)
E2B_BF16_DRIFT = 5.5e-3


_CAPMAN = None


@pytest.fixture(scope="session", autouse=True)
def _progress_channel(request):
    global _CAPMAN
    _CAPMAN = request.config.pluginmanager.getplugin("capturemanager")
    yield


def progress(msg):
    """A progress line of a long test, written past pytest's output capture:
    a run that prints nothing for minutes is taken to be hung."""
    if _CAPMAN is None:
        print(msg, flush=True)
        return
    with _CAPMAN.global_and_fixture_disabled():
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    return torch, torch.device("cuda:0")


def _engine(cfg, quant, w, max_batch, max_ctx, max_rows, kv_quant="bf16"):
    from w4a16_weight_streaming_amd import Engine
    return Engine(cfg, quant, w, max_batch=max_batch, max_ctx=max_ctx, max_rows=max_rows,
                  kv_quant=kv_quant)


class Stats:
    def __init__(self, quant, drift=0.0):
        self.tol, self.n, self.agree, self.worst = TOL[quant], 0, 0, 0.0
        self.drift = drift   # workload sensitivity (see E2B_BF16_DRIFT)
        self.flips = []
        self.min_gap = float("inf")

    def add(self, got_logits, got_tok, ref_logits, where=""):
        got = np.asarray(got_logits, np.float64)
        err = float(np.max(np.abs(got - ref_logits)) / np.max(np.abs(ref_logits)))
        self.worst = max(self.worst, err)
        assert err <= self.tol, f"{where}: logit error {err:.3e} > {self.tol}"
        own = int(np.argmax(np.asarray(got_logits, np.float32)))   # first maximum
        assert got_tok == own, f"{where}: argmax {got_tok} != first maximum {own} of its logits"
        ref_tok = int(np.argmax(ref_logits))
        top2 = np.sort(ref_logits)[-2:]
        gap = top2[1] - top2[0]
        self.min_gap = min(self.min_gap, float(gap))
        # a different token is a near-tie below a 1e-2 gap, or below twice the
        # workload's pinned drift (relative to max |logit|) where that is larger
        gap_min = max(1e-2, 2 * self.drift * float(np.max(np.abs(ref_logits))))
        if gap > gap_min:
            assert got_tok == ref_tok, f"{where}: token {got_tok} != oracle {ref_tok} (gap {gap:.3e})"
        e = float(np.max(np.abs(got - ref_logits)))
        assert ref_logits[got_tok] >= ref_logits[ref_tok] - 2 * e, \
            f"{where}: token {got_tok} is not an argmax within error {e:.3e}"
        self.n += 1
        self.agree += int(got_tok == ref_tok)
        if got_tok != ref_tok:
            self.flips.append(f"{where}: gap {gap:.2e} err {e:.2e}")

    def finish(self, label="", min_agree=None):
        """Print the run's record; with min_agree, assert the greedy agreement
        rate (the 512-step workloads: >= 0.99)."""
        print(f"[{label}] steps {self.n} agree {self.agree} ({self.agree / max(self.n, 1):.4f}) "
              f"worst rel err {self.worst:.3e} smallest oracle top-2 gap {self.min_gap:.3e}"
              + "".join(f"\n  near-tie flip at {f}" for f in self.flips), flush=True)
        if min_agree is not None:
            assert self.agree >= min_agree * self.n, \
                f"greedy agreement {self.agree}/{self.n} below {min_agree}"


def run_greedy(torch, eng, orc, prompts, steps, quant, logits=True):
    """Prefill each sequence, then `steps` batched greedy decode steps, comparing
    every step's logits with the teacher-forced oracle."""
    dev = eng.device
    V = eng.cfg.vocab_size
    B = len(prompts)
    st = Stats(quant)
    am = torch.zeros(B, dtype=torch.int32, device=dev)
    lg = torch.zeros(B, V, dtype=torch.float32, device=dev)
    nxt = []
    for b, p in enumerate(prompts):
        a1 = torch.zeros(1, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        eng.prefill(b, torch.from_numpy(np.asarray(p, np.int32)).to(dev), 0, a1, l1)
        eng.check()
        _, ref = orc.prefill(b, p)
        st.add(l1.cpu().numpy()[0], int(a1.item()), ref, f"prefill seq {b}")
        nxt.append(int(a1.item()))
    lens = [len(p) for p in prompts]
    for i in range(steps):
        tok = torch.tensor(nxt, dtype=torch.int32, device=dev)
        pos = torch.tensor(lens, dtype=torch.int32, device=dev)
        eng.decode_step(tok, pos, am, lg)
        eng.check()
        got_l, got_t = lg.cpu().numpy(), am.cpu().numpy()
        for b in range(B):
            _, ref, _ = orc.step(b, nxt[b], lens[b])
            st.add(got_l[b], int(got_t[b]), ref, f"step {i} seq {b}")
        nxt = [int(t) for t in got_t]
        lens = [x + 1 for x in lens]
    st.finish(f"{eng.cfg.num_hidden_layers} layers {quant} B={B}")
    return st


# ---------------------------------------------------------------- matvec
def _as_dev(torch, a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    return torch.from_numpy(a).to(dev)


@pytest.mark.parametrize("mode", ["one_row", "batched"])
@pytest.mark.parametrize("quant", ["bf16", "w4a16"])
@pytest.mark.parametrize("N,K", [(64, 32), (40, 128), (96, 3072), (96, 256), (256, 512), (300, 1536),
                                 (128, 2048), (64, 4096), (32, 6144), (24, 12288), (1536, 12288),
                                 (24576, 1536)])
def test_matvec_one_hot_is_exact(torch_dev, quant, N, K, mode):
    """x = e_k returns column k of the decoded matrix bit for bit (int4 unpack
    and scale exact; nibble order natural; K slices summed correctly), through
    the one-row matvec kernel (one call per row) and through the batched
    matrix-core path (all rows in one call), which reads the weights from the
    fragment-ordered copy batched decode uses when N % 16 == 0 (one or two
    column tiles per wave by shape) and the row-major layout otherwise."""
    torch, dev = torch_dev
    from w4a16_weight_streaming_amd import matvec
    seed = 100 + K
    if quant == "bf16":
        w = synth.normal_bf16((N, K), seed, "w")
        scale = None
    else:
        w = synth.bits32((N, K // 8), seed, "w")
        scale = synth.uniform_bf16((N, K // 32), seed, "s", 0.002, 0.02)
    ks = sorted(k for k in set([0, 1, 7, 8, 31, 32, 33, K // 2, K - 1] +
                                list(range(3, K, max(1, K // 13)))) if k < K)
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = torch.zeros(len(ks), N, dtype=torch.float32, device=dev)
    wd_, sd_ = _as_dev(torch, w, dev), None if scale is None else _as_dev(torch, scale, dev)
    xd = torch.from_numpy(x).to(dev)
    if mode == "batched":
        matvec(quant, wd_, sd_, xd, y)
    else:
        for r in range(len(ks)):
            matvec(quant, wd_, sd_, xd[r:r + 1], y[r:r + 1])
    got = y.cpu().numpy()
    for r, k in enumerate(ks):
        e = np.zeros(K)
        e[k] = 1.0
        ref = oracle.linear(quant, w, scale, N, K, e)          # exact decoded column
        assert np.array_equal(got[r].astype(np.float64), ref), (k, np.max(np.abs(got[r] - ref)))


@pytest.mark.parametrize("quant", ["bf16", "w4a16"])
@pytest.mark.parametrize("N,K,rows", [(1536, 1536, 1), (2560, 1536, 3), (1536, 4096, 1),
                                      (1536, 12288, 2), (160, 256, 5), (32, 32, 1),
                                      (2560, 1536, 64), (1536, 12288, 70), (300, 2048, 65),
                                      (96, 1024, 7), (1000, 4096, 130)])
def test_matvec_random_matches_oracle(torch_dev, quant, N, K, rows):
    """Random x: |y - y_oracle| <= c * sum_k |w_nk x_k|.  x is carried as a bf16
    hi/lo pair (<= 2^-18 relative) and sums are fp32: c = 1e-5 for bf16 weights
    (a dropped lo part would show as ~2^-9); for W4A16 the biased code sums
    (128 + c) x cancel against 136 sum x, worst case ~6e-5, so c = 1e-4."""
    torch, dev = torch_dev
    from w4a16_weight_streaming_amd import matvec
    rng = np.random.default_rng(K + N)
    if quant == "bf16":
        w = synth.normal_bf16((N, K), 7, "w")
        scale = None
        wd = synth.bf16_to_f32(w).astype(np.float64)
    else:
        w = synth.bits32((N, K // 8), 7, "w")
        scale = synth.uniform_bf16((N, K // 32), 7, "s", 0.002, 0.02)
        wd = np.stack([[oracle.decode_weight("w4a16", w, scale, N, K, n, k) for k in range(K)]
                       for n in range(min(N, 4))])
    x = rng.normal(size=(rows, K)).astype(np.float32)
    y = torch.zeros(rows, N, dtype=torch.float32, device=dev)
    matvec(quant, _as_dev(torch, w, dev), None if scale is None else _as_dev(torch, scale, dev),
           torch.from_numpy(x).to(dev), y)
    got = y.cpu().numpy()
    for r in range(rows):
        ref = oracle.linear(quant, w, scale, N, K, x[r].astype(np.float64))
        nb = wd.shape[0]
        c = 1e-5 if quant == "bf16" else 1e-4
        bound = c * (np.abs(wd) @ np.abs(x[r].astype(np.float64)))
        assert np.all(np.abs(got[r, :nb] - ref[:nb]) <= bound + 1e-30)
        scale_all = np.max(np.abs(ref))
        assert np.max(np.abs(got[r] - ref)) <= 1e-4 * scale_all * np.sqrt(K)


# ---------------------------------------------------------------- whole step, toy
@pytest.mark.parametrize("name", ["toy", "toy10"])
@pytest.mark.parametrize("quant,embed_quant", [("bf16", "bf16"), ("w4a16", "bf16"), ("w4a16", "w4a16")])
def test_toy_greedy_parity(torch_dev, name, quant, embed_quant):
    """8-token prompt, 32 greedy steps (crosses the 16-wide window); the
    vocabulary tables in bf16 or int4."""
    torch, dev = torch_dev
    cfg = synth.get_config(name)
    w = synth.generate(cfg, quant, seed=0, embed_quant=embed_quant)
    eng = _engine(cfg, quant, w, 1, 48, 8)
    orc = oracle.Oracle(cfg, quant, w, 1, 48)
    run_greedy(torch, eng, orc, [synth.tokens(8, 1, cfg["vocab_size"])], 32, quant)


@pytest.mark.parametrize("name", ["toy", "toy10"])
@pytest.mark.parametrize("quant", ["bf16", "w4a16"])
def test_toy_int8_cache_greedy_parity(torch_dev, name, quant):
    """The int8 K/V cache (one fp32 scale per cached row): 8-token prompt, 32
    greedy steps across the 16-wide window, against the oracle with the same
    cache format.  W4A16 scales U(0.002, 0.0066), the E2B range: with the
    int8 cache the toy's U(0.002, 0.02) range turns a 1e-5 difference of a
    cached row into logit changes near the bound in the oracle itself
    (tests/test_workload_conditioning.py)."""
    torch, dev = torch_dev
    cfg = synth.get_config(name)
    w = synth.generate(cfg, quant, seed=0, scale_lo=0.002, scale_hi=0.0066)
    eng = _engine(cfg, quant, w, 1, 48, 8, kv_quant="int8")
    orc = oracle.Oracle(cfg, quant, w, 1, 48, kv_quant="int8")
    run_greedy(torch, eng, orc, [synth.tokens(8, 1, cfg["vocab_size"])], 32, quant)


@pytest.mark.parametrize("kv_quant", ["bf16", "int8"])
def test_toy_batched_ragged(torch_dev, kv_quant):
    """Four sequences at different positions in one batched step; a long
    context (max_ctx 2048: 64 attention chunks of 32 keys) with prefill split
    into several passes (max_rows 16); bf16 or int8 cache (W4A16 scales of
    the E2B range for the int8 cache, as in the int8 greedy test)."""
    torch, dev = torch_dev
    cfg = synth.get_config("toy10")
    sc = (0.002, 0.0066) if kv_quant == "int8" else (None, None)
    w = synth.generate(cfg, "w4a16", seed=3, scale_lo=sc[0], scale_hi=sc[1])
    eng = _engine(cfg, "w4a16", w, 4, 2048, 16, kv_quant=kv_quant)
    orc = oracle.Oracle(cfg, "w4a16", w, 4, 2048, kv_quant=kv_quant)
    prompts = [synth.tokens(n, 20 + n, cfg["vocab_size"]) for n in (8, 37, 1, 70)]
    run_greedy(torch, eng, orc, prompts, 12, "w4a16")


def test_wide_heads_long_window(torch_dev):
    """Head dims 256/512 with 8 query heads (the E2B attention shapes) at a
    small width, window 32, 100 positions."""
    torch, dev = torch_dev
    cfg = dict(synth.get_config("toy10"), name="wide", num_attention_heads=8, head_dim=256,
               global_head_dim=512, sliding_window=32)
    w = synth.generate(cfg, "bf16", seed=4)
    eng = _engine(cfg, "bf16", w, 2, 128, 64)
    orc = oracle.Oracle(cfg, "bf16", w, 2, 128)
    prompts = [synth.tokens(90, 5, cfg["vocab_size"]), synth.tokens(40, 6, cfg["vocab_size"])]
    run_greedy(torch, eng, orc, prompts, 8, "bf16")


@pytest.mark.parametrize("nq,kv_quant", [(8, "bf16"), (2, "bf16"), (4, "int8")])
def test_wide_heads_chunked_prefill(torch_dev, nq, kv_quant):
    """The matrix-core prefill attention (head dims 256/512, 16 queries of
    16 / nq rows per block) over many key chunks: a 700-token prompt in three
    prefill passes (300 rows at position 0, 257 at 300, 143 at 557: odd row
    counts leave a part-filled query tile), window 160 (two chunks per
    sliding-layer group), max_ctx 1024 (full layers over eight), then 6
    greedy steps; every pass's last-row logits and every step against the
    oracle."""
    torch, dev = torch_dev
    cfg = dict(synth.get_config("toy10"), name="wide", num_attention_heads=nq, head_dim=256,
               global_head_dim=512, sliding_window=160)
    w = synth.generate(cfg, "bf16", seed=11)
    V = cfg["vocab_size"]
    eng = _engine(cfg, "bf16", w, 1, 1024, 300, kv_quant=kv_quant)
    orc = oracle.Oracle(cfg, "bf16", w, 1, 1024, kv_quant=kv_quant)
    prompt = synth.tokens(700, 12, V)
    st = Stats("bf16")
    a1 = torch.zeros(1, dtype=torch.int32, device=dev)
    l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
    for p0, p1 in ((0, 300), (300, 557), (557, 700)):
        eng.prefill(0, torch.from_numpy(prompt[p0:p1]).to(dev), p0, a1, l1)
        eng.check()
        _, ref = orc.prefill(0, prompt[p0:p1], pos0=p0)
        st.add(l1.cpu().numpy()[0], int(a1.item()), ref, f"prefill {p0}..{p1 - 1}")
    nxt, pos = int(a1.item()), 700
    am = torch.zeros(1, dtype=torch.int32, device=dev)
    lg = torch.zeros(1, V, dtype=torch.float32, device=dev)
    for i in range(6):
        eng.decode_step(torch.tensor([nxt], dtype=torch.int32, device=dev),
                        torch.tensor([pos], dtype=torch.int32, device=dev), am, lg)
        eng.check()
        _, ref, _ = orc.step(0, nxt, pos)
        st.add(lg.cpu().numpy()[0], int(am.item()), ref, f"step {i} (position {pos})")
        nxt, pos = int(am.item()), pos + 1
    orc.close()
    st.finish(f"wide heads nq={nq} {kv_quant} cache, chunked prefill")


def test_batched_passes_agree_bitwise(torch_dev):
    """A row of a batched pass is computed independently of the other rows:
    a 20-token prefill (one batched pass) and the same tokens decoded as row 2
    of 3-row batches (the decode attention writes its own K/V) give the same
    cache bits and logits.  The one-row path (matvec kernel instead of the
    matrix cores) agrees with them to rounding."""
    torch, dev = torch_dev
    cfg = synth.get_config("toy10")
    w = synth.generate(cfg, "w4a16", seed=5)
    V = cfg["vocab_size"]
    p = synth.tokens(20, 9, V)
    eng = _engine(cfg, "w4a16", w, 3, 48, 32)
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    l_pre = torch.zeros(1, V, dtype=torch.float32, device=dev)
    eng.prefill(0, torch.from_numpy(p).to(dev), 0, a, l_pre)
    l_one = torch.zeros(1, V, dtype=torch.float32, device=dev)
    for i, t in enumerate(p):   # same tokens, one by one, into cache row 1
        eng.prefill(1, torch.tensor([t], dtype=torch.int32, device=dev), i, a, l_one)
    # decode path into cache row 2 (rows 0 and 1 decode at positions 20.. meanwhile)
    a3 = torch.zeros(3, dtype=torch.int32, device=dev)
    l_dec = torch.zeros(3, V, dtype=torch.float32, device=dev)
    for i, t in enumerate(p):
        tok = torch.tensor([t, t, t], dtype=torch.int32, device=dev)
        pos = torch.tensor([20 + i, 20 + i, i], dtype=torch.int32, device=dev)
        eng.decode_step(tok, pos, a3, l_dec)
    eng.check()
    assert torch.equal(l_pre[0], l_dec[2])
    ref = l_pre[0].double()
    err = float((l_one[0].double() - ref).abs().max() / ref.abs().max())
    assert err <= 1e-3, err
    for l in range(cfg["num_hidden_layers"]):
        hd = synth.layer_head_dim(cfg, l)
        for which in (0, 1):
            kv = eng.kv_tensor(l, which, hd)
            assert torch.equal(kv[0, :20], kv[2, :20])
            k0 = synth.bf16_to_f32(kv[0, :20].cpu().numpy().view(np.uint16)).astype(np.float64)
            k1 = synth.bf16_to_f32(kv[1, :20].cpu().numpy().view(np.uint16)).astype(np.float64)
            # one-row vs batched: bf16 rounding flips of the cached values
            assert np.max(np.abs(k1 - k0)) <= 2.0 ** -6 * np.max(np.abs(k0)) + 1e-3, (l, which)


def test_kv_sharing_and_cache_contents(torch_dev):
    """Shared layers read their source layer's region (same address, hence
    bit-identical K/V); the cached K/V match the oracle's to bf16 rounding."""
    torch, dev = torch_dev
    cfg = synth.get_config("toy10")
    w = synth.generate(cfg, "bf16", seed=6)
    eng = _engine(cfg, "bf16", w, 1, 32, 16)
    orc = oracle.Oracle(cfg, "bf16", w, 1, 32)
    p = synth.tokens(12, 2, cfg["vocab_size"])
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    eng.prefill(0, torch.from_numpy(p).to(dev), 0, a)
    eng.check()
    orc.prefill(0, p)
    smap = eng.model.kv_share_map()
    for l in range(cfg["num_hidden_layers"]):
        for which in (0, 1):
            assert eng.kv_view(l, which) == eng.kv_view(smap[l], which)
            assert orc.kv_source(l) == smap[l]
    # layer 0's K/V depend on the token alone: at most one bf16 ulp from the
    # oracle (the rounding sees fp32 vs fp64 inputs), almost always equal.
    # Later layers also carry the effect of such one-ulp differences at earlier
    # positions through attention, so they are held to a vector-relative bound.
    exact = total = 0
    for l in sorted(set(smap)):
        hd = synth.layer_head_dim(cfg, l)
        for which in (0, 1):
            got = synth.bf16_to_f32(eng.kv_tensor(l, which, hd)[0, :12].cpu().numpy().view(np.uint16))
            for pos in range(12):
                ref = orc.kv_row(l, which, 0, pos, hd)     # already bf16-valued
                if l == 0:
                    tol = 2.0 ** -7 * np.abs(ref) + 1e-5 * np.max(np.abs(ref))
                    exact += int(np.sum(got[pos] == ref))
                    total += hd
                else:
                    tol = 2.0 ** -7 * np.abs(ref) + 2e-3 * np.max(np.abs(ref))
                assert np.all(np.abs(got[pos] - ref) <= tol), (l, which, pos)
    assert exact >= 0.99 * total, (exact, total)


def test_int8_cache_contents(torch_dev):
    """The int8 cache holds, for every cached row, the codes and the scale the
    oracle's quantizer gives (decided in fp32 on both sides): layer 0's rows
    depend on the token alone, so their codes agree almost everywhere (a code
    may move by one where the kernel's row, carried at about 2^-17 relative,
    and the oracle's fp64 one round differently at a half step) and the
    scales to that precision."""
    torch, dev = torch_dev
    cfg = synth.get_config("toy10")
    w = synth.generate(cfg, "bf16", seed=6)
    eng = _engine(cfg, "bf16", w, 1, 32, 16, kv_quant="int8")
    orc = oracle.Oracle(cfg, "bf16", w, 1, 32, kv_quant="int8")
    p = synth.tokens(12, 2, cfg["vocab_size"])
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    eng.prefill(0, torch.from_numpy(p).to(dev), 0, a)
    eng.check()
    orc.prefill(0, p)
    hd = synth.layer_head_dim(cfg, 0)
    exact = total = 0
    for which in (0, 1):
        codes = eng.kv_tensor(0, which, hd)[0, :12].cpu().numpy().astype(np.int64)
        sc = eng.kv_scales(0, which)[0, :12].cpu().numpy().astype(np.float64)
        for pos in range(12):
            ref = orc.kv_row(0, which, 0, pos, hd)              # code * scale, exact in fp64
            rs = np.float32(np.max(np.abs(ref)) / 127.0)        # the oracle's scale (fp32 grid)
            assert abs(sc[pos] - rs) <= 1e-4 * rs, (which, pos, sc[pos], rs)
            rc = np.rint(ref / float(rs)).astype(np.int64)
            assert np.all(np.abs(codes[pos] - rc) <= 1), (which, pos)
            assert np.max(np.abs(codes[pos])) == 127
            exact += int(np.sum(codes[pos] == rc))
            total += hd
    assert exact >= 0.99 * total, (exact, total)


def _continuous_batching(torch, eng, orc, V, prompts, lengths, quant, label, drift=0.0):
    """Serve `prompts` (request i wants lengths[i] decode steps) through the
    paged cache with at most eng.max_batch live rows: admit a request when a
    slot and its pages are free (reserve, prefill into its slot), decode the
    live rows together, and on finishing release the slot's pages and move
    the last live slot into its place.  Every live row of every step is
    compared with the oracle's own run of that request (oracle sequence i)."""
    dev = eng.device
    st = Stats(quant, drift)
    pending = list(range(len(prompts)))
    live = []                      # per row: [request, next token, position, steps done]
    admitted_late = 0
    lg = torch.zeros(eng.max_batch, V, dtype=torch.float32, device=dev)
    steps = 0
    while pending or live:
        while pending and len(live) < eng.max_batch:
            i = pending[0]
            need = len(prompts[i]) + lengths[i]
            if eng.pages_free() < (need + 127) // 128:
                break
            pending.pop(0)
            slot = len(live)
            eng.reserve(slot, need)
            a = torch.zeros(1, dtype=torch.int32, device=dev)
            l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
            eng.prefill(slot, torch.from_numpy(prompts[i]).to(dev), 0, a, l1)
            eng.check()
            _, ref = orc.prefill(i, prompts[i])
            st.add(l1.cpu().numpy()[0], int(a.item()), ref, f"request {i} prefill (slot {slot})")
            live.append([i, int(a.item()), len(prompts[i]), 0])
            admitted_late += int(steps > 0)
        assert live, "no request fits the pool"
        B = len(live)
        tok = torch.tensor([r[1] for r in live], dtype=torch.int32, device=dev)
        pos = torch.tensor([r[2] for r in live], dtype=torch.int32, device=dev)
        am = torch.zeros(B, dtype=torch.int32, device=dev)
        eng.decode_step(tok, pos, am, lg)
        eng.check()
        got_l, got_t = lg[:B].cpu().numpy(), am.cpu().numpy()
        steps += 1
        for b, r in enumerate(live):
            _, ref, _ = orc.step(r[0], r[1], r[2])
            st.add(got_l[b], int(got_t[b]), ref, f"request {r[0]} step {r[3]} (row {b}, position {r[2]})")
            r[1], r[2], r[3] = int(got_t[b]), r[2] + 1, r[3] + 1
        for b in reversed(range(len(live))):          # retire, then compact
            i = live[b][0]
            if live[b][3] >= lengths[i]:
                eng.release(b)
                last = len(live) - 1
                if b != last:
                    eng.move(last, b)
                    live[b] = live[last]
                live.pop()
    assert eng.pages_free() == eng.n_pages
    assert admitted_late > 0      # requests joined a running batch
    st.finish(label)


@pytest.mark.parametrize("kv_quant", ["bf16", "int8"])
def test_toy_paged_continuous_batching(torch_dev, kv_quant):
    """Paged cache (128-position pages, a pool too small for every request at
    once), 8 requests of uneven prompt and output lengths through 4 slots;
    positions cross page boundaries."""
    torch, dev = torch_dev
    cfg = synth.get_config("toy10")
    w = synth.generate(cfg, "w4a16", seed=9, scale_lo=0.002, scale_hi=0.0066)
    V = cfg["vocab_size"]
    plen = [5, 140, 1, 120, 17, 64, 200, 9]
    olen = [20, 7, 33, 12, 3, 25, 10, 40]
    prompts = [synth.tokens(n, 60 + i, V) for i, n in enumerate(plen)]
    from w4a16_weight_streaming_amd import Engine
    eng_p = Engine(cfg, "w4a16", w, max_batch=4, max_ctx=256, max_rows=64, kv_quant=kv_quant, n_pages=7)
    orc = oracle.Oracle(cfg, "w4a16", w, len(prompts), 256, kv_quant=kv_quant)
    _continuous_batching(torch, eng_p, orc, V, prompts, olen, "w4a16", f"toy10 paged {kv_quant} cache")


def test_paged_position_without_page_is_flagged(torch_dev):
    """A decode row whose position lies past its slot's reserved pages is
    flagged on the device error word (its cache row goes to the pool's spare
    page, which no sequence owns), and a valid step afterwards passes."""
    torch, dev = torch_dev
    from w4a16_weight_streaming_amd import E2BError, Engine
    cfg = synth.get_config("toy")
    w = synth.generate(cfg, "bf16", seed=8)
    eng = Engine(cfg, "bf16", w, max_batch=2, max_ctx=256, max_rows=8, n_pages=4)
    eng.reserve(0, 100)                        # one page: positions 0..127
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    eng.prefill(0, torch.from_numpy(synth.tokens(8, 1, cfg["vocab_size"])).to(dev), 0, a)
    eng.check()
    eng.decode_step(a.clone(), torch.tensor([130], dtype=torch.int32, device=dev), a)
    with pytest.raises(E2BError) as e:
        eng.check()
    assert "reserved page" in str(e.value)
    eng.decode_step(a.clone(), torch.tensor([8], dtype=torch.int32, device=dev), a)
    eng.check()
    with pytest.raises(E2BError):
        eng.reserve(1, 5 * 128)                # more pages than are free
    assert eng.pages_free() == 3


def test_deterministic_replay(torch_dev):
    torch, dev = torch_dev
    cfg = synth.get_config("toy")
    w = synth.generate(cfg, "w4a16", seed=7)
    V = cfg["vocab_size"]
    outs = []
    for _ in range(2):
        eng = _engine(cfg, "w4a16", w, 2, 32, 8)
        a = torch.zeros(2, dtype=torch.int32, device=dev)
        lg = torch.zeros(2, V, dtype=torch.float32, device=dev)
        for b in range(2):
            eng.prefill(b, torch.from_numpy(synth.tokens(8, 30 + b, V)).to(dev), 0, a[b:b + 1])
        for i in range(6):
            eng.decode_step(a.clone(), torch.full((2,), 8 + i, dtype=torch.int32, device=dev), a, lg)
        eng.check()
        outs.append(lg.clone())
    assert torch.equal(outs[0], outs[1])


def test_device_error_word(torch_dev):
    """Out-of-range tokens and positions are flagged, not read or written."""
    torch, dev = torch_dev
    from w4a16_weight_streaming_amd import E2BError
    from w4a16_weight_streaming_amd.binding import E2B_EDEVICE
    cfg = synth.get_config("toy")
    w = synth.generate(cfg, "bf16", seed=8)
    eng = _engine(cfg, "bf16", w, 1, 16, 8)
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    ok_tok = torch.tensor([5], dtype=torch.int32, device=dev)
    eng.decode_step(torch.tensor([cfg["vocab_size"] + 3], dtype=torch.int32, device=dev),
                    torch.tensor([0], dtype=torch.int32, device=dev), a)
    with pytest.raises(E2BError) as e:
        eng.check()
    assert e.value.code == E2B_EDEVICE and "vocabulary" in str(e.value)
    eng.decode_step(ok_tok, torch.tensor([16], dtype=torch.int32, device=dev), a)
    with pytest.raises(E2BError) as e:
        eng.check()
    assert "position" in str(e.value)
    eng.decode_step(ok_tok, torch.tensor([0], dtype=torch.int32, device=dev), a)
    eng.check()   # cleared, and a valid step passes


# ---------------------------------------------------------------- E2B shape
E2B_PROMPT, E2B_STEPS, E2B_BATCH = 128, 512, 64
# the E2B workloads: bf16, W4A16 (bf16 vocabulary tables), and W4A16 with the
# vocabulary tables in int4 too (the int4 lm_head; shorter runs)
E2B_WORKLOADS = {"bf16": ("bf16", "bf16"), "w4a16": ("w4a16", "bf16"), "w4a16-emb4": ("w4a16", "w4a16")}


_E2B_WEIGHTS = {}


def e2b_weights(quant, embed_quant="bf16"):
    """Seed-0 E2B tensors, generated once per format for the whole module."""
    key = (quant, embed_quant)
    if key not in _E2B_WEIGHTS:
        progress(f"[e2b] generating seed-0 {quant} weights ({embed_quant} vocabulary tables)")
        _E2B_WEIGHTS[key] = synth.generate(synth.get_config("e2b"), quant, seed=0, embed_quant=embed_quant)
    return _E2B_WEIGHTS[key]


@pytest.fixture(scope="module", params=list(E2B_WORKLOADS))
def e2b_model(request):
    cfg = synth.get_config("e2b")
    quant, eq = E2B_WORKLOADS[request.param]
    return cfg, quant, e2b_weights(quant, eq)


@pytest.fixture(scope="module")
def e2b_engine(torch_dev, e2b_model):
    """One engine per weight format, shared by the E2B tests: 64 sequences of
    up to 128 + 512 positions, 128-row prefill passes."""
    cfg, quant, w = e2b_model
    eng = _engine(cfg, quant, w, E2B_BATCH, E2B_PROMPT + E2B_STEPS + 8, 128)
    yield eng
    del eng


def test_e2b_gathers_bit_exact(torch_dev, e2b_model, e2b_engine):
    """The embedding gathers of the step (a1, a2's table row) equal the table
    rows (widened bf16, or int4 decoded exactly) times sqrt(H) / sqrt(P)
    rounded once to fp32, bit for bit,
    for the first and last vocabulary rows and random ones; the oracle's fp64
    embedding agrees to within the fp32 rounding of the constant and the
    product."""
    torch, dev = torch_dev
    cfg, quant, w = e2b_model
    eng = e2b_engine
    V, H = cfg["vocab_size"], cfg["hidden_size"]
    LP = cfg["num_hidden_layers"] * cfg["hidden_size_per_layer_input"]
    toks = np.concatenate([[0, 1, V - 2, V - 1], synth.tokens(60, 11, V)]).astype(np.int32)
    h = torch.zeros(len(toks), H, dtype=torch.float32, device=dev)
    tp = torch.zeros(len(toks), LP, dtype=torch.float32, device=dev)
    eng.embed(torch.from_numpy(toks).to(dev), h, tp)
    eng.check()
    got_h, got_tp = h.cpu().numpy(), tp.cpu().numpy()
    def rows(name):   # the table rows as fp32: widened bf16, or decoded int4 (exact in fp32)
        if name in w:
            return synth.bf16_to_f32(w[name][toks])
        u = w[name + "_packed"][toks].view(np.uint32)
        codes = np.stack([(u >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], -1)
        codes = codes.reshape(len(toks), -1).astype(np.float32) - 8
        return codes * np.repeat(synth.bf16_to_f32(w[name + "_scale"][toks]), 32, axis=1)
    want_h = rows("model.embed_tokens.weight") * np.float32(np.sqrt(H))
    want_tp = rows("model.embed_tokens_per_layer.weight") * np.float32(np.sqrt(cfg["hidden_size_per_layer_input"]))
    assert want_h.dtype == np.float32 and want_tp.dtype == np.float32
    assert np.array_equal(got_h, want_h)
    assert np.array_equal(got_tp, want_tp)   # sqrt(256) = 16: exact, no rounding at all
    # the oracle's exact fp64 embedding: the fp32 constant sqrt(H) is off by at
    # most 2^-24 relative (half an ulp) and the product rounds once (half an
    # ulp), so the exact value lies within one ulp of the kernel's plus the
    # constant's share, 1.5 ulp
    orc = oracle.Oracle(cfg, quant, w, 1, 8)
    for r, t in enumerate(toks[:8]):
        e, _ = orc.inputs(int(t))
        ulp = np.spacing(np.abs(got_h[r]).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(e - got_h[r]) <= 1.5 * ulp), t
    orc.close()


def test_e2b_greedy_512_parity(torch_dev, e2b_model, e2b_engine):
    """The single-sequence workloads as written (bf16, W4A16): a 128-token
    random prompt through e2b_prefill (one 128-row matrix-core pass), then 512
    greedy steps by replaying the captured decode graph (the launch the bench
    times), KV length 129..640.  Every step's 262,144 logits against the
    teacher-forced oracle; greedy agreement >= 99% of the 513 choices."""
    torch, dev = torch_dev
    cfg, quant, w = e2b_model
    eng = e2b_engine
    V, P, S = cfg["vocab_size"], E2B_PROMPT, E2B_STEPS
    if eng.embed_quant == "w4a16":
        S = 64        # the int4-table variant: a shorter run
        quant_label = "w4a16 + int4 vocabulary tables"
    else:
        quant_label = quant
    prompt = synth.tokens(P, 1, V)
    progress(f"\n[e2b {quant_label} B=1] GPU: {P}-token prefill, {S} graph steps")
    s = torch.cuda.Stream(dev)
    gl = np.empty((S, V), np.float32)
    fed, gt = [], []
    with torch.cuda.stream(s):
        a = torch.zeros(1, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        eng.prefill(0, torch.from_numpy(prompt).to(dev), 0, a, l1)
        eng.check()
        pre_l, pre_t = l1.cpu().numpy()[0], int(a.item())
        tok, pos = a.clone(), torch.tensor([P], dtype=torch.int32, device=dev)
        lg = torch.zeros(1, V, dtype=torch.float32, device=dev)
        g = eng.capture(tok, pos, tok, lg, advance=True)
        for i in range(S):
            fed.append(int(tok.item()))
            g.replay()
            s.synchronize()
            gl[i] = lg.cpu().numpy()[0]
            gt.append(int(tok.item()))
        eng.check()
        assert int(pos.item()) == P + S
        g.close()
    orc = oracle.Oracle(cfg, quant, w, 1, P + S + 1)
    st = Stats(quant, E2B_BF16_DRIFT if quant == "bf16" else 0.0)
    _, ref = orc.prefill(0, prompt)
    st.add(pre_l, pre_t, ref, "prefill (last row)")
    for i in range(S):
        _, ref, _ = orc.step(0, fed[i], P + i)
        st.add(gl[i], gt[i], ref, f"step {i} (position {P + i})")
        if i % 64 == 63:
            progress(f"[e2b {quant_label} B=1] oracle at step {i + 1}/{S}: worst rel err {st.worst:.3e}, "
                     f"agree {st.agree}/{st.n}")
    orc.close()
    st.finish(f"e2b {quant_label} B=1, {P}-token prompt + {S} steps", min_agree=0.99)


def test_e2b_batch64_prefill_graph_parity(torch_dev, e2b_model, e2b_engine):
    """The batched workload: 64 sequences, each a 128-token random prompt
    (seed 1 + b) through its own e2b_prefill pass, then 16 greedy steps of the
    captured 64-row decode graph (the bench's launch); the first and last
    sequences against the teacher-forced oracle at the prefill and every
    step."""
    torch, dev = torch_dev
    cfg, quant, w = e2b_model
    eng = e2b_engine
    V, P, B, S = cfg["vocab_size"], E2B_PROMPT, E2B_BATCH, 16
    rows = [0, 63]
    if eng.embed_quant == "w4a16":   # the int4-table variant: a shorter run
        S, rows = 4, [63]
    prompts = [synth.tokens(P, 1 + b, V) for b in range(B)]
    s = torch.cuda.Stream(dev)
    pre = {}
    gl, gt, fed = np.empty((S, len(rows), V), np.float32), [], []
    with torch.cuda.stream(s):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        for b in range(B):
            eng.prefill(b, torch.from_numpy(prompts[b]).to(dev), 0, tok[b:b + 1], l1)
            if b in rows:
                pre[b] = l1.cpu().numpy()[0].copy()
        eng.check()
        pos = torch.full((B,), P, dtype=torch.int32, device=dev)
        lg = torch.zeros(B, V, dtype=torch.float32, device=dev)
        pre_t = tok.cpu().numpy().copy()
        g = eng.capture(tok, pos, tok, lg, advance=True)
        for i in range(S):
            fed.append(tok.cpu().numpy().copy())
            g.replay()
            s.synchronize()
            gl[i] = lg[rows].cpu().numpy()
            gt.append(tok.cpu().numpy().copy())
        eng.check()
        g.close()
    orc = oracle.Oracle(cfg, quant, w, len(rows), P + S + 1)
    st = Stats(quant, E2B_BF16_DRIFT if quant == "bf16" else 0.0)
    for j, b in enumerate(rows):
        _, ref = orc.prefill(j, prompts[b])
        st.add(pre[b], int(pre_t[b]), ref, f"prefill seq {b}")
        progress(f"[e2b {quant} B=64] oracle prefill of sequence {b} done")
    for i in range(S):
        for j, b in enumerate(rows):
            _, ref, _ = orc.step(j, int(fed[i][b]), P + i)
            st.add(gl[i, j], int(gt[i][b]), ref, f"step {i} seq {b}")
    orc.close()
    st.finish(f"e2b {quant} B=64, sequences {rows}")


def _seed_cache(torch, eng, cfg, T_of, orc=None, orc_rows=()):
    """Seeded synthetic K/V (bf16 N(0, 1), like normed keys and values) at
    positions 0 .. T_of[b]-1 of every sequence b, written into the GPU cache
    and, for the sequences in orc_rows (oracle sequence i = orc_rows[i]), into
    the oracle's.  Stands in for a long prefill; comes from the shared input
    generator, not from either implementation."""
    dev = eng.device
    smap = eng.model.kv_share_map()
    progress(f"[seeded caches] contexts {T_of}")
    for l in range(cfg["num_hidden_layers"]):
        if smap[l] != l:
            continue
        hd = synth.layer_head_dim(cfg, l)
        kt, vt = eng.kv_tensor(l, 0, hd), eng.kv_tensor(l, 1, hd)
        for b, T in enumerate(T_of):
            kb = synth.normal_bf16((T, hd), 500 + b, f"cache.k.{l}", 0.0, 1.0)
            vb = synth.normal_bf16((T, hd), 500 + b, f"cache.v.{l}", 0.0, 1.0)
            kt[b, :T] = torch.from_numpy(kb.view(np.int16)).to(dev)
            vt[b, :T] = torch.from_numpy(vb.view(np.int16)).to(dev)
            if orc is not None and b in orc_rows:
                orc.kv_load(l, orc_rows.index(b), 0, kb, vb)


def _graph_decode_vs_oracle(torch, eng, orc, cfg, quant, T_of, rows, steps, seed):
    """`steps` greedy steps of a captured decode graph (the launch the bench
    times) from positions T_of; the sampled rows' logits against the oracle,
    teacher-forced on the GPU's tokens."""
    dev = eng.device
    B, V = len(T_of), cfg["vocab_size"]
    st = Stats(quant)
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        tok = torch.from_numpy(synth.tokens(B, seed, V)).to(dev)
        pos = torch.tensor(T_of, dtype=torch.int32, device=dev)
        lg = torch.zeros(B, V, dtype=torch.float32, device=dev)
        g = eng.capture(tok, pos, tok, lg, advance=True)
        for i in range(steps):
            fed = tok.cpu().numpy().copy()
            g.replay()
            s.synchronize()
            eng.check()
            got_l, got_t = lg.cpu().numpy(), tok.cpu().numpy()
            for j, b in enumerate(rows):
                _, ref, _ = orc.step(j, int(fed[b]), T_of[b] + i)
                st.add(got_l[b], int(got_t[b]), ref, f"step {i} row {b} (position {T_of[b] + i})")
            progress(f"[{quant} B={B} seeded caches] step {i + 1}/{steps} checked")
        g.close()
    st.finish(f"{quant} B={B} from seeded caches")


def test_e2b_w4a16_int8_cache_parity(torch_dev):
    """E2B shape, W4A16 weights with the int8 K/V cache: a 64-token prompt
    through one 64-row prefill pass (K/V written by the prefill kernel), then
    48 greedy steps of the captured decode graph (K/V written by the attention
    kernel), every step's logits against the oracle with the same cache."""
    torch, dev = torch_dev
    cfg = synth.get_config("e2b")
    w = e2b_weights("w4a16")
    V, P, S = cfg["vocab_size"], 64, 48
    eng = _engine(cfg, "w4a16", w, 1, P + S + 8, 128, kv_quant="int8")
    prompt = synth.tokens(P, 1, V)
    s = torch.cuda.Stream(dev)
    gl, fed, gt = np.empty((S, V), np.float32), [], []
    with torch.cuda.stream(s):
        a = torch.zeros(1, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        eng.prefill(0, torch.from_numpy(prompt).to(dev), 0, a, l1)
        eng.check()
        pre_l, pre_t = l1.cpu().numpy()[0], int(a.item())
        tok, pos = a.clone(), torch.tensor([P], dtype=torch.int32, device=dev)
        lg = torch.zeros(1, V, dtype=torch.float32, device=dev)
        g = eng.capture(tok, pos, tok, lg, advance=True)
        for i in range(S):
            fed.append(int(tok.item()))
            g.replay()
            s.synchronize()
            gl[i] = lg.cpu().numpy()[0]
            gt.append(int(tok.item()))
        eng.check()
        g.close()
    orc = oracle.Oracle(cfg, "w4a16", w, 1, P + S + 1, kv_quant="int8")
    st = Stats("w4a16")
    _, ref = orc.prefill(0, prompt)
    st.add(pre_l, pre_t, ref, "prefill (last row)")
    for i in range(S):
        _, ref, _ = orc.step(0, fed[i], P + i)
        st.add(gl[i], gt[i], ref, f"step {i} (position {P + i})")
    orc.close()
    st.finish(f"e2b w4a16 int8 cache B=1, {P}-token prompt + {S} steps", min_agree=0.99)


def test_e2b_w4a16_int8_cache_batched_parity(torch_dev):
    """The int8 K/V cache under batched decode at full size: 4 sequences of
    uneven prompts (40, 64, 17, 90 tokens) prefilled into their slots, then 12
    steps of the captured 4-row decode graph (each row's attention split over
    chunks and merged by the combine kernel, each row writing its own int8 K/V
    row); rows 0 and 3 against the oracle with the same cache."""
    torch, dev = torch_dev
    cfg = synth.get_config("e2b")
    w = e2b_weights("w4a16")
    V, S = cfg["vocab_size"], 12
    lens = [40, 64, 17, 90]
    rows = [0, 3]
    B = len(lens)
    eng = _engine(cfg, "w4a16", w, B, max(lens) + S + 8, 128, kv_quant="int8")
    prompts = [synth.tokens(n, 40 + b, V) for b, n in enumerate(lens)]
    s = torch.cuda.Stream(dev)
    pre, gl, gt, fed = {}, np.empty((S, len(rows), V), np.float32), [], []
    with torch.cuda.stream(s):
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        for b in range(B):
            eng.prefill(b, torch.from_numpy(prompts[b]).to(dev), 0, tok[b:b + 1], l1)
            if b in rows:
                pre[b] = l1.cpu().numpy()[0].copy()
        eng.check()
        pre_t = tok.cpu().numpy().copy()
        pos = torch.tensor(lens, dtype=torch.int32, device=dev)
        lg = torch.zeros(B, V, dtype=torch.float32, device=dev)
        g = eng.capture(tok, pos, tok, lg, advance=True)
        for i in range(S):
            fed.append(tok.cpu().numpy().copy())
            g.replay()
            s.synchronize()
            gl[i] = lg[rows].cpu().numpy()
            gt.append(tok.cpu().numpy().copy())
        eng.check()
        g.close()
    orc = oracle.Oracle(cfg, "w4a16", w, len(rows), max(lens) + S + 1, kv_quant="int8")
    st = Stats("w4a16")
    for j, b in enumerate(rows):
        _, ref = orc.prefill(j, prompts[b])
        st.add(pre[b], int(pre_t[b]), ref, f"prefill seq {b}")
        progress(f"[e2b w4a16 int8 cache B={B}] oracle prefill of sequence {b} done")
    for i in range(S):
        for j, b in enumerate(rows):
            _, ref, _ = orc.step(j, int(fed[i][b]), lens[b] + i)
            st.add(gl[i, j], int(gt[i][b]), ref, f"step {i} seq {b} (position {lens[b] + i})")
    orc.close()
    st.finish(f"e2b w4a16 int8 cache B={B}, sequences {rows}")


def test_e2b_paged_continuous_batching(torch_dev):
    """Full E2B shape (bf16 weights: the paging is the same for both formats
    and the bf16 oracle is the faster), paged cache: 5 requests (prompts 150,
    40, 1, 130 and 20 tokens, 3-10 decode steps) through 3 slots; head dims
    256/512 over positions that cross the 128-position page boundary."""
    torch, dev = torch_dev
    from w4a16_weight_streaming_amd import Engine
    cfg = synth.get_config("e2b")
    w = e2b_weights("bf16")
    V = cfg["vocab_size"]
    plen, olen = [150, 40, 1, 130, 20], [6, 10, 8, 3, 5]
    prompts = [synth.tokens(n, 80 + i, V) for i, n in enumerate(plen)]
    eng = Engine(cfg, "bf16", w, max_batch=3, max_ctx=512, max_rows=128, n_pages=5)
    orc = oracle.Oracle(cfg, "bf16", w, len(prompts), 512)
    _continuous_batching(torch, eng, orc, V, prompts, olen, "bf16", "e2b bf16 paged", E2B_BF16_DRIFT)


@pytest.mark.parametrize("B", [1, 8])
def test_e2b_long_context_graph_parity(torch_dev, B):
    """Long context at full size (W4A16): contexts near 8,000 (seeded
    caches), 2 steps of the captured graph, first and last rows against the
    oracle -- full-layer attention over ~8,000 keys, sliding layers over 512."""
    torch, dev = torch_dev
    cfg = synth.get_config("e2b")
    w = e2b_weights("w4a16")
    T_of = [8000 - 123 * b for b in range(B)]
    rows = sorted({0, B - 1})
    eng = _engine(cfg, "w4a16", w, B, 8064, 64)
    orc = oracle.Oracle(cfg, "w4a16", w, len(rows), 8064)
    _seed_cache(torch, eng, cfg, T_of, orc, rows)
    _graph_decode_vs_oracle(torch, eng, orc, cfg, "w4a16", T_of, rows, 2, 78)


def test_e2b_chunk_prefill_at_long_context(torch_dev):
    """A prefill pass deep into a long context at full size (W4A16): seeded
    caches up to position 3000, then 97 tokens in one pass at 3000..3096
    (full layers: ~3,100 keys over 25 chunks per query tile, sliding layers
    over 512 plus the tile), the pass's last-row logits and 2 graph steps
    after it against the oracle."""
    torch, dev = torch_dev
    cfg = synth.get_config("e2b")
    w = e2b_weights("w4a16")
    V, T0, P = cfg["vocab_size"], 3000, 97
    eng = _engine(cfg, "w4a16", w, 1, 3200, 128)
    orc = oracle.Oracle(cfg, "w4a16", w, 1, 3200)
    _seed_cache(torch, eng, cfg, [T0], orc, [0])
    prompt = synth.tokens(P, 31, V)
    st = Stats("w4a16")
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        a1 = torch.zeros(1, dtype=torch.int32, device=dev)
        l1 = torch.zeros(1, V, dtype=torch.float32, device=dev)
        eng.prefill(0, torch.from_numpy(prompt).to(dev), T0, a1, l1)
        s.synchronize()
        eng.check()
    _, ref = orc.prefill(0, prompt, pos0=T0)
    st.add(l1.cpu().numpy()[0], int(a1.item()), ref, f"prefill {T0}..{T0 + P - 1}")
    st.finish(f"w4a16 prefill pass at context {T0}")
    _graph_decode_vs_oracle(torch, eng, orc, cfg, "w4a16", [T0 + P], [0], 2, 79)
    orc.close()
