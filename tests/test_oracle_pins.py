"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong nibble order or window edge)
fails at least one of them.  CPU only.
"""
import math

import numpy as np
import pytest

import golden
import oracle
import synth
from oracle.naive import Naive


def bf16(vals):
    return synth.f32_to_bf16(np.asarray(vals, np.float32))


# ---------------------------------------------------------------- W4A16 unpack
def test_nibble_order_fixture():
    """Known words decode to the printed codes, in natural K order."""
    words, q = golden.nibble_case()
    K = 32
    w = words.reshape(1, K // 8)
    for s in (1.0, 0.25, 0.0078125):
        scale = bf16([s])
        got = [oracle.decode_weight("w4a16", w, scale, 1, K, 0, k) for k in range(K)]
        assert np.array_equal(np.array(got), q * s)
        y = oracle.linear("w4a16", w, scale, 1, K, np.ones(K))
        assert y[0] == q.sum() * s


def test_unpack_is_exact_in_fp32():
    """Every level -8..7 times every bf16 scale in [0.002, 0.02] is exact in
    fp32 (4 + 8 significant bits), so an fp32 kernel can reproduce the oracle's
    decoded weights bit for bit ("... Colab TPU", cell 3.1: the repack's values
    are bit-for-bit the trained ones)."""
    lo, hi = synth.f32_to_bf16(np.float32([0.002, 0.02]))
    scales = synth.bf16_to_f32(np.arange(lo, hi + 1, dtype=np.uint16)).astype(np.float64)
    q = np.arange(-8, 8, dtype=np.float64)
    prod = q[:, None] * scales[None, :]
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)


def test_one_hot_extracts_columns_with_their_group_scale():
    """x = e_k returns column k exactly; columns 31 and 32 read different scales."""
    rng = np.random.default_rng(0)
    N, K = 3, 64
    codes = rng.integers(0, 16, size=(N, K))
    words = np.zeros((N, K // 8), np.uint32)
    for k in range(K):     # pack by the fixture's rule: element 8j+i in bits [4i, 4i+4)
        words[:, k // 8] |= (codes[:, k].astype(np.uint32) << np.uint32(4 * (k % 8)))
    scales = bf16([[0.5, 0.125]] * N)
    for k in (0, 7, 8, 31, 32, 63):
        x = np.zeros(K)
        x[k] = 1.0
        y = oracle.linear("w4a16", words.view(np.int32), scales, N, K, x)
        s = 0.5 if k < 32 else 0.125
        assert np.array_equal(y, (codes[:, k] - 8) * s)


def test_bf16_linear_is_widening():
    w = bf16([[1.5, -2.0, 0.333], [0.0, 3.0, -1.0]])
    y = oracle.linear("bf16", w, None, 2, 3, [1.0, 10.0, 100.0])
    wf = synth.bf16_to_f32(w).astype(np.float64)
    assert np.array_equal(y, wf @ np.array([1.0, 10.0, 100.0]))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (1.0, -3.0, 1e-3):
        y = oracle.rmsnorm(np.full(16, c), eps=eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    x = np.array([3.0, 4.0])                   # mean square 12.5
    assert np.allclose(oracle.rmsnorm(x, eps=0.0), x / math.sqrt(12.5), rtol=1e-15)
    g = bf16([2.0, -0.5])
    assert np.allclose(oracle.rmsnorm(x, g, eps=0.0), x / math.sqrt(12.5) * [2.0, -0.5], rtol=1e-15)
    assert np.array_equal(oracle.rmsnorm(np.zeros(8)), np.zeros(8))   # eps keeps 0 -> 0


# ---------------------------------------------------------------- GELU (tanh)
def test_gelu_tanh():
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(1.0) == pytest.approx(0.8411919906082768, abs=1e-15)
    for x in np.linspace(-6, 6, 121):
        g, gm = oracle.gelu_tanh(x), oracle.gelu_tanh(-x)
        assert g - gm == pytest.approx(x, abs=1e-12)           # x Phi(x) - (-x)Phi(-x) = x
        erf_form = 0.5 * x * (1 + math.erf(x / math.sqrt(2)))
        assert abs(g - erf_form) < 5e-4                         # tanh form tracks the erf form
    assert oracle.gelu_tanh(20.0) == pytest.approx(20.0)
    assert oracle.gelu_tanh(-20.0) == pytest.approx(0.0, abs=1e-12)


# ---------------------------------------------------------------- RoPE
def test_rope_rotate_half():
    hd, half = 8, 4
    assert np.array_equal(oracle.rope(np.arange(hd, dtype=float), 0, 1e4), np.arange(hd))
    for p in (1, 7, 100):
        e0 = np.zeros(hd); e0[0] = 1.0
        y = oracle.rope(e0, p, 1e4)             # frequency theta^0 = 1
        assert y[0] == pytest.approx(math.cos(p)) and y[half] == pytest.approx(math.sin(p))
        eh = np.zeros(hd); eh[half] = 1.0
        y = oracle.rope(eh, p, 1e4)
        assert y[0] == pytest.approx(-math.sin(p)) and y[half] == pytest.approx(math.cos(p))
        e1 = np.zeros(hd); e1[1] = 1.0
        y = oracle.rope(e1, p, 1e4)              # second pair turns at theta^(-2/hd)
        ang = p * 1e4 ** (-2 / hd)
        assert y[1] == pytest.approx(math.cos(ang)) and y[1 + half] == pytest.approx(math.sin(ang))
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=hd), rng.normal(size=hd)
    a = oracle.rope(q, 5, 1e6) @ oracle.rope(k, 3, 1e6)
    b = oracle.rope(q, 1005, 1e6) @ oracle.rope(k, 1003, 1e6)
    assert a == pytest.approx(b, rel=1e-9)       # depends on relative position only
    assert np.linalg.norm(oracle.rope(q, 123, 1e4)) == pytest.approx(np.linalg.norm(q))


# ---------------------------------------------------------------- attention
def test_attend_special_cases():
    rng = np.random.default_rng(2)
    hd, T = 16, 6
    K, V = rng.normal(size=(T, hd)), rng.normal(size=(T, hd))
    q = rng.normal(size=hd)
    assert np.allclose(oracle.attend(q, K, V, 3, 3), V[3])            # one key -> its value
    assert np.allclose(oracle.attend(np.zeros(hd), K, V, 1, 4), V[1:5].mean(0))  # flat scores
    Kd = np.zeros((T, hd)); Kd[2] = 1000 * q / np.linalg.norm(q)
    assert np.allclose(oracle.attend(q, Kd, V, 0, 5), V[2])           # one dominant key
    # scale 1/sqrt(hd): two keys whose scores differ by sqrt(hd) * ln 3 weigh 3:1
    K2 = np.zeros((2, hd)); K2[0, 0] = math.log(3) * math.sqrt(hd)
    e = np.zeros(hd); e[0] = 1.0
    o = oracle.attend(e, K2, np.array([[1.0] + [0] * (hd - 1), [0.0] * hd]), 0, 1)
    assert o[0] == pytest.approx(0.75)


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    rng = np.random.default_rng(3)
    x = rng.normal(size=1000)
    assert oracle.argmax(x) == int(np.argmax(x))


# ---------------------------------------------------------------- layer map and sharing
def _small(name, quant="bf16", **over):
    cfg = synth.get_config(name)
    cfg.update(over)
    return cfg, synth.generate(cfg, quant)


def test_kv_map_e2b_matches_pages():
    cfg = synth.get_config("e2b")
    # the map only depends on the config; build with a tiny vocabulary/width copy
    small = dict(cfg, hidden_size=32, hidden_size_per_layer_input=8, vocab_size=16,
                 intermediate_size=32, head_dim=8, global_head_dim=16, num_attention_heads=1)
    w = synth.generate(small, "bf16")
    o = oracle.Oracle(small, "bf16", w, 1, 4)
    assert [o.kv_source(l) for l in range(35)] == golden.kv_share_map_e2b()


def test_kv_map_toys():
    for name, want in (("toy", [0, 1, 2, 2, 4]), ("toy10", [0, 1, 2, 3, 4, 3, 3, 3, 3, 4])):
        cfg, w = _small(name)
        o = oracle.Oracle(cfg, "bf16", w, 1, 4)
        assert [o.kv_source(l) for l in range(cfg["num_hidden_layers"])] == want


def test_shared_layers_read_their_source_kv():
    cfg, w = _small("toy10")
    o = oracle.Oracle(cfg, "bf16", w, 1, 32)
    for p, t in enumerate(synth.tokens(20, 5, cfg["vocab_size"])):
        o.step(0, t, p, logits=False)
    for l in range(5, 10):
        src = o.kv_source(l)
        hd = synth.layer_head_dim(cfg, l)
        for p in (0, 7, 19):
            for which in (0, 1):
                assert np.array_equal(o.kv_row(l, which, 0, p, hd), o.kv_row(src, which, 0, p, hd))


def test_bf16_cache_rounds_stored_kv():
    """With the bf16 cache, stored K/V are bf16 values: the nearest-even bf16 of
    what the fp64 cache stores for the same inputs (layer 0, position 0)."""
    cfg, w = _small("toy", "bf16")
    a = oracle.Oracle(cfg, "bf16", w, 1, 8, kv_bf16=False)
    b = oracle.Oracle(cfg, "bf16", w, 1, 8, kv_bf16=True)
    for o in (a, b):
        for p, t in enumerate((5, 9, 11)):
            o.step(0, t, p, logits=False)
    hd = synth.layer_head_dim(cfg, 0)
    for which in (0, 1):
        full = a.kv_row(0, which, 0, 0, hd)
        rounded = b.kv_row(0, which, 0, 0, hd)
        assert not np.array_equal(full, rounded)
        assert np.array_equal(rounded, synth.bf16_to_f32(synth.f32_to_bf16(full.astype(np.float32))))
        for p in range(3):
            r = b.kv_row(2, which, 0, p, hd)
            assert np.array_equal(r, synth.bf16_to_f32(synth.f32_to_bf16(r.astype(np.float32))))


def test_sliding_equals_full_within_window():
    toks = synth.tokens(16, 9, 4096)
    cfg_w, w = _small("toy10", "w4a16")
    cfg_f = dict(cfg_w, sliding_window=1 << 20)
    a = oracle.Oracle(cfg_w, "w4a16", w, 1, 32)
    b = oracle.Oracle(cfg_f, "w4a16", w, 1, 32)
    for p, t in enumerate(toks):                   # T <= W = 16: identical, bit for bit
        assert np.array_equal(a.step(0, t, p)[1], b.step(0, t, p)[1])
    ra, rb = a.step(0, 3, 16)[1], b.step(0, 3, 16)[1]
    assert not np.array_equal(ra, rb)               # T = 17 > W: the window bites


# ---------------------------------------------------------------- per-layer inputs
def test_per_layer_inputs_closed_forms():
    cfg, w = _small("toy")
    L, P, H = cfg["num_hidden_layers"], cfg["hidden_size_per_layer_input"], cfg["hidden_size"]
    x = 17
    # zero projection: pli = E_ple[x] * sqrt(P) * 2^-1/2
    w0 = dict(w)
    w0["model.per_layer_model_projection.weight"] = np.zeros((L * P, H), np.uint16)
    e, pli = oracle.Oracle(cfg, "bf16", w0, 1, 4).inputs(x)
    row = synth.bf16_to_f32(w["model.embed_tokens_per_layer.weight"][x]).astype(np.float64)
    assert np.allclose(pli.ravel(), row * math.sqrt(P) * math.sqrt(0.5), rtol=1e-15)
    assert np.allclose(e, synth.bf16_to_f32(w["model.embed_tokens.weight"][x]) * math.sqrt(H),
                       rtol=1e-15)
    # zero token table, projection = constant per slice: pli = sign * gain * 2^-1/2
    w1 = dict(w)
    w1["model.embed_tokens_per_layer.weight"] = np.zeros_like(w["model.embed_tokens_per_layer.weight"])
    emb = synth.bf16_to_f32(w["model.embed_tokens.weight"][x]).astype(np.float64)
    proj = np.zeros((L * P, H), np.float32)
    proj[:, 0] = 1.0
    w1["model.per_layer_model_projection.weight"] = bf16(proj)
    g = synth.bf16_to_f32(w["model.per_layer_projection_norm.weight"]).astype(np.float64)
    _, pli = oracle.Oracle(cfg, "bf16", w1, 1, 4).inputs(x)
    c = emb[0] * math.sqrt(H) * H ** -0.5          # every projected entry equals c
    want = np.sign(c) * abs(c) / math.sqrt(c * c + cfg["rms_eps"]) * g * math.sqrt(0.5)
    assert np.allclose(pli, np.broadcast_to(want, (L, P)), rtol=1e-12)


# ---------------------------------------------------------------- cached vs brute force
@pytest.mark.parametrize("name", ["toy", "toy10"])
@pytest.mark.parametrize("quant,embed_quant", [("bf16", "bf16"), ("w4a16", "bf16"), ("w4a16", "w4a16")])
@pytest.mark.parametrize("kv_bf16", [True, False])
def test_cached_oracle_matches_bruteforce(name, quant, embed_quant, kv_bf16):
    """Cached decode == re-running the whole sequence (tolerance: fp64 roundoff),
    across the sliding-window edge (sequence 26 > window 16), with the cache
    in bf16 and in fp64, and with the vocabulary tables in bf16 or int4."""
    cfg = synth.get_config(name)
    w = synth.generate(cfg, quant, embed_quant=embed_quant)
    o = oracle.Oracle(cfg, quant, w, 2, 40, kv_bf16=kv_bf16)
    nv = Naive(cfg, quant, w, kv_bf16=kv_bf16)
    toks = list(synth.tokens(26, 11, cfg["vocab_size"]))
    ref = nv.forward(toks)
    for p, t in enumerate(toks):
        r, lg, _ = o.step(1, t, p)
        assert np.max(np.abs(lg - ref[p])) < 1e-11 * max(1.0, np.abs(ref[p]).max())
        assert r == int(np.argmax(ref[p]))


def _unpack_codes(packed):
    """int4 codes of packed words, natural order (element 8j+i in bits 4i..4i+3)."""
    u = packed.view(np.uint32)
    return np.stack([(u >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], axis=-1).reshape(
        u.shape[0], u.shape[1] * 8).astype(np.int64)


@pytest.mark.parametrize("name", ["toy", "toy10"])
def test_int4_vocabulary_tables_reduce_to_bf16_tables(name):
    """Special case: with power-of-two group scales every decoded value
    (c - 8) * 2^-e has at most four significant bits, so it is a bf16 number.
    A model whose two vocabulary tables are int4 must then give exactly the
    logits of the same model with those values stored as bf16 tables: the
    embedding gather, the per-layer table gather and the tied lm_head all read
    the int4 tables ("Six Serving Engines on One Cloud TPU v5e Chip", What
    Changes and What Stays: the vocabulary tables in int4; Step 3: an int4
    lm_head).  A wrong nibble order or scale index breaks the equality."""
    cfg = synth.get_config(name)
    w4 = synth.generate(cfg, "w4a16", seed=5, embed_quant="w4a16")
    rng = np.random.default_rng(0)
    wb = {k: v for k, v in w4.items() if not k.startswith("model.embed_tokens")}
    for t in ("model.embed_tokens.weight", "model.embed_tokens_per_layer.weight"):
        sc = w4[t + "_scale"]
        pw = rng.integers(-9, -5, size=sc.shape)                      # scales 2^-9 .. 2^-6
        w4[t + "_scale"] = synth.f32_to_bf16(np.ldexp(np.ones(sc.shape, np.float32), pw))
        vals = (_unpack_codes(w4[t + "_packed"]) - 8) * np.repeat(np.ldexp(1.0, pw), 32, axis=1)
        bits = synth.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(synth.bf16_to_f32(bits).astype(np.float64), vals)   # exact in bf16
        wb[t] = bits
    toks = synth.tokens(10, 3, cfg["vocab_size"])
    o4 = oracle.Oracle(cfg, "w4a16", w4, 1, 16)
    ob = oracle.Oracle(cfg, "w4a16", wb, 1, 16)
    assert o4.embed_quant == "w4a16" and ob.embed_quant == "bf16"
    for p, t in enumerate(toks):
        r4, l4, _ = o4.step(0, int(t), p)
        rb, lb, _ = ob.step(0, int(t), p)
        assert np.array_equal(l4, lb) and r4 == rb, p


def test_int8_cache_rows_are_symmetric_absmax_quantization():
    """The int8 cache's row quantizer ("One TPU chip, eight agents": int8 KV,
    one byte per element): the scale is max |x| / 127 (fp32), the extreme
    element lands on +-127, every element is within half a step of its code
    times the scale, signs are kept, and a row of zeros gives scale 0."""
    rng = np.random.default_rng(3)
    rows = [rng.normal(size=256), rng.normal(size=512) * 1e-3, -np.abs(rng.normal(size=64)),
            np.eye(1, 128, 5)[0] * 7.0, np.linspace(-1, 1, 256)]
    for x in rows:
        q, sc = oracle.quant_int8(x)
        xf = x.astype(np.float32)
        amax = np.float32(np.max(np.abs(xf)))
        assert np.float32(sc) == amax / np.float32(127)
        assert np.all(np.abs(q.astype(np.int64)) <= 127)
        assert abs(int(q[np.argmax(np.abs(xf))])) == 127
        err = np.abs(xf.astype(np.float64) - q.astype(np.float64) * sc)
        assert np.all(err <= 0.5 * sc * (1 + 2.0 ** -20)), np.max(err / sc)
        big = np.abs(xf) >= 0.5 * sc
        assert np.all(np.sign(q[big]) == np.sign(xf[big]))
    q, sc = oracle.quant_int8(np.zeros(64))
    assert sc == 0.0 and not np.any(q)


@pytest.mark.parametrize("name", ["toy", "toy10"])
@pytest.mark.parametrize("quant", ["bf16", "w4a16"])
def test_int8_cache_oracle_matches_bruteforce(name, quant):
    """Cached decode with the int8 cache == re-running the whole sequence with
    every key and value row quantized the same way (numpy), across the
    sliding-window edge."""
    cfg, w = _small(name, quant)
    o = oracle.Oracle(cfg, quant, w, 1, 40, kv_quant="int8")
    nv = Naive(cfg, quant, w, kv_quant="int8")
    toks = list(synth.tokens(26, 12, cfg["vocab_size"]))
    ref = nv.forward(toks)
    for p, t in enumerate(toks):
        r, lg, _ = o.step(0, t, p)
        assert np.max(np.abs(lg - ref[p])) < 1e-11 * max(1.0, np.abs(ref[p]).max())
        assert r == int(np.argmax(ref[p]))
    # and it is a different cache than bf16: the logits move
    ob = oracle.Oracle(cfg, quant, w, 1, 40)
    lb = [ob.step(0, t, p)[1] for p, t in enumerate(toks)]
    assert max(np.max(np.abs(lb[p] - ref[p])) for p in range(len(toks))) > 1e-6


def test_greedy_prefill_then_decode_matches_bruteforce():
    cfg, w = _small("toy", "w4a16")
    prompt = list(synth.tokens(8, 1, cfg["vocab_size"]))
    nv = Naive(cfg, "w4a16", w)
    ref_toks, _ = nv.greedy(prompt, 12)
    o = oracle.Oracle(cfg, "w4a16", w, 1, 40)
    t, _ = o.prefill(0, prompt)
    got = [t]
    for i in range(11):
        t, _, _ = o.step(0, t, len(prompt) + i)
        got.append(t)
    assert got == ref_toks


# ---------------------------------------------------------------- inventory (shape reading)
def _bytes(cfg, quant):
    tot, nlin = 0, 0
    for s in synth.tensor_specs(cfg, kv_all_layers=False):
        n = int(np.prod(s.shape))
        if s.kind == "linear" and quant == "w4a16":
            tot += n // 2 + 2 * (n // cfg["group_size"])
        else:
            tot += 2 * n
        nlin += s.kind == "linear"
    return tot, nlin


def test_e2b_inventory_matches_page_totals():
    """hidden 1536 and 8 query heads are not printed on the pages; the printed
    byte totals pin them (each query head moves the bf16 total by ~66 MB)."""
    g = golden.kv("weight_bytes.txt")
    cfg = synth.get_config("e2b")
    b16, nlin = _bytes(cfg, "bf16")
    w4, _ = _bytes(cfg, "w4a16")
    assert abs(b16 - int(g["bf16_total"])) / int(g["bf16_total"]) < 1e-4
    assert round(w4 / 1e9, 3) == float(g["w4a16_total_gb"])
    assert nlin == int(g["quantized_linears"])
    assert round(2 * cfg["vocab_size"] * cfg["hidden_size"] / 1e9, 3) == float(g["embed_gb"])
    ple = 2 * cfg["vocab_size"] * cfg["num_hidden_layers"] * cfg["hidden_size_per_layer_input"]
    assert round(ple / 1e9, 2) == float(g["ple_table_gb"])
    assert len(synth.tensor_specs(cfg, kv_all_layers=True)) == int(g["parameters_all_kv"])
    for nq in (7, 9):
        other, _ = _bytes(dict(cfg, num_attention_heads=nq), "bf16")
        assert abs(other - int(g["bf16_total"])) / int(g["bf16_total"]) > 5e-3


def test_kv_load_places_rows_where_prefill_does():
    """kv_load stores bf16 rows at (layer, sequence, position): an oracle whose
    cache is loaded with another oracle's prefill cache (sequence 1 into
    sequence 0) decodes the next token bit-identically; a layer that reads
    shared K/V refuses a load."""
    cfg = synth.get_config("toy10")
    V = cfg["vocab_size"]
    w = synth.generate(cfg, "bf16", seed=3)
    a = oracle.Oracle(cfg, "bf16", w, 2, 24)
    b = oracle.Oracle(cfg, "bf16", w, 2, 24)
    toks = synth.tokens(10, 4, V)
    a.prefill(1, toks)
    owners = [l for l in range(cfg["num_hidden_layers"]) if a.kv_source(l) == l]
    for l in owners:
        hd = synth.layer_head_dim(cfg, l)
        k = np.stack([a.kv_row(l, 0, 1, p, hd) for p in range(10)]).astype(np.float32)
        v = np.stack([a.kv_row(l, 1, 1, p, hd) for p in range(10)]).astype(np.float32)
        b.kv_load(l, 0, 0, synth.f32_to_bf16(k), synth.f32_to_bf16(v))
    ta, la, _ = a.step(1, 17, 10)
    tb, lb, _ = b.step(0, 17, 10)
    assert ta == tb and np.array_equal(la, lb)
    shared = [l for l in range(cfg["num_hidden_layers"]) if a.kv_source(l) != l][0]
    with pytest.raises(RuntimeError):
        b.kv_load(shared, 0, 0, np.zeros((1, 64), np.uint16), np.zeros((1, 64), np.uint16))
