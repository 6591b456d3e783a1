"""Conditioning of the E2B W4A16 workload (CPU, the oracle alone).

The cache the pages describe holds K/V in bf16 ("Gemma 4 E2B in JAX on One
TPU v5e", Step 2; "One TPU chip, eight agents", KV memory math).  Any
implementation that computes a key in another precision than the oracle may
round one cached element to the neighbouring bf16 value.  Whether a logit
bound of 3e-2 of max |logit| can hold at all then depends on how far one such
one-ulp difference carries through 35 random layers.

This pins the reading that the E2B W4A16 workload draws its group scales from
U(0.002, 0.0066) (dequantized weights with rms 0.02, like the bf16 workload's
N(0, 0.02)) and not from U(0.002, 0.02) (rms 0.068): with the wider scales the
oracle's own logits leave the bound within a few steps when a single cached
key element moves by one bf16 ulp, so no implementation could be held to it;
with the narrower scales the same change stays four orders of magnitude
inside it.
"""
import numpy as np
import pytest

import oracle
import synth

PROMPT, STEPS = 4, 6


def _logit_drift(scale_lo, scale_hi):
    """Max over STEPS teacher-forced steps of max |logit difference| / max
    |logit| between an unperturbed run and one where element 0 of layer 0's
    cached key at position 0 is moved up by one bf16 ulp after the prompt."""
    cfg = synth.get_config("e2b")
    w = synth.generate(cfg, "w4a16", seed=0, scale_lo=scale_lo, scale_hi=scale_hi)
    toks = synth.tokens(PROMPT + STEPS, 1, cfg["vocab_size"])
    hd = synth.layer_head_dim(cfg, 0)
    runs = []
    for perturb in (False, True):
        orc = oracle.Oracle(cfg, "w4a16", w, 1, PROMPT + STEPS + 1)
        orc.prefill(0, toks[:PROMPT], logits=False)
        if perturb:
            # the cache holds bf16 values: widen to fp32, take the bits, step one ulp
            k = synth.f32_to_bf16(orc.kv_row(0, 0, 0, 0, hd).astype(np.float32))
            v = synth.f32_to_bf16(orc.kv_row(0, 1, 0, 0, hd).astype(np.float32))
            k[0] += 1
            orc.kv_load(0, 0, 0, k[None], v[None])
        lg = [orc.step(0, int(toks[PROMPT + i]), PROMPT + i)[1] for i in range(STEPS)]
        orc.close()
        runs.append(np.array(lg))
    del w
    base, pert = runs
    return max(float(np.max(np.abs(pert[i] - base[i])) / np.max(np.abs(base[i]))) for i in range(STEPS))


@pytest.mark.slow
def test_e2b_w4a16_scale_range_decides_whether_the_bound_can_hold():
    wide = _logit_drift(0.002, 0.02)
    narrow = _logit_drift(0.002, 0.0066)
    print(f"one-ulp cache change: drift {wide:.3e} (scales U(0.002, 0.02)), "
          f"{narrow:.3e} (U(0.002, 0.0066))")
    assert wide > 3e-2, wide            # the bound cannot hold for any bf16-cache implementation
    assert narrow < 3e-3, narrow        # ten times inside the bound


def _jitter_drift(name, quant, scales, kv_quant, rel, steps=32):
    """Max over `steps` teacher-forced steps of the relative logit change when
    every cached K/V element is computed with relative error ~rel (the
    oracle's jitter hook, applied before the cache rounds the row)."""
    cfg = synth.get_config(name)
    w = synth.generate(cfg, quant, seed=0, scale_lo=scales[0], scale_hi=scales[1])
    toks = synth.tokens(8 + steps, 1, cfg["vocab_size"])
    runs = []
    for j in (0.0, rel):
        orc = oracle.Oracle(cfg, quant, w, 1, 8 + steps + 1, kv_quant=kv_quant)
        orc.set_kv_jitter(j, 7)
        orc.prefill(0, toks[:8], logits=False)
        runs.append(np.array([orc.step(0, int(toks[8 + i]), 8 + i)[1] for i in range(steps)]))
        orc.close()
    a, b = runs
    return max(float(np.max(np.abs(a[i] - b[i])) / np.max(np.abs(a[i]))) for i in range(steps))


def test_toy_int8_cache_scale_range():
    """The same reading on the toy with the int8 K/V cache: the kernels carry
    activations to about 2^-17 relative (a bf16 hi/lo pair), so their cached
    rows differ from the fp64 oracle's by ~1e-5 relative.  At that level the
    toy10 W4A16 model with U(0.002, 0.02) scales moves its own int8-cache
    logits by more than half the 3e-2 bound (a cached value's rounding is a
    whole int8 step), with U(0.002, 0.0066) by an order of magnitude less
    than a tenth of it.  The int8-cache parity tests therefore draw W4A16
    toy scales from U(0.002, 0.0066), as the E2B workload does."""
    wide = _jitter_drift("toy10", "w4a16", (0.002, 0.02), "int8", 3e-5)
    narrow = _jitter_drift("toy10", "w4a16", (0.002, 0.0066), "int8", 3e-5)
    print(f"row error 3e-5, int8 cache: drift {wide:.3e} (U(0.002, 0.02)), {narrow:.3e} (U(0.002, 0.0066))")
    assert wide > 1.5e-2, wide
    assert narrow < 3e-3, narrow


@pytest.mark.slow
def test_e2b_bf16_cache_rounding_sensitivity():
    """The E2B bf16 workload (weights N(0, 0.02)) against the E2B W4A16 one
    under the same change: every cached K/V element computed with a relative
    error of 3e-6 before the cache rounds it to bf16 (about the kernels' own
    arithmetic error; it flips the rounding of the elements that sit that close
    to a rounding boundary).  Within 4 teacher-forced steps the bf16
    workload's logits move by about 5.5e-3 of max |logit|, the W4A16 one's by
    about 1e-5.  Two bf16 logits closer than twice that drift can therefore
    trade places in any implementation that does not reproduce the fp64
    oracle's values bit for bit: the bf16 greedy parity tests count a
    different token below that gap as a near-tie (E2B_BF16_DRIFT)."""
    bf = _jitter_drift("e2b", "bf16", (None, None), "bf16", 3e-6, steps=4)
    wq = _jitter_drift("e2b", "w4a16", (0.002, 0.0066), "bf16", 3e-6, steps=4)
    print(f"row error 3e-6, bf16 cache: drift {bf:.3e} (bf16 weights), {wq:.3e} (W4A16)")
    assert bf > 4e-3, bf
    assert wq < 1e-4, wq
