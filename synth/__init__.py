"""Seeded synthetic workloads for the Gemma-4-E2B-shaped decode step.

This module is shared input plumbing: it turns (seed, tensor name, index) into
bytes and holds none of the decoder's arithmetic.  Both the fp64 oracle under
``oracle/`` and the HIP library consume exactly the bytes produced here.

Canonical tensor format (what both consumers read):

* bf16 tensors: ``numpy.uint16`` arrays holding raw bfloat16 bit patterns.
* W4A16 linears (compressed-tensors style): ``<name>.weight_packed`` int32
  ``[N, K/8]`` where word ``j`` of row ``n`` holds K-elements ``8j..8j+7`` and
  element ``8j+i`` sits in bits ``[4i, 4i+4)`` as the offset code ``q + 8``;
  ``<name>.weight_scale`` bf16 ``[N, K/32]``, one scale per 32 consecutive K.
  The generator draws the packed words as uniform bits, so every code is
  uniform on 0..15, i.e. ``q`` is uniform on -8..7.

Distributions (synthetic random init; no trained checkpoint is used):

* linear weights (bf16 mode) and both embedding tables: N(0, 0.02)
* W4A16 codes: uniform; scales: U(0.002, 0.02) for the toy workloads and
  U(0.002, 0.0066) for the E2B workload (dequantized rms 0.02, as bf16)
* RMSNorm gains: 1 + N(0, 0.02); layer scalars: U(0.5, 1.0)
* prompt tokens: uniform over the vocabulary

The model shapes follow the Gemma 4 E2B configuration printed on "Porting
Gemma 4 E2B to SGLang-JAX on One Cloud TPU v5e" (Step 1 table: 35 layers, 20
KV-shared, per-layer input 256, one KV head, head dims 256/512, 4 sliding + 1
full repeating) and the 4.70 GB per-layer table of "One TPU chip, eight
agents" (Measured section).  hidden 1536, 8 query heads, window 512 and the
toy sizes are workload parameters of this project, not page facts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import zlib
from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# ---------------------------------------------------------------------------
# workload presets (plain data; HF-style field names)
# ---------------------------------------------------------------------------
_BASE = dict(num_key_value_heads=1, layer_pattern_period=5, use_double_wide_mlp=1,
             group_size=32, rms_eps=1e-6, rope_theta_sliding=1.0e4, rope_theta_full=1.0e6,
             w4a16_scale=(0.002, 0.02))

CONFIGS: Dict[str, dict] = {
    # 5 layers (4 sliding + 1 full), last 2 KV-shared, window 16
    "toy": dict(_BASE, name="toy", num_hidden_layers=5, num_kv_shared_layers=2, hidden_size=256,
                num_attention_heads=2, head_dim=64, global_head_dim=128, sliding_window=16,
                intermediate_size=512, hidden_size_per_layer_input=32, vocab_size=4096),
    # 10 layers (2 full), last 5 KV-shared: exercises full-layer sharing
    "toy10": dict(_BASE, name="toy10", num_hidden_layers=10, num_kv_shared_layers=5, hidden_size=256,
                  num_attention_heads=2, head_dim=64, global_head_dim=128, sliding_window=16,
                  intermediate_size=512, hidden_size_per_layer_input=32, vocab_size=4096),
    # full E2B shape
    # full E2B shape.  W4A16 group scales U(0.002, 0.0066): the dequantized
    # weights then have rms 0.02, the same as the bf16 workload's N(0, 0.02)
    # (the W4A16 workload is the bf16 one with quantized storage).
    "e2b": dict(_BASE, name="e2b", num_hidden_layers=35, num_kv_shared_layers=20, hidden_size=1536,
                num_attention_heads=8, head_dim=256, global_head_dim=512, sliding_window=512,
                intermediate_size=6144, hidden_size_per_layer_input=256, vocab_size=262144,
                w4a16_scale=(0.002, 0.0066)),
}


def get_config(name: str) -> dict:
    return dict(CONFIGS[name])


def layer_is_full(cfg: dict, l: int) -> bool:
    """Layer type by position: the 5-periodic '4 sliding, 1 full' pattern."""
    p = cfg["layer_pattern_period"]
    return (l % p) == p - 1


def layer_head_dim(cfg: dict, l: int) -> int:
    return cfg["global_head_dim"] if layer_is_full(cfg, l) else cfg["head_dim"]


def layer_intermediate(cfg: dict, l: int) -> int:
    first_shared = cfg["num_hidden_layers"] - cfg["num_kv_shared_layers"]
    wide = cfg["use_double_wide_mlp"] and l >= first_shared
    return cfg["intermediate_size"] * (2 if wide else 1)


# ---------------------------------------------------------------------------
# tensor inventory
# ---------------------------------------------------------------------------
@dataclass
class Spec:
    name: str          # canonical parameter name (no .weight_packed suffix)
    shape: Tuple[int, ...]
    kind: str          # "linear" | "embed" | "gain" | "scalar"


def tensor_specs(cfg: dict, kv_all_layers: bool = True) -> List[Spec]:
    """Every parameter of the decoder.  K-side tensors (k_proj, v_proj, k_norm)
    are listed for every layer when ``kv_all_layers`` (like the bf16 export);
    consumers that share K/V ignore the ones they do not read."""
    H, V, L = cfg["hidden_size"], cfg["vocab_size"], cfg["num_hidden_layers"]
    P, nq = cfg["hidden_size_per_layer_input"], cfg["num_attention_heads"]
    first_shared = L - cfg["num_kv_shared_layers"]
    out = [Spec("model.embed_tokens.weight", (V, H), "embed"),
           Spec("model.embed_tokens_per_layer.weight", (V, L * P), "embed"),
           Spec("model.per_layer_model_projection.weight", (L * P, H), "linear"),
           Spec("model.per_layer_projection_norm.weight", (P,), "gain"),
           Spec("model.norm.weight", (H,), "gain")]
    for l in range(L):
        hd, I = layer_head_dim(cfg, l), layer_intermediate(cfg, l)
        pre = f"model.layers.{l}."
        kv = kv_all_layers or l < first_shared
        out += [Spec(pre + "input_layernorm.weight", (H,), "gain"),
                Spec(pre + "self_attn.q_proj.weight", (nq * hd, H), "linear")]
        if kv:
            out += [Spec(pre + "self_attn.k_proj.weight", (hd, H), "linear"),
                    Spec(pre + "self_attn.v_proj.weight", (hd, H), "linear")]
        out += [Spec(pre + "self_attn.o_proj.weight", (H, nq * hd), "linear"),
                Spec(pre + "self_attn.q_norm.weight", (hd,), "gain")]
        if kv:
            out += [Spec(pre + "self_attn.k_norm.weight", (hd,), "gain")]
        out += [Spec(pre + "post_attention_layernorm.weight", (H,), "gain"),
                Spec(pre + "pre_feedforward_layernorm.weight", (H,), "gain"),
                Spec(pre + "mlp.gate_proj.weight", (I, H), "linear"),
                Spec(pre + "mlp.up_proj.weight", (I, H), "linear"),
                Spec(pre + "mlp.down_proj.weight", (H, I), "linear"),
                Spec(pre + "post_feedforward_layernorm.weight", (H,), "gain"),
                Spec(pre + "per_layer_input_gate.weight", (P, H), "linear"),
                Spec(pre + "per_layer_projection.weight", (H, P), "linear"),
                Spec(pre + "post_per_layer_input_norm.weight", (H,), "gain"),
                Spec(pre + "layer_scalar", (1,), "scalar")]
    return out


# ---------------------------------------------------------------------------
# native generator
# ---------------------------------------------------------------------------
def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_normal_bf16.argtypes = [vp, i64, u64, f32, f32]
        lib.synth_uniform_bf16.argtypes = [vp, i64, u64, f32, f32]
        lib.synth_bits32.argtypes = [vp, i64, u64]
        lib.synth_tokens.argtypes = [vp, i64, u64, ctypes.c_int32]
        _lib = lib
    return _lib


def _stream(name: str) -> int:
    return zlib.crc32(name.encode()) | (len(name) << 32)


def _key(seed: int, name: str) -> int:
    return _load().synth_key(seed, _stream(name))


def normal_bf16(shape, seed: int, name: str, mean: float = 0.0, std: float = 0.02) -> np.ndarray:
    a = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(a.ctypes.data, a.size, _key(seed, name), mean, std)
    return a


def uniform_bf16(shape, seed: int, name: str, lo: float, hi: float) -> np.ndarray:
    a = np.empty(shape, dtype=np.uint16)
    _load().synth_uniform_bf16(a.ctypes.data, a.size, _key(seed, name), lo, hi)
    return a


def bits32(shape, seed: int, name: str) -> np.ndarray:
    a = np.empty(shape, dtype=np.int32)
    _load().synth_bits32(a.ctypes.data, a.size, _key(seed, name))
    return a


def tokens(n: int, seed: int, vocab: int, stream: str = "prompt") -> np.ndarray:
    a = np.empty((n,), dtype=np.int32)
    _load().synth_tokens(a.ctypes.data, n, _key(seed, stream), vocab)
    return a


def generate(cfg: dict, quant: str = "bf16", seed: int = 0, kv_all_layers: bool = True,
             scale_lo: float = None, scale_hi: float = None,
             embed_quant: str = "bf16") -> Dict[str, np.ndarray]:
    """All tensors of one synthetic model, keyed by canonical name.

    quant "bf16": linears are ``<name>`` bf16 [N, K].
    quant "w4a16": linears are ``<name>_packed`` int32 [N, K/8] plus
    ``<name>_scale`` bf16 [N, K/32] (name ends in ``.weight`` so the keys are
    ``...weight_packed`` / ``...weight_scale``).
    embed_quant "w4a16": the two vocabulary tables (the tied token embedding
    and the per-layer table) in that same format too, codes uniform and group
    scales from the workload's W4A16 range (the int4 vocabulary tables of the
    pages' "text-emb4" build); "bf16": N(0, 0.02) bf16 tables.
    """
    assert quant in ("bf16", "w4a16") and embed_quant in ("bf16", "w4a16")
    G = cfg["group_size"]
    lo, hi = cfg.get("w4a16_scale", (0.002, 0.02))
    scale_lo = lo if scale_lo is None else scale_lo
    scale_hi = hi if scale_hi is None else scale_hi
    out: Dict[str, np.ndarray] = {}
    for s in tensor_specs(cfg, kv_all_layers=kv_all_layers):
        if s.kind == "embed" and embed_quant == "w4a16":
            N, K = s.shape
            out[s.name + "_packed"] = bits32((N, K // 8), seed, s.name + "_packed")
            out[s.name + "_scale"] = uniform_bf16((N, K // G), seed, s.name + "_scale", scale_lo, scale_hi)
        elif s.kind == "embed":
            out[s.name] = normal_bf16(s.shape, seed, s.name)
        elif s.kind == "gain":
            out[s.name] = normal_bf16(s.shape, seed, s.name, 1.0, 0.02)
        elif s.kind == "scalar":
            out[s.name] = uniform_bf16(s.shape, seed, s.name, 0.5, 1.0)
        elif quant == "bf16":
            out[s.name] = normal_bf16(s.shape, seed, s.name)
        else:
            N, K = s.shape
            assert K % G == 0
            out[s.name + "_packed"] = bits32((N, K // 8), seed, s.name + "_packed")
            out[s.name + "_scale"] = uniform_bf16((N, K // G), seed, s.name + "_scale",
                                                  scale_lo, scale_hi)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to float32 (a reinterpretation)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even narrowing of float32 to raw bf16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)
