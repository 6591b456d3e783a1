"""fp64 CPU oracle of the Gemma-4-E2B-shaped decode step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its binding) never does, and
this package imports nothing from it.

Two independent references live here:

* ``oracle.c`` (wrapped by :class:`Oracle`): a plain double-precision step with
  a K/V cache, OpenMP over the output rows of each matrix-vector product and
  nothing else (no blocking, fusion or reordering).
* ``naive.py``: a numpy brute force that re-runs the whole sequence every step
  with no cache, for tiny shapes only.

Both follow the definitions on the pages "Gemma 4 E2B in JAX on One TPU v5e"
(Step 4: RMSNorm), "Porting Gemma 4 E2B to SGLang-JAX" (Steps 1, 3, 4, 5:
layer table, per-layer embeddings, shared K/V, double-wide MLP), "One TPU
chip, eight agents" (The engine: kv_share_map and the W4A16 packing) and
"Gemma 4 E2B in Pure JAX on a Colab TPU" (intro table, cells 2.2 and 3.1:
group-of-32 scales, tied lm_head, exact unpack).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "num_hidden_layers", "num_kv_shared_layers", "hidden_size", "num_attention_heads",
        "num_key_value_heads", "head_dim", "global_head_dim", "sliding_window",
        "layer_pattern_period", "intermediate_size", "use_double_wide_mlp",
        "hidden_size_per_layer_input", "vocab_size", "quant", "group_size")] + \
        [(n, ctypes.c_double) for n in ("rms_eps", "rope_theta_sliding", "rope_theta_full")] + \
        [("kv_bf16", ctypes.c_int), ("embed_quant", ctypes.c_int), ("kv_quant", ctypes.c_int)]


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp,
                               src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.orc_error.restype = ctypes.c_char_p
        L.orc_create.restype = vp
        L.orc_create.argtypes = [ctypes.POINTER(OrcConfig), i32, ctypes.POINTER(ctypes.c_char_p),
                                 ctypes.POINTER(vp), i32, i32]
        L.orc_destroy.argtypes = [vp]
        L.orc_step.restype = i32
        L.orc_step.argtypes = [vp, i32, i32, i32, dp, dp]
        L.orc_step_ex.restype = i32
        L.orc_step_ex.argtypes = [vp, i32, i32, i32, i32, dp, dp]
        L.orc_prefill.restype = i32
        L.orc_prefill.argtypes = [vp, i32, dp, i32, i32, dp]
        L.orc_kv_source.restype = i32
        L.orc_kv_source.argtypes = [vp, i32]
        L.orc_kv_row.restype = ctypes.POINTER(ctypes.c_double)
        L.orc_kv_row.argtypes = [vp, i32, i32, i32, i32]
        L.orc_kv_load.restype = i32
        L.orc_kv_load.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.orc_set_kv_jitter.argtypes = [vp, ctypes.c_double, ctypes.c_uint64]
        L.orc_kv_set.restype = i32
        L.orc_kv_set.argtypes = [vp, i32, i32, i32, i32, dp]
        L.orc_linear_apply.argtypes = [i32, vp, vp, i32, i32, i32, dp, dp]
        L.orc_decode_weight.restype = ctypes.c_double
        L.orc_decode_weight.argtypes = [i32, vp, vp, i32, i32, i32, i64, i64]
        L.orc_rmsnorm.argtypes = [dp, i32, vp, ctypes.c_double, dp]
        L.orc_gelu_tanh.restype = ctypes.c_double
        L.orc_gelu_tanh.argtypes = [ctypes.c_double]
        L.orc_rope.argtypes = [dp, i32, i32, ctypes.c_double]
        L.orc_attend.argtypes = [dp, i32, dp, dp, i32, i32, dp]
        L.orc_argmax.restype = i32
        L.orc_argmax.argtypes = [dp, i32]
        L.orc_debug_inputs.restype = i32
        L.orc_debug_inputs.argtypes = [vp, i32, dp, dp]
        L.orc_set_threads.argtypes = [i32]
        L.orc_quant_int8.argtypes = [dp, i32, vp, vp]
        L.orc_get_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def make_config(cfg: dict, quant: str, kv_bf16: bool = True, embed_quant: str = "bf16",
                kv_quant: str = "bf16") -> OrcConfig:
    c = OrcConfig()
    for name, _ in OrcConfig._fields_:
        if name == "quant":
            c.quant = 1 if quant == "w4a16" else 0
        elif name == "kv_bf16":
            c.kv_bf16 = 1 if kv_bf16 else 0
        elif name == "embed_quant":
            c.embed_quant = 1 if embed_quant == "w4a16" else 0
        elif name == "kv_quant":
            c.kv_quant = 1 if kv_quant == "int8" else 0
        else:
            setattr(c, name, cfg[name])
    return c


class Oracle:
    """The C reference over one synthetic model (tensors from ``synth``)."""

    def __init__(self, cfg: dict, quant: str, tensors: Dict[str, np.ndarray], max_seq: int,
                 max_ctx: int, kv_bf16: bool = True, embed_quant: str = None, kv_quant: str = "bf16"):
        self.cfg, self.quant = cfg, quant
        self.V, self.H = cfg["vocab_size"], cfg["hidden_size"]
        self._keep = {k: np.ascontiguousarray(v) for k, v in tensors.items()}
        names = list(self._keep)
        self._names = (ctypes.c_char_p * len(names))(*[n.encode() for n in names])
        self._ptrs = (ctypes.c_void_p * len(names))(*[_ptr(self._keep[n]) for n in names])
        if embed_quant is None:   # the vocabulary tables' format, read off the tensors
            embed_quant = "w4a16" if "model.embed_tokens.weight_packed" in tensors else "bf16"
        self.embed_quant = embed_quant
        self.kv_quant = kv_quant   # "bf16" (or fp64 without kv_bf16) / "int8"
        self._cfg = make_config(cfg, quant, kv_bf16, embed_quant, kv_quant)
        self.max_seq, self.max_ctx = max_seq, max_ctx
        h = lib().orc_create(ctypes.byref(self._cfg), len(names), self._names, self._ptrs,
                             max_seq, max_ctx)
        if not h:
            raise RuntimeError("oracle: " + lib().orc_error().decode())
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().orc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def step(self, seq: int, token: int, pos: int, logits: bool = True, hidden: bool = False):
        """One token; returns (argmax, logits[V] float64 or None, y[H] or None)."""
        lg = np.empty(self.V, np.float64) if logits else None
        y = np.empty(self.H, np.float64) if hidden else None
        r = lib().orc_step(self._h, seq, int(token), int(pos), _ptr(lg) if logits else None,
                           _ptr(y) if hidden else None)
        if r < 0:
            raise RuntimeError("oracle: " + lib().orc_error().decode())
        return r, lg, y

    def prefill(self, seq: int, toks, pos0: int = 0, logits: bool = True):
        t = np.ascontiguousarray(toks, dtype=np.int32)
        lg = np.empty(self.V, np.float64) if logits else None
        r = lib().orc_prefill(self._h, seq, _ptr(t), len(t), pos0, _ptr(lg) if logits else None)
        if r < 0:
            raise RuntimeError("oracle: " + lib().orc_error().decode())
        return r, lg

    def inputs(self, token: int):
        """(e [H], pli [L, P]) for one token: the embedding and per-layer inputs."""
        L, P = self.cfg["num_hidden_layers"], self.cfg["hidden_size_per_layer_input"]
        e = np.empty(self.H, np.float64)
        pli = np.empty(L * P, np.float64)
        if lib().orc_debug_inputs(self._h, int(token), _ptr(e), _ptr(pli)) != 0:
            raise RuntimeError("oracle: token out of range")
        return e, pli.reshape(L, P)

    def kv_source(self, l: int) -> int:
        return lib().orc_kv_source(self._h, l)

    def kv_row(self, l: int, which: int, seq: int, pos: int, hd: int) -> np.ndarray:
        p = lib().orc_kv_row(self._h, l, which, seq, pos)
        return np.ctypeslib.as_array(p, shape=(hd,)).copy()

    def set_kv_jitter(self, rel: float, seed: int = 1) -> None:
        """Test hook: multiply each new K/V element by (1 + rel * u), u uniform in
        [-1, 1) (seeded), before the cache rounds it -- an implementation that
        computes the same rows with relative error ~rel.  0 turns it off."""
        lib().orc_set_kv_jitter(self._h, float(rel), int(seed))

    def kv_set(self, l: int, which: int, seq: int, pos: int, row) -> None:
        """Overwrite one cached K (0) or V (1) row of a K/V-owning layer with the
        given values (test set-up: a controlled perturbation of the cache)."""
        r = np.ascontiguousarray(row, np.float64)
        if lib().orc_kv_set(self._h, l, which, seq, pos, _ptr(r)) != 0:
            raise RuntimeError("oracle: bad kv_set arguments")

    def kv_load(self, l: int, seq: int, pos0: int, k_bits: np.ndarray, v_bits: np.ndarray):
        """Set cached positions pos0.. of a K/V-owning layer from bf16 bits [n, hd]
        (test set-up: seeded cache contents in place of a long prefill)."""
        k = np.ascontiguousarray(k_bits, np.uint16)
        v = np.ascontiguousarray(v_bits, np.uint16)
        if lib().orc_kv_load(self._h, l, seq, pos0, k.shape[0], _ptr(k), _ptr(v)) != 0:
            raise RuntimeError("oracle: bad kv_load arguments")


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's products (process-wide)."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


# ---- single pieces, for the pins -------------------------------------------
def linear(quant: str, w: np.ndarray, scale: Optional[np.ndarray], N: int, K: int, x,
           G: int = 32) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty(N, np.float64)
    lib().orc_linear_apply(1 if quant == "w4a16" else 0, _ptr(w),
                           _ptr(scale) if scale is not None else None, N, K, G, _ptr(x), _ptr(y))
    return y


def decode_weight(quant, w, scale, N, K, n, k, G=32) -> float:
    return lib().orc_decode_weight(1 if quant == "w4a16" else 0, _ptr(w),
                                   _ptr(scale) if scale is not None else None, N, K, G, n, k)


def rmsnorm(x, gain_bf16=None, eps=1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), len(x), _ptr(gain_bf16) if gain_bf16 is not None else None, eps,
                      _ptr(y))
    return y


def gelu_tanh(x: float) -> float:
    return lib().orc_gelu_tanh(float(x))


def rope(x, pos: int, theta: float) -> np.ndarray:
    y = np.array(x, np.float64, copy=True)
    lib().orc_rope(_ptr(y), len(y), pos, theta)
    return y


def attend(q, K, V, j0: int, j1: int) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    o = np.empty(len(q), np.float64)
    lib().orc_attend(_ptr(q), len(q), _ptr(K), _ptr(V), j0, j1, _ptr(o))
    return o


def quant_int8(x):
    """(codes int8 [n], scale) of one cached row, as the int8 cache stores it."""
    x = np.ascontiguousarray(x, np.float64)
    q = np.empty(len(x), np.int8)
    sc = np.empty(1, np.float32)
    lib().orc_quant_int8(_ptr(x), len(x), _ptr(q), _ptr(sc))
    return q, float(sc[0])


def argmax(x) -> int:
    x = np.ascontiguousarray(x, np.float64)
    return lib().orc_argmax(_ptr(x), len(x))
