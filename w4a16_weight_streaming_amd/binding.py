"""ctypes binding of libe2b (include/e2b.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels.  PyTorch is
used for device memory (weight arena, K/V cache, workspace, token and logit
buffers) and for the current HIP stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_PKG, "libe2b.so")
_lib = None

E2B_OK, E2B_EINVAL, E2B_ERANGE, E2B_ENOMEM, E2B_EHIP, E2B_EDEVICE, E2B_ESTATE = range(7)
KINDS = {"qkv": 1, "o": 2, "gate_up": 3, "down": 4, "ple_gate": 5, "ple_proj": 6, "ple_model": 7,
         "lm_head": 8, "attn": 9}
QUANT = {"bf16": 0, "w4a16": 1}
KVQ = {"bf16": 0, "int8": 1}
DTYPE_BF16, DTYPE_INT32 = 0, 1


class E2BError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"e2b error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_hidden_layers", "num_kv_shared_layers", "hidden_size", "num_attention_heads",
        "num_key_value_heads", "head_dim", "global_head_dim", "sliding_window",
        "layer_pattern_period", "intermediate_size", "use_double_wide_mlp",
        "hidden_size_per_layer_input", "vocab_size", "quant", "embed_quant", "kv_quant",
        "group_size")] + \
        [(n, ctypes.c_float) for n in ("rms_eps", "rope_theta_sliding", "rope_theta_full")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 2), ("data", ctypes.c_void_p)]


def lib_path() -> str:
    return _LIB


def load_library():
    """Load libe2b.so.  torch is imported first so that the library binds to
    the HIP runtime torch already loaded (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads libamdhip64 first)
    if not os.path.exists(_LIB):
        raise E2BError(E2B_ESTATE, f"{_LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(_LIB)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.e2b_last_error.restype = ctypes.c_char_p
    L.e2b_config_preset.argtypes = [ctypes.c_char_p, ctypes.POINTER(Config)]
    L.e2b_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
    L.e2b_destroy.argtypes = [vp]
    L.e2b_destroy.restype = None
    L.e2b_kv_share_map.argtypes = [vp, vp]
    for f in ("e2b_weight_bytes", "e2b_arena_bytes"):
        getattr(L, f).restype = sz
        getattr(L, f).argtypes = [vp]
    L.e2b_kv_bytes.restype = sz
    L.e2b_kv_bytes.argtypes = [vp, i32, i32]
    L.e2b_workspace_bytes.restype = sz
    L.e2b_workspace_bytes.argtypes = [vp, i32]
    L.e2b_load_weights.argtypes = [vp, ctypes.POINTER(Tensor), i32, vp, sz, vp]
    L.e2b_kv_alloc.argtypes = [vp, vp, sz, i32, i32]
    L.e2b_decode_step.argtypes = [vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.e2b_prefill.argtypes = [vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    L.e2b_check.argtypes = [vp, vp, vp]
    L.e2b_graph_capture.argtypes = [vp, vp, vp, i32, vp, vp, vp, sz, i32, vp, ctypes.POINTER(vp)]
    L.e2b_graph_replay.argtypes = [vp, vp]
    L.e2b_graph_destroy.argtypes = [vp]
    L.e2b_graph_destroy.restype = None
    L.e2b_profile_begin.argtypes = [vp, i32]
    L.e2b_profile_read.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double)]
    L.e2b_kv_view.argtypes = [vp, i32, i32, ctypes.POINTER(vp)]
    L.e2b_matvec_workspace_bytes.restype = sz
    L.e2b_matvec_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.e2b_matvec.argtypes = [i32, vp, vp, i32, i32, vp, i32, vp, vp, sz, vp]
    L.e2b_embed.argtypes = [vp, vp, i32, vp, vp, vp, sz, vp]
    L.e2b_matvec_noalloc_max_bytes.restype = sz
    L.e2b_matvec_noalloc_max_bytes.argtypes = []
    L.e2b_matvec_noalloc.argtypes = [i32, vp, vp, i32, i32, vp, i32, vp, vp]
    L.e2b_stream_reduce.argtypes = [vp, sz, vp, vp]
    L.e2b_kv_paged_bytes.restype = sz
    L.e2b_kv_paged_bytes.argtypes = [vp, i32]
    L.e2b_kv_alloc_paged.argtypes = [vp, vp, sz, i32, vp, i32, i32, vp]
    L.e2b_seq_reserve.argtypes = [vp, i32, i32, vp]
    L.e2b_seq_release.argtypes = [vp, i32, vp]
    L.e2b_seq_move.argtypes = [vp, i32, i32, vp]
    L.e2b_pages_free.argtypes = [vp]
    L.e2b_stream_reduce_blocks.argtypes = []
    for f in ("e2b_config_preset", "e2b_create", "e2b_kv_share_map", "e2b_load_weights",
              "e2b_kv_alloc", "e2b_decode_step", "e2b_prefill", "e2b_check", "e2b_kv_view",
              "e2b_matvec", "e2b_matvec_noalloc", "e2b_embed", "e2b_stream_reduce",
              "e2b_stream_reduce_blocks", "e2b_kv_alloc_paged", "e2b_seq_reserve", "e2b_seq_release",
              "e2b_seq_move", "e2b_pages_free", "e2b_graph_capture", "e2b_graph_replay", "e2b_profile_begin",
              "e2b_profile_read"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != E2B_OK:
        raise E2BError(rc, load_library().e2b_last_error().decode())


def config_preset(name: str, quant: str = "bf16", embed_quant: str = "bf16",
                  kv_quant: str = "bf16") -> Config:
    c = Config()
    _check(load_library().e2b_config_preset(name.encode(), ctypes.byref(c)))
    c.quant = QUANT[quant]
    c.embed_quant = QUANT[embed_quant]
    c.kv_quant = KVQ[kv_quant]
    return c


def config_from_dict(d: dict, quant: str, embed_quant: str = "bf16", kv_quant: str = "bf16") -> Config:
    c = Config()
    for n, _ in Config._fields_:
        if n == "quant":
            c.quant = QUANT[quant]
        elif n == "embed_quant":
            c.embed_quant = QUANT[embed_quant]
        elif n == "kv_quant":
            c.kv_quant = KVQ[kv_quant]
        else:
            setattr(c, n, d[n])
    return c


class Model:
    """Host descriptor only (no device memory): sizes and the K/V share map."""

    def __init__(self, cfg: Config):
        self._lib = load_library()
        self.cfg = cfg
        h = ctypes.c_void_p()
        _check(self._lib.e2b_create(ctypes.byref(cfg), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self._lib.e2b_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    def kv_share_map(self):
        out = np.zeros(self.cfg.num_hidden_layers, np.int32)
        _check(self._lib.e2b_kv_share_map(self.handle, out.ctypes.data))
        return out.tolist()

    def weight_bytes(self) -> int:
        return self._lib.e2b_weight_bytes(self.handle)

    def arena_bytes(self) -> int:
        return self._lib.e2b_arena_bytes(self.handle)

    def kv_bytes(self, max_batch: int, max_ctx: int) -> int:
        return self._lib.e2b_kv_bytes(self.handle, max_batch, max_ctx)

    def workspace_bytes(self, max_rows: int) -> int:
        return self._lib.e2b_workspace_bytes(self.handle, max_rows)


def _tensor_table(tensors: Dict[str, np.ndarray]):
    keep, arr = [], (Tensor * len(tensors))()
    for i, (name, a) in enumerate(tensors.items()):
        a = np.ascontiguousarray(a)
        keep.append(a)
        if a.dtype == np.uint16:
            dt = DTYPE_BF16
        elif a.dtype in (np.int32, np.uint32):
            dt = DTYPE_INT32
        else:
            raise E2BError(E2B_EINVAL, f"tensor {name}: dtype {a.dtype} is not bf16 bits or int32")
        arr[i].name = name.encode()
        arr[i].dtype = dt
        arr[i].ndim = a.ndim
        arr[i].shape[0] = a.shape[0]
        arr[i].shape[1] = a.shape[1] if a.ndim > 1 else 0
        arr[i].data = a.ctypes.data
    return arr, keep


def matvec(quant: str, w, scale, x, y, ws=None):
    """y[r] = W x[r] on the device (torch tensors): w bf16-bits int16 [N, K] or
    packed int32 [N, K/8]; scale bf16-bits int16 [N, K/32] or None; x fp32
    [rows, K]; y fp32 [rows, N]; ws uint8 scratch if K needs splitting."""
    import torch
    L = load_library()
    N = y.shape[-1]
    K = x.shape[-1]
    rows = x.numel() // K
    need = L.e2b_matvec_workspace_bytes(QUANT[quant], N, K, rows)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(L.e2b_matvec(QUANT[quant], w.data_ptr(), 0 if scale is None else scale.data_ptr(), N, K,
                        x.data_ptr(), rows, y.data_ptr(), 0 if ws is None else ws.data_ptr(),
                        0 if ws is None else ws.numel(), torch.cuda.current_stream(x.device).cuda_stream))
    return y


def stream_reduce(buf, out):
    """The calibration read: one pass over the bytes of device tensor `buf`
    (a multiple of 16 bytes), per-block sums into `out` (float32, at least
    e2b_stream_reduce_blocks() entries).  Asynchronous on the current stream."""
    import torch
    L = load_library()
    assert out.dtype == torch.float32 and out.numel() >= L.e2b_stream_reduce_blocks()
    _check(L.e2b_stream_reduce(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                               torch.cuda.current_stream(buf.device).cuda_stream))


class Engine:
    """A loaded model bound to device memory on one GPU.

    cfg: preset name or a config dict (HF-style field names); quant "bf16" or
    "w4a16"; tensors: canonical host tensors (see include/e2b.h).
    """

    def __init__(self, cfg, quant: str, tensors: Dict[str, np.ndarray], max_batch: int,
                 max_ctx: int, max_rows: Optional[int] = None, device: str = "cuda:0",
                 kv_quant: str = "bf16", n_pages: int = 0):
        import torch
        self.torch = torch
        if not torch.cuda.is_available():
            raise E2BError(E2B_ESTATE, "no GPU visible to torch; libe2b has no CPU path")
        self.device = torch.device(device)
        arch = torch.cuda.get_device_properties(self.device).gcnArchName
        if not arch.startswith("gfx950"):
            raise E2BError(E2B_ESTATE, f"device is {arch}; libe2b is built for gfx950 only")
        # the vocabulary tables' format follows the tensors given
        eq = "w4a16" if "model.embed_tokens.weight_packed" in tensors else "bf16"
        c = (config_preset(cfg, quant, eq, kv_quant) if isinstance(cfg, str)
             else config_from_dict(cfg, quant, eq, kv_quant))
        self.embed_quant, self.kv_quant = eq, kv_quant
        self.model = Model(c)
        self.cfg = c
        self.quant = quant
        self.max_batch, self.max_ctx = max_batch, max_ctx
        self.max_rows = max_rows or max(max_batch, 1)
        L = self.model._lib
        with torch.cuda.device(self.device):
            self.arena = torch.empty(self.model.arena_bytes(), dtype=torch.uint8, device=self.device)
            table, keep = _tensor_table(tensors)
            _check(L.e2b_load_weights(self.model.handle, table, len(tensors), self.arena.data_ptr(),
                                      self.arena.numel(), self._stream()))
            del keep
            self.n_pages = n_pages
            if n_pages:   # paged cache: a pool of n_pages pages and its page table
                self.kv = torch.empty(max(L.e2b_kv_paged_bytes(self.model.handle, n_pages), 1),
                                      dtype=torch.uint8, device=self.device)
                stride = (max_ctx + 127) // 128
                self.page_table = torch.full((max_batch, stride), -1, dtype=torch.int32, device=self.device)
                _check(L.e2b_kv_alloc_paged(self.model.handle, self.kv.data_ptr(), self.kv.numel(), n_pages,
                                            self.page_table.data_ptr(), max_batch, max_ctx, self._stream()))
            else:
                self.kv = torch.empty(max(self.model.kv_bytes(max_batch, max_ctx), 1),
                                      dtype=torch.uint8, device=self.device)
                _check(L.e2b_kv_alloc(self.model.handle, self.kv.data_ptr(), self.kv.numel(),
                                      max_batch, max_ctx))
            self.ws = torch.zeros(self.model.workspace_bytes(self.max_rows), dtype=torch.uint8,
                                  device=self.device)

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    @staticmethod
    def _ptr(t) -> int:
        return 0 if t is None else t.data_ptr()

    def decode_step(self, tokens, positions, argmax_out, logits_out=None):
        """tokens, positions, argmax_out: int32 device tensors [B];
        logits_out: float32 device tensor [B, V] or None.  Asynchronous."""
        B = tokens.numel()
        assert tokens.dtype == positions.dtype == argmax_out.dtype == self.torch.int32
        assert positions.numel() == B and argmax_out.numel() >= B
        if logits_out is not None:
            assert logits_out.dtype == self.torch.float32 and logits_out.numel() >= B * self.cfg.vocab_size
        _check(self.model._lib.e2b_decode_step(
            self.model.handle, tokens.data_ptr(), positions.data_ptr(), B, self._ptr(logits_out),
            argmax_out.data_ptr(), self.ws.data_ptr(), self.ws.numel(), self._stream()))

    def prefill(self, seq: int, tokens, pos0: int, argmax_out, logits_out=None):
        """tokens: int32 device tensor [n]; writes K/V for positions pos0..pos0+n-1
        of cache row seq and the last position's argmax (and logits)."""
        assert tokens.dtype == self.torch.int32 and argmax_out.dtype == self.torch.int32
        _check(self.model._lib.e2b_prefill(
            self.model.handle, seq, tokens.data_ptr(), tokens.numel(), pos0, self._ptr(logits_out),
            argmax_out.data_ptr(), self.ws.data_ptr(), self.ws.numel(), self._stream()))

    def embed(self, tokens, h_out, tokple_out):
        """The step's embedding gathers alone: h_out float32 [n, H] = E[t] * sqrt(H),
        tokple_out float32 [n, L*P] = E_ple[t] * sqrt(P).  Asynchronous; n must not
        exceed max_rows."""
        n = tokens.numel()
        assert tokens.dtype == self.torch.int32 and h_out.dtype == tokple_out.dtype == self.torch.float32
        assert h_out.numel() >= n * self.cfg.hidden_size
        assert tokple_out.numel() >= n * self.cfg.num_hidden_layers * self.cfg.hidden_size_per_layer_input
        _check(self.model._lib.e2b_embed(self.model.handle, tokens.data_ptr(), n, h_out.data_ptr(),
                                         tokple_out.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                         self._stream()))

    # ---- paged cache: the library's page allocator
    def reserve(self, slot: int, n_positions: int):
        _check(self.model._lib.e2b_seq_reserve(self.model.handle, slot, n_positions, self._stream()))

    def release(self, slot: int):
        _check(self.model._lib.e2b_seq_release(self.model.handle, slot, self._stream()))

    def move(self, src: int, dst: int):
        _check(self.model._lib.e2b_seq_move(self.model.handle, src, dst, self._stream()))

    def pages_free(self) -> int:
        return self.model._lib.e2b_pages_free(self.model.handle)

    def kv_view(self, layer: int, which: int) -> int:
        """Device address of the K (0) / V (1) region layer `layer` reads."""
        out = ctypes.c_void_p()
        _check(self.model._lib.e2b_kv_view(self.model.handle, layer, which, ctypes.byref(out)))
        return out.value or 0

    def kv_tensor(self, layer: int, which: int, hd: int):
        """The K or V region layer `layer` reads, as a view [max_batch, max_ctx,
        hd] of the K/V buffer (no copy): bf16 bits (int16), or int8 codes."""
        addr = self.kv_view(layer, which)
        off = addr - self.kv.data_ptr()
        n = self.max_batch * self.max_ctx * hd
        if self.kv_quant == "int8":
            return self.kv[off:off + n].view(self.torch.int8).view(self.max_batch, self.max_ctx, hd)
        return self.kv[off:off + 2 * n].view(self.torch.int16).view(self.max_batch, self.max_ctx, hd)

    def kv_scales(self, layer: int, which: int):
        """int8 cache: the K (0) or V (1) row scales layer `layer` reads, float32
        view [max_batch, max_ctx]."""
        assert self.kv_quant == "int8"
        addr = self.kv_view(layer, 2 + which)
        off = addr - self.kv.data_ptr()
        n = self.max_batch * self.max_ctx
        return self.kv[off:off + 4 * n].view(self.torch.float32).view(self.max_batch, self.max_ctx)

    def capture(self, tokens, positions, argmax_out, logits_out=None, advance: bool = True):
        """Capture one decode step (+ positions += 1) as a graph on the current
        stream (must not be the null stream).  Returns a Graph."""
        g = ctypes.c_void_p()
        _check(self.model._lib.e2b_graph_capture(
            self.model.handle, tokens.data_ptr(), positions.data_ptr(), tokens.numel(),
            self._ptr(logits_out), argmax_out.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
            1 if advance else 0, self._stream(), ctypes.byref(g)))
        return Graph(self, g)

    def profile_begin(self, kind: str):
        _check(self.model._lib.e2b_profile_begin(self.model.handle, KINDS[kind]))

    def profile_read(self):
        """(launches, total_ms, total_bytes) of the profiled kind; stops profiling."""
        n, ms, by = ctypes.c_int(), ctypes.c_double(), ctypes.c_double()
        _check(self.model._lib.e2b_profile_read(self.model.handle, ctypes.byref(n), ctypes.byref(ms),
                                                 ctypes.byref(by)))
        return n.value, ms.value, by.value

    def check(self):
        """Synchronise and raise E2BError if a kernel flagged a bad token/position."""
        _check(self.model._lib.e2b_check(self.model.handle, self.ws.data_ptr(), self._stream()))


class Graph:
    """A captured decode step; replay() enqueues it on the current stream."""

    def __init__(self, eng: "Engine", handle):
        self.eng, self.handle = eng, handle

    def replay(self):
        _check(self.eng.model._lib.e2b_graph_replay(self.handle, self.eng._stream()))

    def close(self):
        if getattr(self, "handle", None):
            self.eng.model._lib.e2b_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()
