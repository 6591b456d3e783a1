"""Brute-force numpy reference: re-runs the whole token sequence through every
layer at every step, with no K/V cache.  TEST INFRASTRUCTURE (tiny shapes only).

Written as a second, differently structured formulation of the same step, so
that the cached C oracle can be pinned against it (the "cached decode versus
re-running the full model over the growing sequence" check described on "One
TPU chip, eight agents", The engine):

* weights are decoded to whole float64 matrices with vectorised bit ops;
* attention is one masked score matrix per head over the whole sequence
  (causal, plus the sliding-window band on sliding layers); with kv_bf16 the
  keys and values are rounded to bf16 as the cache stores them;
* RoPE is a complex rotation of the (i, i + hd/2) pairs;
* RMSNorm uses a vector norm.
"""
from __future__ import annotations

import numpy as np


def _bf(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _round_bf16(a):
    """fp64 -> fp32 -> nearest-even bf16, back to fp64 (the cache stores bf16)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _int8_rows(a):
    """Each row (one token's K or V) as symmetric int8 with one scale, decided
    in float32: scale = max |x| / 127, codes nearest-even, read back as
    code * scale."""
    a32 = np.asarray(a, np.float32)
    sc = np.max(np.abs(a32), axis=-1, keepdims=True) / np.float32(127)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sc > 0, np.rint(a32 / sc), np.float32(0))
    return np.clip(q, -127, 127).astype(np.float64) * sc.astype(np.float64)


def _layer_is_full(cfg, l):
    return l % cfg["layer_pattern_period"] == cfg["layer_pattern_period"] - 1


def _dense(tensors, name, quant, G=32):
    if quant == "bf16":
        return _bf(tensors[name])
    packed = tensors[name + "_packed"].view(np.uint32)
    N, K8 = packed.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    codes = (packed[:, :, None] >> shifts) & np.uint32(15)
    q = codes.reshape(N, K8 * 8).astype(np.float64) - 8.0
    return q * np.repeat(_bf(tensors[name + "_scale"]), G, axis=1)


def _norm(x, g=None, eps=1e-6):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    r = np.linalg.norm(x, axis=-1, keepdims=True) / np.sqrt(d)
    y = x / np.sqrt(r * r + eps)
    return y if g is None else y * g


def _gelu(x):
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def _rope(x, positions, theta):
    """x [..., T, hd]; rotate pair (i, i+hd/2) by angle p * theta^(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half) / hd)
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


class Naive:
    def __init__(self, cfg: dict, quant: str, tensors: dict, kv_bf16: bool = True, kv_quant: str = "bf16"):
        self.cfg, self.quant, self.kv_bf16, self.kv_quant = cfg, quant, kv_bf16, kv_quant
        c = cfg
        self.L, self.H, self.P = c["num_hidden_layers"], c["hidden_size"], c["hidden_size_per_layer_input"]
        self.nq, self.V = c["num_attention_heads"], c["vocab_size"]
        self.first = self.L - c["num_kv_shared_layers"]
        t = tensors
        # the vocabulary tables: bf16, or int4 codes with group scales
        eq = "w4a16" if "model.embed_tokens.weight_packed" in t else "bf16"
        self.E = _dense(t, "model.embed_tokens.weight", eq)
        self.Eple = _dense(t, "model.embed_tokens_per_layer.weight", eq)
        self.Wplmp = _dense(t, "model.per_layer_model_projection.weight", quant)
        self.g_plpn = _bf(t["model.per_layer_projection_norm.weight"])
        self.g_f = _bf(t["model.norm.weight"])
        self.layers = []
        for l in range(self.L):
            p = f"model.layers.{l}."
            full = _layer_is_full(c, l)
            # source of K/V: last non-shared layer of the same type, else itself
            cands = [i for i in range(self.first) if _layer_is_full(c, i) == full]
            src = l if l < self.first or not cands else cands[-1]
            d = dict(full=full, src=src,
                     hd=c["global_head_dim"] if full else c["head_dim"],
                     theta=c["rope_theta_full"] if full else c["rope_theta_sliding"])
            for k in ("input_layernorm", "post_attention_layernorm", "pre_feedforward_layernorm",
                      "post_feedforward_layernorm", "post_per_layer_input_norm"):
                d[k] = _bf(t[p + k + ".weight"])
            d["q_norm"] = _bf(t[p + "self_attn.q_norm.weight"])
            d["scalar"] = float(_bf(t[p + "layer_scalar"])[0])
            for k in ("self_attn.q_proj", "self_attn.o_proj", "mlp.gate_proj", "mlp.up_proj",
                      "mlp.down_proj", "per_layer_input_gate", "per_layer_projection"):
                d[k] = _dense(t, p + k + ".weight", quant)
            if src == l:
                d["k_norm"] = _bf(t[p + "self_attn.k_norm.weight"])
                d["self_attn.k_proj"] = _dense(t, p + "self_attn.k_proj.weight", quant)
                d["self_attn.v_proj"] = _dense(t, p + "self_attn.v_proj.weight", quant)
            self.layers.append(d)

    def forward(self, toks):
        """Logits [T, V] for every position of the sequence toks (positions 0..T-1)."""
        c = self.cfg
        toks = np.asarray(toks)
        T = len(toks)
        pos = np.arange(T)
        L, H, P, nq = self.L, self.H, self.P, self.nq
        e = self.E[toks] * np.sqrt(H)
        tok = (self.Eple[toks] * np.sqrt(P)).reshape(T, L, P)
        proj = _norm((e @ self.Wplmp.T * H ** -0.5).reshape(T, L, P), self.g_plpn)
        pli = (proj + tok) * 2.0 ** -0.5
        h = e.copy()
        kv = {}
        for l, d in enumerate(self.layers):
            hd = d["hd"]
            a = _norm(h, d["input_layernorm"])
            q = (a @ d["self_attn.q_proj"].T).reshape(T, nq, hd).transpose(1, 0, 2)
            q = _rope(_norm(q, d["q_norm"]), pos, d["theta"])
            if d["src"] == l:
                k = _rope(_norm(a @ d["self_attn.k_proj"].T, d["k_norm"]), pos, d["theta"])
                v = _norm(a @ d["self_attn.v_proj"].T)
                if self.kv_quant == "int8":
                    k, v = _int8_rows(k), _int8_rows(v)
                elif self.kv_bf16:
                    k, v = _round_bf16(k), _round_bf16(v)
                kv[l] = (k, v)
            k, v = kv[d["src"]]
            s = q @ k.T / np.sqrt(hd)                      # [nq, T, T]
            i, j = np.meshgrid(pos, pos, indexing="ij")
            allowed = j <= i
            if not d["full"]:
                allowed &= j > i - c["sliding_window"]
            s = np.where(allowed[None], s, -np.inf)
            w = np.exp(s - s.max(axis=-1, keepdims=True))
            w /= w.sum(axis=-1, keepdims=True)
            o = (w @ v).transpose(1, 0, 2).reshape(T, nq * hd)
            h = h + _norm(o @ d["self_attn.o_proj"].T, d["post_attention_layernorm"])
            m = _norm(h, d["pre_feedforward_layernorm"])
            f = (_gelu(m @ d["mlp.gate_proj"].T) * (m @ d["mlp.up_proj"].T)) @ d["mlp.down_proj"].T
            h = h + _norm(f, d["post_feedforward_layernorm"])
            r = _gelu(h @ d["per_layer_input_gate"].T) * pli[:, l, :]
            h = (h + _norm(r @ d["per_layer_projection"].T, d["post_per_layer_input_norm"])) * d["scalar"]
        y = _norm(h, self.g_f)
        return y @ self.E.T

    def greedy(self, prompt, steps):
        """Free-running greedy continuation; every step re-runs the whole sequence."""
        seq = list(prompt)
        out, all_logits = [], []
        for _ in range(steps):
            lg = self.forward(seq)[-1]
            nxt = int(np.argmax(lg))
            out.append(nxt)
            all_logits.append(lg)
            seq.append(nxt)
        return out, np.array(all_logits)
