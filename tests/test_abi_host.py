"""C-ABI host logic on the CPU: the library loads, exports every declared
symbol, and its presets, K/V share map, byte totals and argument validation
agree with the pages.  No call here reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import golden
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from w4a16_weight_streaming_amd import binding, build
    if build.stale():
        build.build(force=True)
    return binding


def declared_functions():
    src = open(os.path.join(ROOT, "include", "e2b.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(e2b_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 15
    L = lib.load_library()
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("name", ["toy", "toy10", "e2b"])
def test_presets_match_workload_configs(lib, name):
    c = lib.config_preset(name).as_dict()
    want = synth.get_config(name)
    for k, v in c.items():
        if k in ("quant", "embed_quant", "kv_quant"):
            continue
        assert v == pytest.approx(want[k], rel=1e-6), k


def test_kv_share_map(lib):
    m = lib.Model(lib.config_preset("e2b"))
    assert m.kv_share_map() == golden.kv_share_map_e2b()
    assert lib.Model(lib.config_preset("toy")).kv_share_map() == [0, 1, 2, 2, 4]
    assert lib.Model(lib.config_preset("toy10")).kv_share_map() == [0, 1, 2, 3, 4, 3, 3, 3, 3, 4]


def test_kv_bytes_match_pages(lib):
    g = golden.kv("kv_bytes.txt")
    m = lib.Model(lib.config_preset("e2b"))
    assert m.kv_bytes(1, 1) == int(g["bytes_per_token"])
    assert m.kv_bytes(1, 256) == int(g["context_256"])
    assert m.kv_bytes(1, 1) != int(g["by_copy_cell"])
    assert m.kv_bytes(64, 640) == 64 * 640 * int(g["bytes_per_token"])


def _inventory_bytes(cfg, quant):
    tot = 0
    for s in synth.tensor_specs(cfg, kv_all_layers=False):
        n = int(np.prod(s.shape))
        tot += (n // 2 + 2 * (n // 32)) if (s.kind == "linear" and quant == "w4a16") else 2 * n
    return tot


def test_weight_bytes_match_pages(lib):
    g = golden.kv("weight_bytes.txt")
    b = lib.Model(lib.config_preset("e2b", "bf16")).weight_bytes()
    w = lib.Model(lib.config_preset("e2b", "w4a16")).weight_bytes()
    assert abs(b - int(g["bf16_total"])) / int(g["bf16_total"]) < 1e-4
    assert round(w / 1e9, 3) == float(g["w4a16_total_gb"])
    cfg = synth.get_config("e2b")
    assert b == _inventory_bytes(cfg, "bf16") and w == _inventory_bytes(cfg, "w4a16")
    m = lib.Model(lib.config_preset("e2b", "w4a16"))
    assert m.arena_bytes() >= m.weight_bytes()
    assert m.workspace_bytes(1) > 0 and m.workspace_bytes(64) > m.workspace_bytes(1)


@pytest.mark.parametrize("field,value", [
    ("num_key_value_heads", 2), ("head_dim", 96), ("global_head_dim", 1024),
    ("num_kv_shared_layers", 35), ("group_size", 64), ("hidden_size", 1000),
    ("intermediate_size", 100), ("num_attention_heads", 9), ("quant", 7)])
def test_create_rejects_bad_configs(lib, field, value):
    c = lib.config_preset("e2b")
    setattr(c, field, value)
    with pytest.raises(lib.E2BError) as e:
        lib.Model(c)
    assert e.value.code == lib.E2B_EINVAL


def test_unknown_preset(lib):
    with pytest.raises(lib.E2BError):
        lib.config_preset("e4b")


def _load(lib, model, tensors):
    table, keep = lib._tensor_table(tensors)
    L = lib.load_library()
    # a non-null, aligned but unmapped arena: every case here fails validation
    # before any device call is made
    rc = L.e2b_load_weights(model.handle, table, len(tensors), 1 << 20, model.arena_bytes(), None)
    return rc, L.e2b_last_error().decode()


def test_load_validation_errors(lib):
    cfg = synth.get_config("toy")
    w = synth.generate(cfg, "w4a16")
    m = lib.Model(lib.config_from_dict(cfg, "w4a16"))
    bad = dict(w)
    del bad["model.layers.2.mlp.down_proj.weight_scale"]
    rc, msg = _load(lib, m, bad)
    assert rc == lib.E2B_EINVAL and "model.layers.2.mlp.down_proj.weight_scale" in msg
    bad = dict(w)
    bad["model.layers.0.self_attn.q_proj.weight_packed"] = np.zeros((128, 8), np.int32)
    rc, msg = _load(lib, m, bad)
    assert rc == lib.E2B_EINVAL and "q_proj" in msg
    bad = dict(w)
    bad["lm_head.weight"] = w["model.embed_tokens.weight"]
    rc, msg = _load(lib, m, bad)
    assert rc == lib.E2B_EINVAL and "lm_head.weight" in msg
    bf = synth.generate(cfg, "bf16")
    rc, msg = _load(lib, m, bf)      # bf16 tensors for a W4A16 model
    assert rc == lib.E2B_EINVAL
    rc, msg = _load(lib, m, w)       # valid table, too-small arena
    L = lib.load_library()
    table, keep = lib._tensor_table(w)
    assert L.e2b_load_weights(m.handle, table, len(w), 1 << 20, 16, None) == lib.E2B_ENOMEM


def test_calls_before_load_are_refused(lib):
    m = lib.Model(lib.config_preset("toy"))
    L = lib.load_library()
    rc = L.e2b_decode_step(m.handle, 256, 256, 1, None, 256, 256, 1 << 30, None)
    assert rc == lib.E2B_ESTATE
    assert L.e2b_kv_alloc(m.handle, 256, 10, 1, 16) == lib.E2B_ENOMEM


def test_matvec_validation(lib):
    L = lib.load_library()
    assert L.e2b_matvec(0, 256, None, 8, 100, 256, 1, 256, None, 0, None) == lib.E2B_EINVAL
    assert L.e2b_matvec(1, 256, None, 8, 1536, 256, 1, 256, None, 0, None) == lib.E2B_EINVAL
    assert L.e2b_matvec_workspace_bytes(0, 1536, 12288, 1) == 6 * 1536 * 4   # six 2048-wide slices
    assert L.e2b_matvec_workspace_bytes(0, 1536, 1536, 1) == 0
    # widths with no matvec instantiation are refused by both paths
    for K in (64, 96, 160, 480, 4608 * 4):
        assert L.e2b_matvec_workspace_bytes(0, 64, K, 3) == 0, K
        assert L.e2b_matvec(0, 256, None, 8, K, 256, 3, 256, 256, 1 << 20, None) == lib.E2B_EINVAL, K
    # several rows: the K-slice partials of the matrix-core product, then (N %
    # 16 == 0, and for W4A16 K % 128 == 0) the weights tiled in fragment order
    up = lambda x: (x + 255) // 256 * 256
    for quant in (0, 1):
        for N, K, r in ((1536, 1536, 3), (1536, 12288, 70), (1536, 4096, 2), (24576, 1536, 64),
                        (40, 1536, 3)):
            total = L.e2b_matvec_workspace_bytes(quant, N, K, r)
            tiled = 0
            if N % 16 == 0 and (not quant or K % 128 == 0):
                tiled = up(N * K // 2) + up(N * (K // 32) * 2) if quant else up(N * K * 2)
            part = total - tiled
            slices = part // (r * N * 4)
            assert part >= 0 and slices in (0, 2, 3, 4, 6, 8, 12, 16), (quant, N, K, r, total)
            assert part == (up(slices * r * N * 4) if slices else 0), (quant, N, K, r, total)
            if slices:
                assert K % slices == 0 and (K // slices) % 32 == 0
    assert L.e2b_matvec_workspace_bytes(2, 1536, 1536, 3) == 0   # unknown quant


def test_paged_cache_sizes_and_state(lib):
    """Paged pool bytes: (n_pages + 1) pages of 128 rows per K/V-owning layer
    (the last a spare), bf16 or int8 rows; the allocator calls refuse a
    contiguous cache."""
    L = lib.load_library()
    m = lib.Model(lib.config_preset("e2b"))
    per_token = m.kv_bytes(1, 1)
    assert L.e2b_kv_paged_bytes(m.handle, 10) == 11 * 128 * per_token
    assert L.e2b_kv_paged_bytes(m.handle, 0) == 0
    assert L.e2b_seq_reserve(m.handle, 0, 10, None) == lib.E2B_ESTATE
    assert L.e2b_seq_release(m.handle, 0, None) == lib.E2B_ESTATE
    assert L.e2b_pages_free(m.handle) == 0
    m8 = lib.Model(lib.config_preset("e2b", kv_quant="int8"))
    rows = 11 * 128
    up = lambda x: (x + 255) // 256 * 256
    want = sum(2 * (rows * hd + up(rows * 4)) for hd in [256] * 12 + [512] * 3)
    assert L.e2b_kv_paged_bytes(m8.handle, 10) == want
