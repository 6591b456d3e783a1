"""The allocation-free matrix-vector product (e2b_matvec_noalloc) against
e2b_matvec, through the C ABI: the same results bit for bit (both run the
same kernels with the same plan; only where the K-slice partials live
differs), on two calls in a row with the second smaller, for one row (the
matvec kernel) and for several rows (the matrix-core product)."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _weights(torch, dev, quant, N, K, seed):
    if quant == "bf16":
        w = synth.normal_bf16((N, K), seed, "w")
        return torch.from_numpy(w.view(np.int16)).to(dev), None
    w = synth.bits32((N, K // 8), seed, "w")
    s = synth.uniform_bf16((N, K // 32), seed, "s", 0.002, 0.02)
    return torch.from_numpy(w).to(dev), torch.from_numpy(s.view(np.int16)).to(dev)


@pytest.mark.parametrize("quant", ["bf16", "w4a16"])
@pytest.mark.parametrize("shapes", [[(1536, 12288, 64), (512, 6144, 3)], [(1536, 12288, 1), (256, 4096, 1)]],
                         ids=["rows", "one_row"])
def test_noalloc_matches_matvec(quant, shapes):
    import torch
    from w4a16_weight_streaming_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    L = binding.load_library()
    q = binding.QUANT[quant]
    stream = torch.cuda.current_stream(dev).cuda_stream
    for i, (N, K, rows) in enumerate(shapes):
        print(f"noalloc {quant} call {i}: N={N} K={K} rows={rows}", flush=True)
        w, s = _weights(torch, dev, quant, N, K, 40 + i)
        x = torch.from_numpy(np.random.default_rng(i).normal(size=(rows, K)).astype(np.float32)).to(dev)
        y_ref = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
        y = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
        binding.matvec(quant, w, s, x, y_ref)
        rc = L.e2b_matvec_noalloc(q, w.data_ptr(), 0 if s is None else s.data_ptr(), N, K, x.data_ptr(),
                                  rows, y.data_ptr(), stream)
        assert rc == binding.E2B_OK, L.e2b_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), float((y - y_ref).abs().max())


def test_noalloc_rejects_partials_beyond_the_scratch():
    """A product whose K-slice partials exceed the scratch is refused before
    anything is enqueued."""
    import torch
    from w4a16_weight_streaming_amd import binding
    dev = torch.device("cuda:0")
    L = binding.load_library()
    cap = L.e2b_matvec_noalloc_max_bytes()
    assert cap == 16 << 20
    # one row of K = 12,288 runs as 6 K slices: 6 x 1 x N x 4 B of partials,
    # 24 MB for N = 10^6 (the same plan e2b_matvec sizes its workspace by;
    # checked on the host first, so the call below can only be refused)
    N, K = 1_000_000, 12288
    need = L.e2b_matvec_workspace_bytes(0, N, K, 1)
    assert need == 6 * N * 4 and need > cap
    buf = torch.zeros(1 << 10, dtype=torch.float32, device=dev)
    p = buf.data_ptr()
    rc = L.e2b_matvec_noalloc(0, p, 0, N, K, p, 1, p, torch.cuda.current_stream(dev).cuda_stream)
    assert rc == binding.E2B_ENOMEM
    assert "scratch" in L.e2b_last_error().decode()
