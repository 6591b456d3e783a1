"""Compile libe2b.so (HIP kernels + C ABI host code) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libe2b.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "attn_prefill.hip", "gemm_bf16.hip", "gemm_w4.hip", "host.cpp")]
HEADERS = [os.path.join(CSRC, "e2b_internal.h"), os.path.join(CSRC, "dev_common.h"),
           os.path.join(CSRC, "gemm_impl.h"),
           os.path.join(ROOT, "include", "e2b.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fuse only the multiply-adds the source writes out (fmaf): the same
    # expression then rounds the same way in every kernel it is inlined into
    "-ffp-contract=off",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source into libe2b.so (always when force): the sources in
    parallel to objects under _build/, then one link."""
    if not force and not stale():
        return LIB
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + "." + tag + ".o")
        r = subprocess.run([hipcc] + HIPCC_FLAGS + ["-c", src, "-o", obj], capture_output=True, text=True)
        return obj, r

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    msgs = []
    for obj, r in results:
        msgs += [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    tmp = LIB + ".tmp" + tag
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-o", tmp] + [o for o, _ in results],
                       capture_output=True, text=True)
    for o, _ in results:
        os.remove(o)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
