"""MI355X-native decode step of a Gemma-4-E2B-shaped decoder (bf16 and W4A16).

The compute path is libe2b.so: hand-written HIP kernels for gfx950 behind a C
ABI (include/e2b.h).  This package only marshals arguments to it; PyTorch
provides device memory and the stream.  There is no CPU or fallback path: if
the library is missing or no gfx950 device is present the calls raise.
"""
from .binding import E2BError, Engine, config_preset, lib_path, load_library, matvec  # noqa: F401
