"""KV-Kaizen compressed decode attention for MI355X (gfx950).

The compute lives in libkk.so (hand-written HIP kernels behind a C ABI, see
include/kk.h); this package is its ctypes binding plus the build script.
"""
from .kk import (KKError, Model, Decoder, LayerSpec, lib, row_stride_bytes, cache_bytes, out_offsets,  # noqa: F401
                 alloc_cache, quantize_write, workspace_bytes, status_string)
