"""KV-Kaizen compressed decode attention for MI355X (gfx950).

The compute lives in libkk.so (hand-written HIP kernels behind a C ABI, see
include/kk.h); this package is its ctypes binding plus the build script.
"""
from . import kk  # noqa: F401
from .kk import (KKError, Model, Decoder, MultiDecoder, GqaModel, GqaDecoder, gqa_alloc_cache,
                 gqa_quantize_write, LayerSpec, Cache, lib, row_stride_bytes, cache_bytes,  # noqa: F401
                 out_offsets, alloc_cache, quantize_write, workspace_bytes, plan_info, PlanInfo, latent_epilogue, status_string, LIB_PATH, KK_OK,
                 KK_ERR_INVALID_ARGUMENT, KK_ERR_UNSUPPORTED, KK_ERR_WORKSPACE_TOO_SMALL, KK_ERR_DEVICE,
                 KK_DTYPE_F32, KK_DTYPE_BF16, KK_NOALLOC_SCRATCH_BYTES)
