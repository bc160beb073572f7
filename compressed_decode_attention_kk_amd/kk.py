"""ctypes binding of libkk.so (the C ABI declared in include/kk.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the decode path runs in the library's
kernels.  The binding fails loudly when the library is missing.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkk.so")

KK_OK, KK_ERR_INVALID_ARGUMENT, KK_ERR_UNSUPPORTED, KK_ERR_WORKSPACE_TOO_SMALL, KK_ERR_DEVICE = range(5)
KK_DTYPE_F32, KK_DTYPE_BF16 = 0, 1
KK_NOALLOC_SCRATCH_BYTES = 256 << 20      # size of the array behind kk_decode_attn_noalloc


class KKError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class LayerCfg(ctypes.Structure):
    _fields_ = [("anchor", ctypes.c_int32), ("d", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class ModelCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("r", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("layers", ctypes.POINTER(LayerCfg))]


class Cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_cus", ctypes.c_int32), ("work_items", ctypes.c_int32), ("merge_blocks", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class GqaCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("layers", ctypes.POINTER(LayerCfg))]


class TableBatch(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(ModelCfg)), ("batch", ctypes.c_int32), ("caches", ctypes.POINTER(Cache))]


_lib = None


def lib():
    """Load libkk.so (built by compressed_decode_attention_kk_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m compressed_decode_attention_kk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kk_row_stride_bytes.restype = ctypes.c_size_t
        L.kk_row_stride_bytes.argtypes = [ctypes.c_int32] * 3
        L.kk_validate_model.argtypes = [ctypes.POINTER(ModelCfg)]
        L.kk_cache_bytes.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.kk_out_offsets.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.kk_quantize_write.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, Cache, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]
        L.kk_decode_workspace_bytes.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.kk_decode_plan_info.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(PlanInfo)]
        L.kk_decode_attn.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(Cache), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
        L.kk_decode_attn_noalloc.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(Cache), ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_void_p]
        L.kk_append_decode.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(Cache), ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        L.kk_multi_out_offsets.argtypes = [ctypes.POINTER(TableBatch), ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.kk_multi_decode_workspace_bytes.argtypes = [ctypes.POINTER(TableBatch), ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.kk_multi_decode_attn.argtypes = [ctypes.POINTER(TableBatch), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
        L.kk_latent_epilogue.argtypes = [ctypes.POINTER(ModelCfg), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.kk_gqa_cache_bytes.argtypes = [ctypes.POINTER(GqaCfg), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.kk_gqa_quantize_write.argtypes = [ctypes.POINTER(GqaCfg), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, Cache, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.kk_gqa_decode_workspace_bytes.argtypes = [ctypes.POINTER(GqaCfg), ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.kk_gqa_decode_attn.argtypes = [ctypes.POINTER(GqaCfg), ctypes.POINTER(Cache), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
        L.kk_status_string.restype = ctypes.c_char_p
        L.kk_status_string.argtypes = [ctypes.c_int]
        for name in ("kk_validate_model", "kk_cache_bytes", "kk_out_offsets", "kk_quantize_write",
                     "kk_decode_workspace_bytes", "kk_decode_plan_info", "kk_decode_attn", "kk_decode_attn_noalloc",
                     "kk_append_decode", "kk_multi_out_offsets",
                     "kk_multi_decode_workspace_bytes", "kk_multi_decode_attn", "kk_latent_epilogue",
                     "kk_gqa_cache_bytes", "kk_gqa_quantize_write", "kk_gqa_decode_workspace_bytes",
                     "kk_gqa_decode_attn"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kk_status_string(status).decode()


def _check(status: int, what: str):
    if status != KK_OK:
        raise KKError(status, what)


def _require(cond, what: str):
    """Argument check of the binding.  The library checks scalars and pointers
    itself but cannot see tensor extents, so these checks guard its kernels
    against short buffers; unlike assert they stay active under python -O."""
    if not cond:
        raise ValueError(what)


def _tensor(t, name: str, dtype=None, contiguous=True):
    _require(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a device tensor")
    if dtype is not None:
        _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if contiguous:
        _require(t.is_contiguous(), f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return KK_DTYPE_F32
    if dt == torch.bfloat16:
        return KK_DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}")


@dataclass
class LayerSpec:
    anchor: int
    d: int
    bits: int
    sm_scale: float


class Model:
    """Per-layer table + shape (a kk_model_cfg)."""

    def __init__(self, layers, n_heads: int, r: int, d_rope: int):
        self.layers = [LayerSpec(int(l.anchor), int(l.d), int(l.bits), float(l.sm_scale)) for l in layers]
        self.n_layers, self.n_heads, self.r, self.d_rope = len(self.layers), int(n_heads), int(r), int(d_rope)
        self._arr = (LayerCfg * self.n_layers)(*[LayerCfg(l.anchor, l.d, l.bits, l.sm_scale) for l in self.layers])
        self._cfg = ModelCfg(self.n_layers, self.n_heads, self.r, self.d_rope, self._arr)

    @property
    def cfg(self):
        return ctypes.byref(self._cfg)

    def anchors(self):
        return [l for l, s in enumerate(self.layers) if s.anchor == l]

    def d_eff(self, l):
        return self.layers[self.layers[l].anchor].d

    def validate(self):
        _check(lib().kk_validate_model(self.cfg), "kk_validate_model")


def row_stride_bytes(d: int, d_rope: int, bits: int) -> int:
    return int(lib().kk_row_stride_bytes(d, d_rope, bits))


def cache_bytes(model: Model, layer: int, batch: int, t_cap: int):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kk_cache_bytes(model.cfg, layer, batch, t_cap, ctypes.byref(cb), ctypes.byref(sb)), "kk_cache_bytes")
    return cb.value, sb.value


def out_offsets(model: Model, batch: int):
    arr = (ctypes.c_int64 * (model.n_layers + 1))()
    _check(lib().kk_out_offsets(model.cfg, batch, arr), "kk_out_offsets")
    return list(arr)


def _check_cache(model: Model, layer: int, codes: torch.Tensor, scales: torch.Tensor, batch: int, t_cap: int):
    """codes / scales are large enough for anchor `layer`'s cache of [batch][t_cap]."""
    cb, sb = cache_bytes(model, layer, batch, t_cap)
    _tensor(codes, f"codes of layer {layer}", torch.uint8)
    _tensor(scales, f"scales of layer {layer}", torch.float32)
    _require(codes.numel() >= cb and scales.numel() * 4 >= sb,
             f"cache of layer {layer} must hold {cb} code bytes and {sb // 4} scales for batch {batch}, t_cap {t_cap}")


def _cache_table(model: Model, caches: dict, batch: int, t_cap: int):
    """kk_cache[n_layers] of the anchors' buffers (entries of inheritors stay NULL)."""
    tab = (Cache * model.n_layers)()
    for l in model.anchors():
        _require(l in caches, f"no cache for anchor layer {l}")
        c, s = caches[l]
        _check_cache(model, l, c, s, batch, t_cap)
        tab[l] = Cache(c.data_ptr(), s.data_ptr())
    return tab


def alloc_cache(model: Model, layer: int, batch: int, t_cap: int, device="cuda"):
    """Device buffers of one anchor cache: (codes uint8 [B, T_cap, stride], scales f32 [B, T_cap])."""
    cb, _ = cache_bytes(model, layer, batch, t_cap)
    stride = cb // (batch * t_cap)
    codes = torch.empty((batch, t_cap, stride), dtype=torch.uint8, device=device)
    scales = torch.empty((batch, t_cap), dtype=torch.float32, device=device)
    return codes, scales


def quantize_write(model: Model, layer: int, latent: torch.Tensor, rope: torch.Tensor, codes: torch.Tensor,
                   scales: torch.Tensor, dst_slot: torch.Tensor, src_index: torch.Tensor | None = None,
                   stream=None):
    """Quantize source rows latent [n_src, >= d] / rope [n_src, d_R] into anchor `layer`'s cache.

    dst_slot: int64 [n_tokens] (seq * t_cap + position); src_index: int32 [n_tokens] or None.
    codes/scales: the anchor's cache buffers [B, T_cap, stride] / [B, T_cap].
    """
    _tensor(latent, "latent", contiguous=False)
    _tensor(rope, "rope", latent.dtype, contiguous=False)
    _require(latent.dim() == 2 and rope.dim() == 2 and latent.stride(1) == 1 and rope.stride(1) == 1,
             "latent and rope must be 2-D with unit column stride")
    _require(rope.shape[0] == latent.shape[0], "latent and rope must have the same number of rows")
    _require(latent.shape[1] >= model.d_eff(layer) and rope.shape[1] >= model.d_rope,
             "latent needs >= d columns and rope >= d_rope columns")
    _tensor(dst_slot, "dst_slot", torch.int64)
    _tensor(scales, "scales", torch.float32)
    _require(scales.dim() == 2, "scales must be [batch, t_cap]")
    batch, t_cap = scales.shape
    _check_cache(model, layer, codes, scales, batch, t_cap)
    if src_index is not None:
        _tensor(src_index, "src_index", torch.int32)
        _require(src_index.numel() == dst_slot.numel(), "src_index and dst_slot must have one entry per token")
    st = lib().kk_quantize_write(model.cfg, layer, _ptr(latent), _ptr(rope), _dtype_code(latent.dtype),
                                 latent.stride(0), rope.stride(0), latent.shape[0], dst_slot.numel(),
                                 _ptr(src_index), _ptr(dst_slot), Cache(codes.data_ptr(), scales.data_ptr()),
                                 batch, t_cap, _stream(stream))
    _check(st, "kk_quantize_write")


def workspace_bytes(model: Model, batch: int, max_seq_len: int, split_tokens: int = 0) -> int:
    b = ctypes.c_size_t()
    _check(lib().kk_decode_workspace_bytes(model.cfg, batch, max_seq_len, split_tokens, ctypes.byref(b)),
           "kk_decode_workspace_bytes")
    return b.value


def plan_info(model: Model, batch: int, max_seq_len: int, split_tokens: int = 0, n_cus: int = 0) -> PlanInfo:
    """The decode step's work plan for n_cus compute units (0: the current device's)."""
    info = PlanInfo()
    _check(lib().kk_decode_plan_info(model.cfg, batch, max_seq_len, split_tokens, n_cus, ctypes.byref(info)),
           "kk_decode_plan_info")
    return info


class Decoder:
    """Holds the cache pointer table, output and workspace for repeated decode steps."""

    def __init__(self, model: Model, caches: dict, batch: int, t_cap: int, max_seq_len: int,
                 split_tokens: int = 0, device="cuda"):
        self.model, self.batch, self.t_cap, self.max_seq_len = model, batch, t_cap, max_seq_len
        self.split_tokens = split_tokens
        self.caches = caches
        self._ctab = _cache_table(model, caches, batch, t_cap)
        offs = out_offsets(model, batch)
        self.offsets = offs
        self.out = torch.empty(offs[-1], dtype=torch.float32, device=device)
        wb = workspace_bytes(model, batch, max_seq_len, split_tokens)
        self.workspace = _workspace(wb, device)
        self.ws_bytes = wb

    def __call__(self, q_lat: torch.Tensor, q_rope: torch.Tensor, seq_lens: torch.Tensor, stream=None):
        m = self.model
        _check_queries(q_lat, q_rope, m.n_layers, self.batch, m.n_heads, m.r, m.d_rope)
        _check_lens(seq_lens, self.batch)
        ws = self.workspace
        wptr = (ws.data_ptr() + 255) // 256 * 256
        st = lib().kk_decode_attn(m.cfg, self._ctab, self.batch, self.t_cap, _ptr(seq_lens), self.max_seq_len,
                                  _ptr(q_lat), _ptr(q_rope), _dtype_code(q_lat.dtype), _ptr(self.out),
                                  self.split_tokens, ctypes.c_void_p(wptr), self.ws_bytes, _stream(stream))
        _check(st, "kk_decode_attn")
        return self.out

    def noalloc(self, q_lat: torch.Tensor, q_rope: torch.Tensor, seq_lens: torch.Tensor, stream=None):
        """kk_decode_attn_noalloc: the same step with the split partials in the
        library's static device array (this object's workspace is not used)."""
        m = self.model
        _check_queries(q_lat, q_rope, m.n_layers, self.batch, m.n_heads, m.r, m.d_rope)
        _check_lens(seq_lens, self.batch)
        st = lib().kk_decode_attn_noalloc(m.cfg, self._ctab, self.batch, self.t_cap, _ptr(seq_lens),
                                          self.max_seq_len, _ptr(q_lat), _ptr(q_rope), _dtype_code(q_lat.dtype),
                                          _ptr(self.out), self.split_tokens, _stream(stream))
        _check(st, "kk_decode_attn_noalloc")
        return self.out

    def append(self, new_latent: torch.Tensor, new_rope: torch.Tensor, q_lat: torch.Tensor, q_rope: torch.Tensor,
               seq_lens: torch.Tensor, stream=None):
        """kk_append_decode: write each sequence's new token (row seq_lens[s] - 1) into
        every anchor cache, then decode over the extended caches.  new_latent
        [n_layers, batch, r] and new_rope [n_layers, batch, d_rope], one dtype."""
        m = self.model
        _tensor(new_latent, "new_latent")
        _tensor(new_rope, "new_rope", new_latent.dtype)
        _require(tuple(new_latent.shape) == (m.n_layers, self.batch, m.r), "new_latent must be [n_layers, batch, r]")
        _require(tuple(new_rope.shape) == (m.n_layers, self.batch, m.d_rope),
                 "new_rope must be [n_layers, batch, d_rope]")
        _check_queries(q_lat, q_rope, m.n_layers, self.batch, m.n_heads, m.r, m.d_rope)
        _check_lens(seq_lens, self.batch)
        wptr = (self.workspace.data_ptr() + 255) // 256 * 256
        st = lib().kk_append_decode(m.cfg, self._ctab, self.batch, self.t_cap, _ptr(seq_lens), self.max_seq_len,
                                    _ptr(new_latent), _ptr(new_rope), _dtype_code(new_latent.dtype),
                                    _ptr(q_lat), _ptr(q_rope), _dtype_code(q_lat.dtype), _ptr(self.out),
                                    self.split_tokens, ctypes.c_void_p(wptr), self.ws_bytes, _stream(stream))
        _check(st, "kk_append_decode")
        return self.out

    def layer_out(self, l: int) -> torch.Tensor:
        """View of layer l's output [B, H, d_eff]."""
        m = self.model
        return self.out[self.offsets[l]:self.offsets[l + 1]].view(self.batch, m.n_heads, m.d_eff(l))


def _workspace(nbytes: int, device):
    """Device buffer of >= nbytes from a 256-byte aligned address (see the callers' wptr)."""
    return torch.empty((max(nbytes, 256) + 3) // 4 + 64, dtype=torch.float32, device=device)


def _check_queries(q_lat, q_rope, n_layers, batch, n_heads, r, d_rope):
    _tensor(q_lat, "q_lat")
    _tensor(q_rope, "q_rope", q_lat.dtype)
    _require(tuple(q_lat.shape) == (n_layers, batch, n_heads, r), "q_lat must be [n_layers, batch, n_heads, r]")
    _require(tuple(q_rope.shape) == (n_layers, batch, n_heads, d_rope),
             "q_rope must be [n_layers, batch, n_heads, d_rope]")


def _check_lens(seq_lens, batch):
    _tensor(seq_lens, "seq_lens", torch.int32)
    _require(seq_lens.numel() == batch, f"seq_lens must have {batch} entries")


class MultiDecoder:
    """kk_multi_decode_attn: one decode step over a batch whose runs of
    sequences use different tables.  runs: list of (Model, caches, batch); the
    runs' sequences follow one another in the batch, in list order."""

    def __init__(self, runs, t_cap: int, max_seq_len: int, split_tokens: int = 0, device="cuda"):
        self.runs = list(runs)
        self.models = [m for m, _, _ in self.runs]
        m0 = self.models[0]
        self.n_layers, self.n_heads, self.r, self.d_rope = m0.n_layers, m0.n_heads, m0.r, m0.d_rope
        self.batches = [int(b) for _, _, b in self.runs]
        self.batch = sum(self.batches)
        self.t_cap, self.max_seq_len, self.split_tokens = t_cap, max_seq_len, split_tokens
        self._ctabs = [_cache_table(m, c, b, t_cap) if c is not None else None for m, c, b in self.runs]
        self._tabs = (TableBatch * len(self.runs))(*[
            TableBatch(ctypes.pointer(m._cfg), b, ctab if ctab is not None else None)
            for (m, _, b), ctab in zip(self.runs, self._ctabs)])
        n = len(self.runs)
        offs = (ctypes.c_int64 * (n * self.n_layers + 1))()
        _check(lib().kk_multi_out_offsets(self._tabs, n, offs), "kk_multi_out_offsets")
        self.offsets = list(offs)
        self.out = torch.empty(self.offsets[-1], dtype=torch.float32, device=device)
        wb = ctypes.c_size_t()
        _check(lib().kk_multi_decode_workspace_bytes(self._tabs, n, max_seq_len, split_tokens, ctypes.byref(wb)),
               "kk_multi_decode_workspace_bytes")
        self.ws_bytes = wb.value
        self.workspace = _workspace(self.ws_bytes, device)

    def __call__(self, q_lat: torch.Tensor, q_rope: torch.Tensor, seq_lens: torch.Tensor, stream=None):
        _require(all(c is not None for c in self._ctabs), "every run needs its caches to decode")
        _check_queries(q_lat, q_rope, self.n_layers, self.batch, self.n_heads, self.r, self.d_rope)
        _check_lens(seq_lens, self.batch)
        wptr = (self.workspace.data_ptr() + 255) // 256 * 256
        st = lib().kk_multi_decode_attn(self._tabs, len(self.runs), self.t_cap, _ptr(seq_lens), self.max_seq_len,
                                        _ptr(q_lat), _ptr(q_rope), _dtype_code(q_lat.dtype), _ptr(self.out),
                                        self.split_tokens, ctypes.c_void_p(wptr), self.ws_bytes, _stream(stream))
        _check(st, "kk_multi_decode_attn")
        return self.out

    def layer_out(self, run: int, l: int) -> torch.Tensor:
        """View of run `run`'s layer l output [batch_run, H, d_eff]."""
        k = run * self.n_layers + l
        return self.out[self.offsets[k]:self.offsets[k + 1]].view(self.batches[run], self.n_heads,
                                                                   self.models[run].d_eff(l))


def latent_epilogue(model: Model, batch: int, o_lat: torch.Tensor, w_uv, w_o, v: torch.Tensor, y: torch.Tensor,
                    stream=None):
    """kk_latent_epilogue: per-head value up-projection (W_UV on the kept
    latent coordinates) and output projection W_O for every layer.

    o_lat: the decode output (packed float32); w_uv: per layer bf16
    [n_heads * d_v, r]; w_o: per layer bf16 [d_model, n_heads * d_v];
    v: float32 [n_layers, batch, n_heads * d_v]; y: float32 [n_layers, batch, d_model].
    """
    L = model.n_layers
    _require(len(w_uv) == L and len(w_o) == L, "one W_UV and one W_O per layer")
    _tensor(w_o[0], "w_o[0]", torch.bfloat16)
    _require(w_o[0].dim() == 2 and w_o[0].shape[1] % model.n_heads == 0, "w_o must be [d_model, n_heads * d_v]")
    d_model, hv = w_o[0].shape
    d_v = hv // model.n_heads
    for l, (a, b) in enumerate(zip(w_uv, w_o)):
        _tensor(a, f"w_uv[{l}]", torch.bfloat16)
        _tensor(b, f"w_o[{l}]", torch.bfloat16)
        _require(tuple(a.shape) == (hv, model.r) and tuple(b.shape) == (d_model, hv),
                 f"layer {l}: w_uv must be [n_heads * d_v, r] and w_o [d_model, n_heads * d_v]")
    _tensor(o_lat, "o_lat", torch.float32)
    _require(o_lat.numel() == out_offsets(model, batch)[-1], "o_lat must be the packed decode output")
    _tensor(v, "v", torch.float32)
    _tensor(y, "y", torch.float32)
    _require(tuple(v.shape) == (L, batch, hv), "v must be [n_layers, batch, n_heads * d_v]")
    _require(tuple(y.shape) == (L, batch, d_model), "y must be [n_layers, batch, d_model]")
    pu = (ctypes.c_void_p * L)(*[t.data_ptr() for t in w_uv])
    po = (ctypes.c_void_p * L)(*[t.data_ptr() for t in w_o])
    st = lib().kk_latent_epilogue(model.cfg, batch, d_v, d_model, _ptr(o_lat), pu, po, _ptr(v), _ptr(y),
                                  _stream(stream))
    _check(st, "kk_latent_epilogue")
    return v, y


class GqaModel:
    """Per-layer table of a grouped-query model (a kk_gqa_cfg): precision and
    depth; each anchor caches all d_head key and value coordinates."""

    def __init__(self, layers, n_q_heads: int, n_kv_heads: int, d_head: int):
        self.layers = [LayerSpec(int(l.anchor), int(l.d), int(l.bits), float(l.sm_scale)) for l in layers]
        self.n_layers, self.n_q_heads, self.n_kv_heads, self.d_head = (len(self.layers), int(n_q_heads),
                                                                        int(n_kv_heads), int(d_head))
        self._arr = (LayerCfg * self.n_layers)(*[LayerCfg(l.anchor, l.d, l.bits, l.sm_scale) for l in self.layers])
        self._cfg = GqaCfg(self.n_layers, self.n_q_heads, self.n_kv_heads, self.d_head, self._arr)

    @property
    def cfg(self):
        return ctypes.byref(self._cfg)

    def anchors(self):
        return [l for l, s in enumerate(self.layers) if s.anchor == l]


def _check_gqa_cache(model: GqaModel, layer: int, codes, scales, batch: int, t_cap: int):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kk_gqa_cache_bytes(model.cfg, layer, batch, t_cap, ctypes.byref(cb), ctypes.byref(sb)),
           "kk_gqa_cache_bytes")
    _tensor(codes, f"codes of layer {layer}", torch.uint8)
    _tensor(scales, f"scales of layer {layer}", torch.float32)
    _require(codes.numel() >= cb.value and scales.numel() * 4 >= sb.value,
             f"cache of layer {layer} must hold {cb.value} code bytes and {sb.value // 4} scales")


def gqa_alloc_cache(model: GqaModel, layer: int, batch: int, t_cap: int, device="cuda"):
    """(codes uint8 [B, n_kv, T_cap, stride], scales f32 [B, n_kv, T_cap]) of one anchor."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kk_gqa_cache_bytes(model.cfg, layer, batch, t_cap, ctypes.byref(cb), ctypes.byref(sb)),
           "kk_gqa_cache_bytes")
    rows = batch * model.n_kv_heads * t_cap
    codes = torch.empty((batch, model.n_kv_heads, t_cap, cb.value // rows), dtype=torch.uint8, device=device)
    scales = torch.empty((batch, model.n_kv_heads, t_cap), dtype=torch.float32, device=device)
    return codes, scales


def gqa_quantize_write(model: GqaModel, layer: int, k: torch.Tensor, v: torch.Tensor, codes: torch.Tensor,
                       scales: torch.Tensor, dst_slot: torch.Tensor, src_index: torch.Tensor | None = None,
                       stream=None):
    """Quantize K and V source rows [n_src, n_kv, d_head] into anchor `layer` at
    slots dst_slot (seq * t_cap + position, int64)."""
    _tensor(k, "k")
    _tensor(v, "v", k.dtype)
    _require(k.shape == v.shape and k.dim() == 3 and tuple(k.shape[1:]) == (model.n_kv_heads, model.d_head),
             "k and v must be [n_src, n_kv_heads, d_head]")
    _tensor(dst_slot, "dst_slot", torch.int64)
    if src_index is not None:
        _tensor(src_index, "src_index", torch.int32)
        _require(src_index.numel() == dst_slot.numel(), "src_index and dst_slot must have one entry per token")
    _tensor(scales, "scales", torch.float32)
    _require(scales.dim() == 3 and scales.shape[1] == model.n_kv_heads, "scales must be [batch, n_kv_heads, t_cap]")
    batch, _, t_cap = scales.shape
    _check_gqa_cache(model, layer, codes, scales, batch, t_cap)
    st = lib().kk_gqa_quantize_write(model.cfg, layer, _ptr(k), _ptr(v), _dtype_code(k.dtype), k.shape[0],
                                     dst_slot.numel(), _ptr(src_index), _ptr(dst_slot),
                                     Cache(codes.data_ptr(), scales.data_ptr()), batch, t_cap, _stream(stream))
    _check(st, "kk_gqa_quantize_write")


class GqaDecoder:
    """kk_gqa_decode_attn for repeated steps: out [n_layers, batch, n_q_heads, d_head]."""

    def __init__(self, model: GqaModel, caches: dict, batch: int, t_cap: int, max_seq_len: int,
                 split_tokens: int = 0, device="cuda"):
        self.model, self.batch, self.t_cap, self.max_seq_len = model, batch, t_cap, max_seq_len
        self.split_tokens = split_tokens
        self.caches = caches
        self._ctab = (Cache * model.n_layers)()
        for l in model.anchors():
            _require(l in caches, f"no cache for anchor layer {l}")
            c, s = caches[l]
            _check_gqa_cache(model, l, c, s, batch, t_cap)
            self._ctab[l] = Cache(c.data_ptr(), s.data_ptr())
        self.out = torch.empty(model.n_layers, batch, model.n_q_heads, model.d_head, dtype=torch.float32,
                               device=device)
        wb = ctypes.c_size_t()
        _check(lib().kk_gqa_decode_workspace_bytes(model.cfg, batch, max_seq_len, split_tokens, ctypes.byref(wb)),
               "kk_gqa_decode_workspace_bytes")
        self.ws_bytes = wb.value
        self.workspace = _workspace(self.ws_bytes, device)

    def __call__(self, q: torch.Tensor, seq_lens: torch.Tensor, stream=None):
        m = self.model
        _tensor(q, "q")
        _require(tuple(q.shape) == (m.n_layers, self.batch, m.n_q_heads, m.d_head),
                 "q must be [n_layers, batch, n_q_heads, d_head]")
        _check_lens(seq_lens, self.batch)
        wptr = (self.workspace.data_ptr() + 255) // 256 * 256
        st = lib().kk_gqa_decode_attn(m.cfg, self._ctab, self.batch, self.t_cap, _ptr(seq_lens), self.max_seq_len,
                                      _ptr(q), _dtype_code(q.dtype), _ptr(self.out), self.split_tokens,
                                      ctypes.c_void_p(wptr), self.ws_bytes, _stream(stream))
        _check(st, "kk_gqa_decode_attn")
        return self.out
