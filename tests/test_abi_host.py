"""The C ABI on the host: the library loads, exports every function that
include/kk.h declares, and its host-only calls (sizes, offsets, table
validation, argument checks that reject a call before anything is enqueued)
behave as documented.  No call here reaches a kernel launch, so no GPU is
needed."""

import ctypes
import math
import os
import re

import pytest

from oracle import kk_oracle as ko

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kk.h")


@pytest.fixture(scope="module")
def kk():
    import compressed_decode_attention_kk_amd as kk
    alt = os.environ.get("KK_HOST_TEST_LIB")
    if alt:
        # the host-only sanitizer build (see test_host_sanitizers.py)
        kk.kk._lib = None
        kk.kk.LIB_PATH = kk.LIB_PATH = alt
    kk.lib()
    return kk


def test_report_library(kk):
    print("sanitized build" if os.environ.get("KK_HOST_TEST_LIB") else "library", kk.LIB_PATH)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(kk_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kk_quantize_write", "kk_decode_attn", "kk_decode_workspace_bytes", "kk_cache_bytes",
              "kk_out_offsets", "kk_validate_model", "kk_row_stride_bytes", "kk_status_string",
              "kk_append_decode", "kk_multi_out_offsets", "kk_multi_decode_workspace_bytes",
              "kk_multi_decode_attn", "kk_latent_epilogue", "kk_gqa_cache_bytes", "kk_gqa_quantize_write",
              "kk_gqa_decode_workspace_bytes", "kk_gqa_decode_attn", "kk_decode_plan_info"):
        assert n in names


def test_noalloc_scratch_size_matches_header(kk):
    import re
    hdr = open(os.path.join(ROOT, "include", "kk.h")).read()
    m = re.search(r"#define KK_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m, "KK_NOALLOC_SCRATCH_BYTES not found in kk.h"
    assert int(m.group(1)) << int(m.group(2)) == kk.KK_NOALLOC_SCRATCH_BYTES


def test_library_exports_every_declared_function(kk):
    L = ctypes.CDLL(kk.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, f"declared in kk.h but not exported: {missing}"


def test_missing_library_fails_loudly(kk, monkeypatch):
    monkeypatch.setattr(kk.kk, "_lib", None)
    monkeypatch.setattr(kk.kk, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libkk.so"))
    with pytest.raises(ImportError):
        kk.kk.lib()


def test_binding_refuses_host_tensors(kk):
    """The binding takes device tensors only: a host tensor is refused with
    ValueError before anything reaches the library (no CPU path)."""
    import torch
    m = kk.Model([kk.LayerSpec(0, 64, 8, 0.1)], 4, 64, 16)
    lat, rope = torch.zeros(8, 64), torch.zeros(8, 16)
    slots = torch.arange(8, dtype=torch.int64)
    codes, scales = torch.zeros(2, 64, 80, dtype=torch.uint8), torch.zeros(2, 64)
    with pytest.raises(ValueError, match="device tensor"):
        kk.quantize_write(m, 0, lat, rope, codes, scales, slots)
    g = kk.GqaModel([kk.LayerSpec(0, 0, 8, 0.1)], 4, 2, 64)
    with pytest.raises(ValueError, match="device tensor"):
        kk.gqa_quantize_write(g, 0, torch.zeros(8, 2, 64), torch.zeros(8, 2, 64), codes, scales, slots)


@pytest.mark.parametrize("d,dr,bits", [(512, 64, 2), (512, 64, 4), (512, 64, 8), (512, 64, 16), (256, 64, 4),
                                       (32, 16, 8), (64, 16, 2), (96, 32, 2), (160, 64, 4), (16, 16, 2)])
def test_row_stride_matches_oracle_layout(kk, d, dr, bits):
    assert kk.row_stride_bytes(d, dr, bits) == ko.row_stride(d + dr, bits)


def test_row_stride_rejects_invalid(kk):
    assert kk.row_stride_bytes(64, 16, 3) == 0
    assert kk.row_stride_bytes(0, 16, 4) == 0
    assert kk.row_stride_bytes(3, 0, 2) == 0          # 6 bits: not whole bytes


def table(rows, r=512, dr=64, heads=8, kk=None):
    layers = [kk.LayerSpec(a, d, b, 1.0 / math.sqrt(max(d, 1) + dr)) for a, d, b in rows]
    return kk.Model(layers, heads, r, dr)


def status(kk, model):
    return kk.lib().kk_validate_model(model.cfg)


def test_validate_model_rules(kk):
    ok = [[0, 512, 4], [0, 0, 0], [2, 256, 16], [2, 0, 0]]
    assert status(kk, table(ok, kk=kk)) == kk.KK_OK
    cases = {
        kk.KK_ERR_INVALID_ARGUMENT: [
            [[0, 0, 0]] * 1 + [[0, 0, 0]],            # layer 0 inherits (anchor 0 has d = 0)
            [[1, 64, 4], [1, 64, 4]],                 # layer 0 points forward
            [[0, 64, 4], [0, 0, 0], [1, 0, 0]],       # inherits an inheritor
            [[0, 64, 3]],                             # bits outside {2,4,8,16}
            [[0, 528, 4]],                            # d > r
            [[0, 64, 4], [2, 0, 0]],                  # anchor index beyond own index
        ],
        kk.KK_ERR_UNSUPPORTED: [
            [[0, 72, 4]],                             # d not a multiple of 16
        ],
    }
    for want, tables in cases.items():
        for t in tables:
            assert status(kk, table(t, kk=kk)) == want, t
    assert status(kk, table([[0, 64, 4]] + [[0, 0, 0]] * 64, kk=kk)) == kk.KK_ERR_UNSUPPORTED   # 65 layers
    assert status(kk, table([[0, 576, 4]], r=640, dr=64, kk=kk)) == kk.KK_ERR_UNSUPPORTED      # d > 512
    assert status(kk, table([[0, 64, 4]], dr=144, kk=kk)) == kk.KK_ERR_UNSUPPORTED             # d_R > 128
    assert status(kk, table([[0, 64, 4]], dr=24, kk=kk)) == kk.KK_ERR_UNSUPPORTED              # d_R % 16
    assert status(kk, table([[0, 512, 4]], dr=80, kk=kk)) == kk.KK_ERR_UNSUPPORTED             # d + d_R > 576
    assert status(kk, table([[0, 448, 4]], dr=128, kk=kk)) == kk.KK_OK                         # d + d_R = 576
    # Q.K reads the latent part in 64-field chunks from field 0 and the RoPE part
    # in 64-field chunks from field d: at most 9 chunks in all
    assert status(kk, table([[0, 480, 4]], dr=96, kk=kk)) == kk.KK_ERR_UNSUPPORTED             # 8 + 2 chunks
    assert status(kk, table([[0, 448, 4]], dr=80, kk=kk)) == kk.KK_OK                          # 7 + 2 chunks
    m = table([[0, 64, 4]], kk=kk)
    m._arr[0].sm_scale = float("nan")
    assert status(kk, m) == kk.KK_ERR_INVALID_ARGUMENT


def test_cache_bytes_and_offsets(kk):
    rows = [[0, 512, 4], [0, 0, 0], [2, 256, 16], [2, 0, 0], [2, 0, 0], [5, 128, 2]]
    m = table(rows, heads=40, kk=kk)
    B, T = 32, 8192
    for a, d, b in [(0, 512, 4), (2, 256, 16), (5, 128, 2)]:
        cb, sb = kk.cache_bytes(m, a, B, T)
        assert cb == B * T * ko.row_stride(d + 64, b)
        assert sb == B * T * 4
    with pytest.raises(kk.KKError) as e:
        kk.cache_bytes(m, 1, B, T)
    assert e.value.status == kk.KK_ERR_INVALID_ARGUMENT
    offs = kk.out_offsets(m, B)
    d_eff = [512, 512, 256, 256, 256, 128]
    want = [0]
    for d in d_eff:
        want.append(want[-1] + B * 40 * d)
    assert offs == want


def test_workspace_sizes(kk):
    rows = [[0, 512, 4], [0, 0, 0], [2, 256, 16]]
    m = table(rows, heads=40, kk=kk)
    # one split per sequence needs no partials
    assert kk.workspace_bytes(m, 4, 1024, 1024) == 0
    small = kk.workspace_bytes(m, 4, 1024, 512)
    smaller = kk.workspace_bytes(m, 4, 1024, 64)
    assert 0 < small < smaller
    assert kk.workspace_bytes(m, 4, 0, 0) == 0
    with pytest.raises(kk.KKError) as e:
        kk.workspace_bytes(m, 4, 1024, 48)                 # not a multiple of the 32-token tile
    assert e.value.status == kk.KK_ERR_INVALID_ARGUMENT


def test_plan_scales_with_compute_units(kk):
    """Automatic splits are planned for the device's compute units: more units,
    more (shorter) work items; an explicit split size ignores them."""
    import synth
    w = synth.workload(3)                                 # 48 layers, 40 heads, B = 32, T = 8192
    m = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    info = {c: kk.plan_info(m, w.batch, w.seq_len, 0, c) for c in (32, 64, 128, 256, 304, 512)}
    items = [info[c].work_items for c in sorted(info)]
    assert items == sorted(items) and items[0] < items[-1]
    for c, i in info.items():
        assert i.n_cus == c
        # about four waves of items over 2 workgroups per compute unit (fewer, longer ones for few units)
        assert i.work_items >= 2 * c or i.max_splits == 1
        assert 1 <= i.max_splits <= 64
    fixed = {c: kk.plan_info(m, w.batch, w.seq_len, 1024, c) for c in (64, 256)}
    assert fixed[64].work_items == fixed[256].work_items and fixed[64].max_splits == 8
    assert fixed[64].workspace_bytes == fixed[256].workspace_bytes
    with pytest.raises(kk.KKError) as e:
        kk.plan_info(m, w.batch, w.seq_len, 0, -1)
    assert e.value.status == kk.KK_ERR_INVALID_ARGUMENT


class _Fake:
    """Distinct, 256-byte aligned, never dereferenced host addresses for
    argument-check calls that must return before any launch."""

    def __init__(self):
        self.buf = ctypes.create_string_buffer(1 << 16)
        self.base = (ctypes.addressof(self.buf) + 255) // 256 * 256

    def __call__(self, i, misalign=0):
        return ctypes.c_void_p(self.base + 1024 * i + misalign)


def test_decode_attn_rejects_bad_arguments_before_launch(kk):
    L = kk.lib()
    rows = [[0, 128, 4], [0, 0, 0], [2, 64, 8]]
    m = table(rows, r=128, dr=32, heads=16, kk=kk)
    fake = _Fake()
    caches = (kk.Cache * 3)()
    caches[0] = kk.Cache(fake(1).value, fake(2).value)
    caches[2] = kk.Cache(fake(3).value, fake(4).value)
    B, T = 4, 1024
    need = kk.workspace_bytes(m, B, T, 64)
    assert need > 0

    def call(**kw):
        a = dict(caches=caches, batch=B, t_cap=T, seq_lens=fake(5), max_len=T, q_lat=fake(6), q_rope=fake(7),
                 q_dtype=kk.KK_DTYPE_F32, out=fake(8), split=64, ws=fake(9), ws_bytes=need)
        a.update(kw)
        return L.kk_decode_attn(m.cfg, a["caches"], a["batch"], a["t_cap"], a["seq_lens"], a["max_len"],
                                a["q_lat"], a["q_rope"], a["q_dtype"], a["out"], a["split"], a["ws"],
                                a["ws_bytes"], None)

    assert call(ws_bytes=need - 1) == kk.KK_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=fake(9, 16)) == kk.KK_ERR_INVALID_ARGUMENT          # workspace not 256-byte aligned
    assert call(ws=None) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(q_lat=fake(6, 4)) == kk.KK_ERR_INVALID_ARGUMENT        # query not 16-byte aligned
    assert call(out=None) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(max_len=T + 1) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(split=33) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(batch=0) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(q_dtype=7) == kk.KK_ERR_INVALID_ARGUMENT
    bad = (kk.Cache * 3)()
    bad[0] = caches[0]                                                 # anchor 2 has no buffers
    assert call(caches=bad) == kk.KK_ERR_INVALID_ARGUMENT
    bad[2] = kk.Cache(fake(3, 8).value, fake(4).value)                 # codes not 16-byte aligned
    assert call(caches=bad) == kk.KK_ERR_INVALID_ARGUMENT


def test_append_decode_rejects_bad_arguments_before_launch(kk):
    L = kk.lib()
    rows = [[0, 128, 4], [0, 0, 0], [2, 64, 8]]
    m = table(rows, r=128, dr=32, heads=16, kk=kk)
    fake = _Fake()
    caches = (kk.Cache * 3)()
    caches[0] = kk.Cache(fake(1).value, fake(2).value)
    caches[2] = kk.Cache(fake(3).value, fake(4).value)
    B, T = 4, 1024
    need = kk.workspace_bytes(m, B, T, 64)

    def call(**kw):
        a = dict(lat=fake(10), rope=fake(11), src=kk.KK_DTYPE_F32, ws_bytes=need, q_dtype=kk.KK_DTYPE_BF16,
                 caches=caches)
        a.update(kw)
        return L.kk_append_decode(m.cfg, a["caches"], B, T, fake(5), T, a["lat"], a["rope"], a["src"], fake(6),
                                  fake(7), a["q_dtype"], fake(8), 64, fake(9), a["ws_bytes"], None)

    assert call(src=3) == kk.KK_ERR_INVALID_ARGUMENT                   # source dtype
    assert call(lat=None) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(rope=fake(11, 2)) == kk.KK_ERR_INVALID_ARGUMENT        # f32 rows not 4-byte aligned
    assert call(ws_bytes=need - 1) == kk.KK_ERR_WORKSPACE_TOO_SMALL    # decode checks come first
    assert call(q_dtype=9) == kk.KK_ERR_INVALID_ARGUMENT
    bad = (kk.Cache * 3)()
    bad[0] = caches[0]
    assert call(caches=bad) == kk.KK_ERR_INVALID_ARGUMENT             # anchor 2 has no buffers


def test_quantize_write_rejects_bad_arguments_before_launch(kk):
    L = kk.lib()
    rows = [[0, 128, 4], [0, 0, 0]]
    m = table(rows, r=128, dr=32, heads=16, kk=kk)
    fake = _Fake()

    def call(layer=0, dtype=kk.KK_DTYPE_F32, lat_ld=128, rope_ld=32, n_src=10, n_tok=10, codes=None, latent=None):
        c = kk.Cache(codes if codes is not None else fake(1).value, fake(2).value)
        return L.kk_quantize_write(m.cfg, layer, latent if latent is not None else fake(3), fake(4), dtype,
                                   lat_ld, rope_ld, n_src, n_tok, None, fake(5), c, 2, 16, None)

    assert call(layer=1) == kk.KK_ERR_INVALID_ARGUMENT                 # an inheriting layer owns no cache
    assert call(layer=2) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(dtype=5) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(lat_ld=64) == kk.KK_ERR_INVALID_ARGUMENT               # row shorter than d
    assert call(rope_ld=16) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(n_tok=-1) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(codes=fake(1, 8).value) == kk.KK_ERR_INVALID_ARGUMENT  # codes not 16-byte aligned
    assert call(latent=fake(3, 2)) == kk.KK_ERR_INVALID_ARGUMENT       # f32 rows not 4-byte aligned
    assert call(n_tok=0) == kk.KK_OK                                   # nothing to write: no launch


def _runs(kk, specs, fake=None, heads=16, r=128, dr=32):
    """specs: list of (table rows, batch); returns (models, TableBatch array, cache arrays)."""
    models, ctabs = [], []
    for i, (rows, b) in enumerate(specs):
        m = table(rows, r=r, dr=dr, heads=heads, kk=kk)
        models.append(m)
        ct = None
        if fake is not None:
            ct = (kk.Cache * len(rows))()
            for l, (a, _, _) in enumerate(rows):
                if a == l:
                    ct[l] = kk.Cache(fake(16 * i + 2 * l + 20).value, fake(16 * i + 2 * l + 21).value)
        ctabs.append(ct)
    arr = (kk.kk.TableBatch * len(specs))(*[kk.kk.TableBatch(ctypes.pointer(m._cfg), b, ct)
                                           for m, (_, b), ct in zip(models, specs, ctabs)])
    return models, arr, ctabs


SPECS = [([[0, 128, 4], [0, 0, 0], [2, 64, 8]], 2), ([[0, 32, 16], [1, 96, 2], [1, 0, 0]], 3)]


def test_multi_offsets_and_workspace(kk):
    L = kk.lib()
    models, arr, _ = _runs(kk, SPECS)
    offs = (ctypes.c_int64 * 7)()
    assert L.kk_multi_out_offsets(arr, 2, offs) == kk.KK_OK
    want, base = [], 0
    for m, (_, b) in zip(models, SPECS):
        one = kk.out_offsets(m, b)
        want += [base + x for x in one[:-1]]
        base += one[-1]
    assert list(offs) == want + [base]
    ws = ctypes.c_size_t()
    assert L.kk_multi_decode_workspace_bytes(arr, 2, 1024, 1024, ctypes.byref(ws)) == kk.KK_OK
    assert ws.value > 0 and ws.value % 256 == 0                         # the plan only (no splits)
    ws_split = ctypes.c_size_t()
    assert L.kk_multi_decode_workspace_bytes(arr, 2, 1024, 64, ctypes.byref(ws_split)) == kk.KK_OK
    assert ws_split.value > ws.value                                    # partials of 16 splits
    assert L.kk_multi_decode_workspace_bytes(arr, 2, 1024, 48, ctypes.byref(ws)) == kk.KK_ERR_INVALID_ARGUMENT
    assert L.kk_multi_out_offsets(arr, 0, offs) == kk.KK_ERR_INVALID_ARGUMENT
    assert L.kk_multi_out_offsets(None, 2, offs) == kk.KK_ERR_INVALID_ARGUMENT
    # the tables must describe one model: same layers, heads, r and d_R
    _, other, _ = _runs(kk, [SPECS[0], ([[0, 128, 4], [0, 0, 0], [2, 64, 8]], 1)], heads=8)
    _, mixed, _ = _runs(kk, [SPECS[0]])
    mix = (kk.kk.TableBatch * 2)(mixed[0], other[1])
    assert L.kk_multi_out_offsets(mix, 2, offs) == kk.KK_ERR_INVALID_ARGUMENT
    _, zero, _ = _runs(kk, [SPECS[0], (SPECS[1][0], 0)])
    assert L.kk_multi_out_offsets(zero, 2, offs) == kk.KK_ERR_INVALID_ARGUMENT
    _, badt, _ = _runs(kk, [SPECS[0], ([[0, 128, 4], [2, 0, 0], [2, 64, 8]], 1)])  # inherits from a later layer
    assert L.kk_multi_out_offsets(badt, 2, offs) == kk.KK_ERR_INVALID_ARGUMENT
    big = (kk.kk.TableBatch * 1025)(*([arr[0]] * 1025))
    assert L.kk_multi_out_offsets(big, 1025, (ctypes.c_int64 * (3 * 1025 + 1))()) == kk.KK_ERR_UNSUPPORTED


def test_multi_decode_rejects_bad_arguments_before_launch(kk):
    L = kk.lib()
    fake = _Fake()
    models, arr, ctabs = _runs(kk, SPECS, fake)
    T = 1024
    need = ctypes.c_size_t()
    assert L.kk_multi_decode_workspace_bytes(arr, 2, T, 64, ctypes.byref(need)) == kk.KK_OK
    need = need.value

    def call(**kw):
        a = dict(tabs=arr, n=2, t_cap=T, seq_lens=fake(5), max_len=T, q_lat=fake(6), q_rope=fake(7),
                 q_dtype=kk.KK_DTYPE_BF16, out=fake(8), split=64, ws=fake(9), ws_bytes=need)
        a.update(kw)
        return L.kk_multi_decode_attn(a["tabs"], a["n"], a["t_cap"], a["seq_lens"], a["max_len"], a["q_lat"],
                                      a["q_rope"], a["q_dtype"], a["out"], a["split"], a["ws"], a["ws_bytes"], None)

    assert call(ws_bytes=need - 1) == kk.KK_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=fake(9, 16)) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(ws=None) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(q_rope=fake(7, 8)) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(seq_lens=None) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(max_len=T + 1) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(split=33) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(q_dtype=4) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(n=0) == kk.KK_ERR_INVALID_ARGUMENT
    nocache = (kk.kk.TableBatch * 2)(arr[0], kk.kk.TableBatch(ctypes.pointer(models[1]._cfg), 3, None))
    assert call(tabs=nocache) == kk.KK_ERR_INVALID_ARGUMENT            # a run without caches
    hole = (kk.Cache * 3)()
    hole[0] = ctabs[1][0]                                              # anchor 1 of run 1 has no buffers
    holed = (kk.kk.TableBatch * 2)(arr[0], kk.kk.TableBatch(ctypes.pointer(models[1]._cfg), 3, hole))
    assert call(tabs=holed) == kk.KK_ERR_INVALID_ARGUMENT
    hole[1] = kk.Cache(fake(60, 4).value, fake(61).value)              # codes not 16-byte aligned
    assert call(tabs=holed) == kk.KK_ERR_INVALID_ARGUMENT


def test_latent_epilogue_rejects_bad_arguments_before_launch(kk):
    L = kk.lib()
    m = table([[0, 128, 4], [0, 0, 0], [2, 64, 8]], r=128, dr=32, heads=16, kk=kk)
    fake = _Fake()
    wu = (ctypes.c_void_p * 3)(fake(10).value, fake(11).value, fake(12).value)
    wo = (ctypes.c_void_p * 3)(fake(13).value, fake(14).value, fake(15).value)

    def call(batch=4, d_v=64, d_model=256, o=None, u=wu, w=wo, v=None, y=None):
        return L.kk_latent_epilogue(m.cfg, batch, d_v, d_model, o or fake(1), u, w, v or fake(2), y or fake(3), None)

    assert call(batch=0) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(d_v=60) == kk.KK_ERR_INVALID_ARGUMENT                  # d_v not a multiple of 8
    assert call(d_model=100) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(o=fake(1, 4)) == kk.KK_ERR_INVALID_ARGUMENT            # o_lat not 16-byte aligned
    assert call(y=fake(3, 8)) == kk.KK_ERR_INVALID_ARGUMENT
    assert call(u=None) == kk.KK_ERR_INVALID_ARGUMENT
    hole = (ctypes.c_void_p * 3)(fake(10).value, None, fake(12).value)  # every layer needs its own weights
    assert call(u=hole) == kk.KK_ERR_INVALID_ARGUMENT
    mis = (ctypes.c_void_p * 3)(fake(13).value, fake(14, 2).value, fake(15).value)
    assert call(w=mis) == kk.KK_ERR_INVALID_ARGUMENT
    bad = table([[0, 100, 4]], r=128, dr=32, heads=16, kk=kk)           # d not a multiple of 16
    assert L.kk_latent_epilogue(bad.cfg, 4, 64, 256, fake(1), wu, wo, fake(2), fake(3), None) != kk.KK_OK


def gqa(kk, rows, nq=8, nkv=2, dh=128):
    layers = [kk.LayerSpec(a, d, b, 0.1) for a, d, b in rows]
    return kk.GqaModel(layers, nq, nkv, dh)


def test_gqa_sizes_and_rules(kk):
    L = kk.lib()
    m = gqa(kk, [[0, 0, 4], [0, 0, 0], [2, 0, 16]])
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.kk_gqa_cache_bytes(m.cfg, 2, 3, 100, ctypes.byref(cb), ctypes.byref(sb)) == kk.KK_OK
    assert cb.value == 3 * 2 * 100 * ko.row_stride(256, 16) and sb.value == 3 * 2 * 100 * 4
    assert L.kk_gqa_cache_bytes(m.cfg, 1, 3, 100, ctypes.byref(cb), ctypes.byref(sb)) == kk.KK_ERR_INVALID_ARGUMENT
    ws = ctypes.c_size_t()
    assert L.kk_gqa_decode_workspace_bytes(m.cfg, 3, 1024, 1024, ctypes.byref(ws)) == kk.KK_OK and ws.value == 0
    assert L.kk_gqa_decode_workspace_bytes(m.cfg, 3, 1024, 64, ctypes.byref(ws)) == kk.KK_OK and ws.value > 0
    assert status_gqa(kk, gqa(kk, [[0, 0, 4]], nq=6, nkv=4)) == kk.KK_ERR_INVALID_ARGUMENT     # H % n_kv != 0
    assert status_gqa(kk, gqa(kk, [[0, 0, 4]], dh=96)) == kk.KK_ERR_UNSUPPORTED                # d_h 64 or 128
    assert status_gqa(kk, gqa(kk, [[0, 0, 4]], nq=66, nkv=1)) == kk.KK_ERR_UNSUPPORTED         # > 32 per KV head
    assert status_gqa(kk, gqa(kk, [[0, 0, 3]])) == kk.KK_ERR_INVALID_ARGUMENT                  # bits
    assert status_gqa(kk, gqa(kk, [[1, 0, 0]])) == kk.KK_ERR_INVALID_ARGUMENT                  # layer 0 inherits


def status_gqa(kk, m):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    return kk.lib().kk_gqa_cache_bytes(m.cfg, 0, 1, 16, ctypes.byref(cb), ctypes.byref(sb))


def test_gqa_calls_reject_bad_arguments_before_launch(kk):
    L = kk.lib()
    m = gqa(kk, [[0, 0, 4], [0, 0, 0], [2, 0, 8]])
    fake = _Fake()
    caches = (kk.Cache * 3)()
    caches[0] = kk.Cache(fake(1).value, fake(2).value)
    caches[2] = kk.Cache(fake(3).value, fake(4).value)
    need = ctypes.c_size_t()
    assert L.kk_gqa_decode_workspace_bytes(m.cfg, 4, 1024, 64, ctypes.byref(need)) == kk.KK_OK
    need = need.value

    def dec(**kw):
        a = dict(caches=caches, max_len=1024, q=fake(6), out=fake(8), split=64, ws=fake(9), ws_bytes=need,
                 q_dtype=kk.KK_DTYPE_BF16)
        a.update(kw)
        return L.kk_gqa_decode_attn(m.cfg, a["caches"], 4, 1024, fake(5), a["max_len"], a["q"], a["q_dtype"],
                                    a["out"], a["split"], a["ws"], a["ws_bytes"], None)

    assert dec(ws_bytes=need - 1) == kk.KK_ERR_WORKSPACE_TOO_SMALL
    assert dec(ws=fake(9, 32)) == kk.KK_ERR_INVALID_ARGUMENT
    assert dec(q=fake(6, 8)) == kk.KK_ERR_INVALID_ARGUMENT
    assert dec(max_len=1025) == kk.KK_ERR_INVALID_ARGUMENT
    assert dec(split=40) == kk.KK_ERR_INVALID_ARGUMENT
    assert dec(q_dtype=5) == kk.KK_ERR_INVALID_ARGUMENT
    bad = (kk.Cache * 3)()
    bad[0] = caches[0]
    assert dec(caches=bad) == kk.KK_ERR_INVALID_ARGUMENT

    def wr(layer=0, dtype=kk.KK_DTYPE_F32, k=None, n_tok=4, codes=None):
        c = kk.Cache(codes if codes is not None else fake(1).value, fake(2).value)
        return L.kk_gqa_quantize_write(m.cfg, layer, k or fake(10), fake(11), dtype, 4, n_tok, None, fake(12), c, 4,
                                       1024, None)

    assert wr(layer=1) == kk.KK_ERR_INVALID_ARGUMENT
    assert wr(dtype=2) == kk.KK_ERR_INVALID_ARGUMENT
    assert wr(k=fake(10, 2)) == kk.KK_ERR_INVALID_ARGUMENT
    assert wr(codes=fake(1, 4).value) == kk.KK_ERR_INVALID_ARGUMENT
    assert wr(n_tok=0) == kk.KK_OK


def test_status_strings(kk):
    seen = {kk.status_string(s) for s in range(5)}
    assert len(seen) == 5 and kk.status_string(0) == "ok"
    assert kk.status_string(99) == "unknown status"


def test_merge_is_cut_into_parts_when_merges_are_few(kk):
    """The merge launch runs one workgroup per (entry, sequence, row chunk),
    or up to 4 per merge (feature ranges) when there are fewer merges than
    4 workgroups per compute unit.  With 1024-token splits every one of the
    48 one-layer chunks of the 40-head table is merged for every sequence."""
    import synth
    w = synth.workload(3)
    m = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    for batch, cus, blocks in ((32, 256, 1536), (8, 256, 384 * 3), (8, 64, 384), (2, 256, 96 * 4), (2, 16, 96)):
        i = kk.plan_info(m, batch, w.seq_len, 1024, cus)
        assert i.max_splits == 8
        assert i.merge_blocks == blocks, (batch, cus, i.merge_blocks)
    # no splits, no merge
    assert kk.plan_info(m, 32, 1024, 1024, 256).merge_blocks == 0


def _chunks_of_table(layers, heads):
    """Row chunks per anchor group entry, as the planner documents them: RB =
    min(3, ceil(min(H, 64) / 16)) blocks of 16 rows; chunks hold whole layers
    when a layer fits (H <= 16 RB), else 16 RB rows; entries of at most 8
    chunks.  Returns [(d, chunks)] per entry."""
    rb = min(3, (min(heads, 64) + 15) // 16)
    chunk_rows = heads * ((16 * rb) // heads) if heads <= 16 * rb else 16 * rb
    out = []
    for a, s in enumerate(layers):
        if s.anchor != a:
            continue
        rows = sum(1 for t in layers if t.anchor == a) * heads
        for r0 in range(0, rows, 8 * chunk_rows):
            n = min(rows, r0 + 8 * chunk_rows) - r0
            out.append((s.d, -(-n // chunk_rows)))
    return out


def test_plan_invariants_over_random_tables(kk):
    """Property test of the planner over random valid tables, batches,
    lengths, split sizes and compute-unit counts (run under ASan/UBSan by the
    sanitizer test too).  With a fixed split size every count is predictable:
    items = chunks x batch x splits, one merge (cut into up to 4 parts when
    merges are fewer than 4 per compute unit) per (chunk, sequence), and the
    workspace is one partial slot (32 d + 192 floats) per item.  Automatic
    splits keep the same structure within bounds."""
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")

    @st.composite
    def tables(draw):
        L = draw(st.integers(1, 64))
        H = draw(st.sampled_from([1, 3, 4, 8, 15, 16, 17, 24, 28, 32, 33, 40, 48, 49, 64, 100, 128]))
        d_rope = draw(st.sampled_from([16, 32, 64, 128]))
        r = 512
        layers, anchors = [], []
        for l in range(L):
            if l > 0 and draw(st.booleans()) and draw(st.booleans()):
                a = draw(st.sampled_from(anchors))
                layers.append(ko.Layer(a, 0, 0, layers[a].sm_scale))
            else:
                d = draw(st.integers(1, min(512, 576 - d_rope) // 16)) * 16
                b = draw(st.sampled_from([2, 4, 8, 16]))
                layers.append(ko.Layer(l, d, b, 1.0 / math.sqrt(d + d_rope)))
                anchors.append(l)
        return layers, H, r, d_rope

    @hyp.settings(max_examples=120, deadline=None, derandomize=True)
    @hyp.given(tables(), st.integers(1, 64), st.integers(0, 70000), st.integers(0, 8), st.integers(1, 1024))
    def check(tab, batch, max_len, split_mult, cus):
        layers, H, r, d_rope = tab
        m = kk.Model(layers, H, r, d_rope)
        ents = _chunks_of_table(layers, H)
        chunks = sum(c for _, c in ents)
        split = 1024 * split_mult
        try:
            info = kk.plan_info(m, batch, max_len, split, cus)
        except kk.KKError as e:
            # only plans past the launch limits are refused
            assert e.status == kk.KK_ERR_UNSUPPORTED and len(ents) > 88
            return
        assert len(ents) <= 88
        assert info.n_cus == cus
        assert 1 <= info.max_splits <= 64
        assert chunks * batch <= info.work_items <= chunks * batch * info.max_splits
        assert (info.max_splits == 1) == (info.merge_blocks == 0) == (info.workspace_bytes == 0)
        if info.max_splits > 1:   # automatic splits may leave some entries unsplit (no merge)
            assert 1 <= info.merge_blocks <= 4 * chunks * batch
        if split > 0:
            S = min(64, max(1, -(-max_len // split))) if max_len > 0 else 1
            assert info.max_splits == S
            assert info.work_items == chunks * batch * S
            if S > 1:
                parts = min(4, max(1, -(-4 * cus // (chunks * batch))))
                assert info.merge_blocks == chunks * batch * parts
                assert info.workspace_bytes == sum(c * batch * S * (32 * d + 192) * 4 for d, c in ents)
            assert kk.workspace_bytes(m, batch, max_len, split) == info.workspace_bytes

    check()
