"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational arithmetic, brute-force enumeration, an independent bit-string
packer, closed forms printed on the KV-Kaizen summary page, a library
attention routine, or identities of softmax attention.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kk_oracle as ko
import synth

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------
# helpers independent of the oracle
# ----------------------------------------------------------------------------

def f32_round(x: Fraction) -> np.float32:
    """Correctly rounded (ties to even) float32 of an exact rational."""
    c = np.float32(float(x))                      # within an ulp or so
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for v in cands:
        err = abs(Fraction(float(v)) - x)
        key = (err, int(np.frombuffer(np.float32(v).tobytes(), np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def nearest_int_even(x: Fraction) -> int:
    f = math.floor(x)
    r = x - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def brute_quantize_row(v: np.ndarray, bits: int):
    """Exact-rational statement of the quantizer: scale = fl32(amax/qmax),
    code = clamp(round_half_even(fl32(v/scale)))."""
    qm = (1 << (bits - 1)) - 1
    amax = max(abs(Fraction(float(x))) for x in v)
    if amax == 0:
        return [0] * len(v), np.float32(0)
    scale = f32_round(amax / qm)
    codes = []
    for x in v:
        quot = f32_round(Fraction(float(x)) / Fraction(float(scale)))
        k = nearest_int_even(Fraction(float(quot)))
        codes.append(max(-qm, min(qm, k)))
    return codes, scale


def bitstring_pack(codes, bits):
    """Row as one big little-endian integer: field j at bit j*b.  b = 16: the
    high bytes of the fields in order, then their low bytes with bit 7 flipped."""
    k = len(codes)
    if bits == 16:
        raw = bytes(((int(c) & 0xFFFF) >> 8) for c in codes) + bytes(((int(c) & 0xFF) ^ 0x80) for c in codes)
        return raw + bytes((len(raw) + 15) // 16 * 16 - len(raw))
    acc = 0
    for j, c in enumerate(codes):
        acc |= (int(c) & ((1 << bits) - 1)) << (j * bits)
    nbytes = k * bits // 8
    raw = acc.to_bytes(nbytes, "little")
    stride = (nbytes + 15) // 16 * 16
    return raw + bytes(stride - nbytes)


# ----------------------------------------------------------------------------
# quantizer
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4, 8, 16])
def test_quantizer_matches_exact_rational_statement(bits):
    rows = [RNG.standard_normal(48).astype(np.float32) * np.float32(10.0 ** RNG.integers(-3, 3)) for _ in range(6)]
    rows.append((np.arange(48, dtype=np.float32) - 20) * np.float32(0.37))
    rows.append(np.float32(1e-30) * RNG.standard_normal(48).astype(np.float32))
    v = np.stack(rows)
    codes, scale = ko.quantize_rows(v, bits)
    for i in range(v.shape[0]):
        bc, bs = brute_quantize_row(v[i], bits)
        assert scale[i] == bs
        assert list(codes[i]) == bc


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantizer_code_is_nearest_level_by_enumeration(bits):
    qm = (1 << (bits - 1)) - 1
    v = RNG.standard_normal((64, 40)).astype(np.float32)
    codes, scale = ko.quantize_rows(v, bits)
    for i in range(v.shape[0]):
        quot = (v[i] / scale[i]).astype(np.float64)      # the single fp32 rounding, widened
        levels = np.arange(-qm, qm + 1)
        for j in range(v.shape[1]):
            dist = np.abs(quot[j] - levels)
            best = levels[dist == dist.min()]
            pick = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert codes[i, j] == pick


def test_quantizer_ties_go_to_even():
    # amax = 127 at b = 8 gives scale exactly 1.0; half-integers are exact ties
    v = np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5]], np.float32)
    codes, scale = ko.quantize_rows(v, 8)
    assert scale[0] == 1.0
    assert list(codes[0]) == [127, 2, 4, -2, -4, 0, 0, 126]


@pytest.mark.parametrize("bits", [2, 4, 8, 16])
def test_quantizer_reconstruction_bound_and_range(bits):
    qm = (1 << (bits - 1)) - 1
    v = (RNG.standard_normal((200, 576)) * np.exp(RNG.standard_normal((200, 1)))).astype(np.float32)
    v[3, 17] = 40.0                                   # an outlier row
    codes, scale = ko.quantize_rows(v, bits)
    xhat = codes.astype(np.float64) * scale.astype(np.float64)[:, None]
    err = np.abs(v.astype(np.float64) - xhat)
    bound = scale.astype(np.float64)[:, None] / 2 + np.abs(v.astype(np.float64)) * 2.0 ** -23
    assert np.all(err <= bound)
    assert np.all(np.abs(codes) <= qm)
    amax_pos = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(codes[np.arange(200), amax_pos]) == qm)
    assert np.all(np.abs(scale.astype(np.float64) * qm - np.abs(v).max(1)) <= np.abs(v).max(1) * 2.0 ** -23)


def test_quantizer_zero_token():
    v = np.zeros((2, 32), np.float32)
    v[1, 5] = -3.0
    codes, scale = ko.quantize_rows(v, 4)
    assert scale[0] == 0 and np.all(codes[0] == 0)
    assert codes[1, 5] == -7 and scale[1] == np.float32(3.0) / np.float32(7.0)


# ----------------------------------------------------------------------------
# rank axis: the cache keeps the FIRST d of the r latent coordinates
# ----------------------------------------------------------------------------

def _rank_pin_failures(write, lat, rope, d, bits):
    """Checks of a cache writer against the rank item of "Three Non-Eviction
    Compression Axes" (keep the first d latent coordinates, then the RoPE
    key), stated without the oracle: the reconstruction bound element by
    element against [lat[:, :d] || rope], the scale as fl32(amax / qmax)
    over exactly those values (exact rationals), invariance under any change
    of the dropped coordinates d..r-1, and sensitivity to every kept one.
    Returns the list of failed checks (empty: the writer passes)."""
    fails = []
    n, dr = rope.shape
    qm = (1 << (bits - 1)) - 1
    packed, scales, codes = write(lat, rope, d, bits)
    if codes.shape != (n, d + dr):
        return ["shape"]
    v = np.concatenate([lat[:, :d], rope], axis=1).astype(np.float64)
    xhat = codes.astype(np.float64) * scales.astype(np.float64)[:, None]
    if not np.all(np.abs(v - xhat) <= scales.astype(np.float64)[:, None] / 2 + np.abs(v) * 2.0 ** -23):
        fails.append("reconstruction")
    for i in range(0, n, max(1, n // 8)):
        amax = max(abs(Fraction(float(x))) for x in v[i])
        if scales[i] != f32_round(amax / qm):
            fails.append("scale")
            break
    bumped = lat.copy()
    bumped[:, d:] = 1e6 * np.sign(RNG.standard_normal(bumped[:, d:].shape)).astype(np.float32)
    p2, s2, _ = write(bumped, rope, d, bits)
    if not (np.array_equal(p2, packed) and np.array_equal(s2.view(np.uint32), scales.view(np.uint32))):
        fails.append("dropped coordinates matter")
    for j in (0, d // 2, d - 1):
        moved = lat.copy()
        moved[:, j] = 3.0 * np.abs(lat).max() + 1.0
        p3, _, _ = write(moved, rope, d, bits)
        if np.array_equal(p3, packed):
            fails.append(f"kept coordinate {j} ignored")
    return fails


def _rank_pin_inputs(n=64, r=64, dr=16):
    rng = np.random.default_rng(77)
    lat = (rng.standard_normal((n, r)) / np.sqrt(1 + np.arange(r) / 8)).astype(np.float32)
    rope = rng.standard_normal((n, dr)).astype(np.float32)
    return lat, rope


@pytest.mark.parametrize("bits", [2, 4, 8, 16])
@pytest.mark.parametrize("d", [16, 32, 48])
def test_write_cache_keeps_first_d_latent_coordinates(bits, d):
    lat, rope = _rank_pin_inputs()
    # the largest value of every row sits just past the kept width: a writer
    # that kept one coordinate too many would take its scale from it
    lat[:, d] = 10.0 * np.abs(lat).max(axis=1)
    assert _rank_pin_failures(ko.write_cache, lat, rope, d, bits) == []


@pytest.mark.parametrize("bits", [8, 16])
def test_rank_pin_rejects_wrong_latent_slices(bits):
    # planted mistakes (writers built from the oracle's quantizer and packer
    # with a wrong slice of the latent): the pin above must reject each one
    def writer(select):
        def w(latent, rope, d, b):
            v = np.concatenate([select(np.asarray(latent, np.float32), d), np.asarray(rope, np.float32)], axis=1)
            codes, scales = ko.quantize_rows(v, b)
            return ko.pack_rows(codes, b), scales, codes
        return w
    mutants = {
        "shifted by one": lambda x, d: x[:, 1:d + 1],
        "last d": lambda x, d: x[:, x.shape[1] - d:],
        "reversed": lambda x, d: x[:, d - 1::-1],
        "every other": lambda x, d: x[:, 0:2 * d:2],
    }
    lat, rope = _rank_pin_inputs()
    d = 32
    assert _rank_pin_failures(writer(lambda x, d: x[:, :d]), lat, rope, d, bits) == []
    for name, sel in mutants.items():
        assert _rank_pin_failures(writer(sel), lat, rope, d, bits), name


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

def test_pack_worked_example_two_bit():
    # fields (1, -1, 0, 1) at 2 bits, LSB first: 01 | 11<<2 | 00<<4 | 01<<6 = 0x4D
    packed = ko.pack_rows(np.array([[1, -1, 0, 1, 0, 0, 0, 0]]), 2)
    assert packed[0, 0] == 0x4D and packed[0, 1] == 0 and packed.shape[1] == 16


def test_pack_worked_example_sixteen_bit_planes():
    # codes (1, -1, 256, -32767) -> high bytes 00 FF 01 80, low bytes 01 FF 00 01 with bit 7 flipped
    codes = np.array([[1, -1, 256, -32767] + [0] * 4])
    packed = ko.pack_rows(codes, 16)
    assert list(packed[0, :4]) == [0x00, 0xFF, 0x01, 0x80]
    assert list(packed[0, 8:12]) == [0x81, 0x7F, 0x80, 0x81]
    assert list(packed[0, 4:8]) == [0, 0, 0, 0] and list(packed[0, 12:16]) == [0x80] * 4
    assert np.array_equal(ko.unpack_rows(packed, 16, 8), codes)


@pytest.mark.parametrize("bits,k", [(2, 48), (2, 576), (4, 48), (4, 320), (8, 48), (8, 576), (16, 48), (16, 576)])
def test_pack_matches_bitstring_and_round_trips(bits, k):
    qm = (1 << (bits - 1)) - 1
    codes = RNG.integers(-qm, qm + 1, size=(7, k))
    packed = ko.pack_rows(codes, bits)
    assert packed.shape[1] % 16 == 0 and packed.shape[1] == ko.row_stride(k, bits)
    for i in range(7):
        assert packed[i].tobytes() == bitstring_pack(codes[i], bits)
    assert np.array_equal(ko.unpack_rows(packed, bits, k), codes)


# ----------------------------------------------------------------------------
# accounting: closed forms printed on the pages
# ----------------------------------------------------------------------------

def test_qwen14b_cache_size_192kib_and_48gib():
    # Background section: 192 KiB per token for Qwen2.5-14B (48 layers, 8 KV heads of 128, bf16),
    # and 48 GiB for 32 sequences of 8k tokens.
    bits = ko.c0_bits(48, 8, 128)
    assert bits == 1_572_864
    assert bits // 8 == 192 * 1024
    assert 32 * 8192 * (bits // 8) == 48 * 2 ** 30


def test_action_space_has_17_actions():
    acts = ko.actions(512)
    assert len(acts) == 17 and len(set(map(str, acts))) == 17
    assert (64, 2) in acts and (512, 16) in acts and "inherit" in acts


def test_precision_only_floor_is_8x_and_depth_only_4x_needs_quarter_anchors():
    # Non-MLA precision-only: every layer stores 2*n_kv*d_h values at b bits -> rho = 16 / b, floor at b = 2.
    L, nkv, dh = 28, 4, 128
    best = ko.c0_bits(L, nkv, dh) / (L * 2 * nkv * dh * min(ko.BITS_SET))
    assert best == 8.0
    # Depth-only: anchors store full bf16 K/V; reaching 4x needs L/4 anchors (3/4 of layers inherit).
    anchors = L // 4
    assert ko.c0_bits(L, nkv, dh) / (anchors * 2 * nkv * dh * 16) == 4.0


def test_uniform_7b_workloads_ratio_and_mixed_14b_budget():
    w1, w2 = synth.workload(1), synth.workload(2)
    lay = lambda w: [ko.Layer(s.anchor, s.d, s.bits, s.sm_scale) for s in w.layers]
    b1 = ko.table_bits_per_token(lay(w1), 64)
    b2 = ko.table_bits_per_token(lay(w2), 64)
    assert b1 == 28 * (576 * 16 + 32) == 258_944
    assert b2 == 28 * (320 * 8 + 32) == 72_576
    assert abs(b1 / b2 - 3.568) < 1e-3
    w3 = synth.workload(3)
    b3 = ko.table_bits_per_token(lay(w3), 64)
    full = 48 * (576 * 16 + 32)
    assert abs(b3 / (full / 4) - 1) <= 0.01
    # eviction keeping 1/8 on top: the decode-time cache is about 32x smaller than the full bf16 MLA cache
    ratio = (full * 65536) / (b3 * 8192)
    assert abs(ratio / 32 - 1) <= 0.011


def test_cache_bytes_match_bits_when_rows_are_unpadded():
    w3 = synth.workload(3)
    tot = 0
    for a in w3.anchors():
        s = w3.layers[a]
        assert ko.row_bytes(s.d + 64, s.bits) == ko.row_stride(s.d + 64, s.bits)
        tot += ko.anchor_cache_bytes(s.d, 64, s.bits, 1, 1)
    lay = [ko.Layer(s.anchor, s.d, s.bits, s.sm_scale) for s in w3.layers]
    assert tot * 8 == ko.table_bits_per_token(lay, 64)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def _cache(t, k, d_rope, bits, seed=0):
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((t, k - d_rope)).astype(np.float32)
    rope = rng.standard_normal((t, d_rope)).astype(np.float32)
    return lat, rope


def test_attention_matches_library_sdpa_fp64():
    H, T, d, dR, bits = 8, 300, 96, 32, 4
    lat, rope = _cache(T, d + dR, dR, bits)
    packed, scales, codes = ko.write_cache(lat, rope, d, bits)
    q = np.random.default_rng(5).standard_normal((H, d + dR))
    sm = 1 / math.sqrt(d + dR)
    o = ko.decode_layer(q[:, :d], q[:, d:], packed, scales, d, dR, bits, sm, T)
    xhat = torch.from_numpy(codes.astype(np.float64) * scales.astype(np.float64)[:, None])
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = xhat[None, None].expand(1, H, T, d + dR)
    vt = xhat[None, None, :, :d].expand(1, H, T, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm)[0, :, 0].numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_attention_closed_forms():
    d, k = 16, 24
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, k))
    q = rng.standard_normal((3, k))
    # T = 1: output is the single value row
    assert np.array_equal(ko.attend(q, x[:1], d, 0.7), np.repeat(x[:1, :d], 3, axis=0))
    # q = 0: uniform weights, output is the mean of the value rows
    o = ko.attend(np.zeros((2, k)), x, d, 0.7)
    assert np.allclose(o, np.repeat(x[:, :d].mean(0, keepdims=True), 2, 0), atol=1e-15, rtol=0)
    # T = 2: sigmoid of the score difference
    z = 0.7 * (q @ x[:2].T)
    s0 = 1 / (1 + np.exp(-(z[:, 0] - z[:, 1])))
    ref = s0[:, None] * x[0, :d] + (1 - s0)[:, None] * x[1, :d]
    assert np.allclose(ko.attend(q, x[:2], d, 0.7), ref, atol=1e-14, rtol=0)
    # empty cache: zero output
    assert np.all(ko.attend(q, x[:0], d, 0.7) == 0)


def test_attention_permutation_invariance_and_split_merge():
    H, T, d, dR = 4, 257, 64, 16
    rng = np.random.default_rng(11)
    xhat = rng.standard_normal((T, d + dR))
    q = rng.standard_normal((H, d + dR)) * 3
    sm = 0.25
    o = ko.attend(q, xhat, d, sm)
    perm = rng.permutation(T)
    assert np.allclose(ko.attend(q, xhat[perm], d, sm), o, atol=1e-13, rtol=0)
    for cuts in ([0, 100, 257], [0, 1, 2, 130, 257], [0, 0, 64, 64, 257, 257]):
        parts = [ko.partial_state(q, xhat[a:b], d, sm) for a, b in zip(cuts[:-1], cuts[1:])]
        assert np.allclose(ko.merge_states(parts), o, atol=1e-13, rtol=0)


def _bruteforce_attention(qv, xhat, d, sm_scale):
    out = []
    for h in range(len(qv)):
        z = [sm_scale * math.fsum(float(qv[h][j]) * float(xhat[t][j]) for j in range(len(qv[h])))
             for t in range(len(xhat))]
        m = max(z)
        w = [math.exp(v - m) for v in z]
        lsum = math.fsum(w)
        out.append([math.fsum(w[t] * float(xhat[t][i]) for t in range(len(xhat))) / lsum for i in range(d)])
    return np.array(out)


def test_tiny_workload_bruteforce():
    w = synth.workload(0)
    lat, rope, _ = synth.source_rows(w, 0)
    ql, qr = synth.queries(w)
    lat, rope = lat[0].numpy(), rope[0].numpy()
    packed, scales, codes = ko.write_cache(lat, rope, 32, 8)
    sm = w.layers[0].sm_scale
    o = ko.decode_layer(ql[0, 0].numpy(), qr[0, 0].numpy(), packed, scales, 32, 16, 8, sm, 256)
    xhat = [[int(c) * float(s) for c in row] for row, s in zip(codes, scales)]
    qv = [list(map(float, ql[0, 0, h, :32])) + list(map(float, qr[0, 0, h])) for h in range(4)]
    ref = _bruteforce_attention(qv, xhat, 32, sm)
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_b16_full_rank_reproduces_uncompressed_attention():
    # least-compressed action (d = r, b = 16) against attention on the unquantized source
    H, T, r, dR = 28, 1024, 512, 64
    rng = np.random.default_rng(3)
    lat = (rng.standard_normal((T, r)) / np.sqrt(1 + np.arange(r) / 8)).astype(np.float32)
    rope = rng.standard_normal((T, dR)).astype(np.float32)
    q = rng.standard_normal((H, r + dR)).astype(np.float32)
    sm = 1 / math.sqrt(r + dR)
    packed, scales, _ = ko.write_cache(lat, rope, r, 16)
    o = ko.decode_layer(q[:, :r], q[:, r:], packed, scales, r, dR, 16, sm, T)
    src = np.concatenate([lat, rope], 1).astype(np.float64)
    ref = ko.attend(q.astype(np.float64), src, r, sm)
    err = np.max(np.abs(o - ref)) / np.max(np.abs(ref))
    assert err <= 2e-3
    assert err <= 1e-4          # 15-bit codes: far inside the bar


def test_inheritor_reads_anchor_cache():
    r, dR, H, T = 128, 32, 6, 70
    rng = np.random.default_rng(21)
    lat, rope = rng.standard_normal((1, T, r)).astype(np.float32), rng.standard_normal((1, T, dR)).astype(np.float32)
    layers = [ko.Layer(0, 64, 4, 0.11), ko.Layer(0, 999, 3, 0.2), ko.Layer(2, 128, 8, 0.1), ko.Layer(0, 0, 0, 0.3)]
    packed, scales, _ = ko.write_cache(lat[0], rope[0], 64, 4)
    caches = {0: (packed[None], scales[None]), 2: (np.zeros((1, T, 160), np.uint8), np.zeros((1, T), np.float32))}
    ql = rng.standard_normal((4, 1, H, r))
    qr = rng.standard_normal((4, 1, H, dR))
    out = ko.decode_step(layers, r, dR, caches, ql, qr, [T])
    for l in (1, 3):
        one = ko.decode_layer(ql[l, 0], qr[l, 0], packed, scales, 64, dR, 4, layers[l].sm_scale, T)
        assert np.array_equal(out[(l, 0)], one)
        assert out[(l, 0)].shape == (H, 64)


def test_table_rules():
    ok = [ko.Layer(0, 64, 8, 1.0), ko.Layer(0, 0, 0, 1.0)]
    assert ko.resolve_table(ok, 64) == [(0, 64, 8), (0, 64, 8)]
    for bad in ([ko.Layer(1, 64, 8, 1.0), ko.Layer(1, 64, 8, 1.0)],          # layer 0 inherits from later
                [ko.Layer(0, 64, 8, 1.0), ko.Layer(1, 64, 3, 1.0)],          # bad bits
                [ko.Layer(0, 65, 8, 1.0)],                                    # d > r
                [ko.Layer(0, 64, 8, 1.0), ko.Layer(0, 0, 0, 1.0), ko.Layer(1, 0, 0, 1.0)]):  # names an inheritor
        with pytest.raises(ValueError):
            ko.resolve_table(bad, 64)


# ----------------------------------------------------------------------------
# latent epilogue (value up-projection, output projection)
# ----------------------------------------------------------------------------

def test_epilogue_identity_blocks_and_permutation():
    """W_UV blocks that copy the kept coordinates (d_v = d) give v = o exactly;
    a permutation W_O then reorders the concatenated heads."""
    rng = np.random.default_rng(3)
    B, H, d, r = 2, 3, 8, 12
    o = rng.standard_normal((B, H, d))
    w_uv = rng.standard_normal((H * d, r))          # columns >= d are never read
    for h in range(H):
        w_uv[h * d:(h + 1) * d, :d] = np.eye(d)
    perm = rng.permutation(H * d)
    w_o = np.eye(H * d)[perm]
    v, y = ko.latent_epilogue(o, w_uv, w_o, d)
    assert np.array_equal(v, o)
    assert np.array_equal(y, o.reshape(B, H * d)[:, perm])


def test_epilogue_ignores_columns_past_the_kept_width():
    rng = np.random.default_rng(4)
    B, H, d, r, dv, D = 2, 2, 8, 16, 5, 7
    o = rng.standard_normal((B, H, d))
    w_uv = rng.standard_normal((H * dv, r))
    w_o = rng.standard_normal((D, H * dv))
    v1, y1 = ko.latent_epilogue(o, w_uv, w_o, dv)
    w_uv[:, d:] = rng.standard_normal((H * dv, r - d)) * 1e6
    v2, y2 = ko.latent_epilogue(o, w_uv, w_o, dv)
    assert np.array_equal(v1, v2) and np.array_equal(y1, y2)


def test_epilogue_after_absorbed_decode_equals_attention_over_projected_values():
    """Linearity of attention in its values: decoding in the latent space and
    then projecting (the absorbed form) equals attention whose values are the
    per-token projections W_UV[h] c_t[:d] (the non-absorbed form), softmax
    taken here with scipy, then W_O."""
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    H, d, r, dr, dv, D, T, bits = 3, 16, 24, 8, 6, 10, 40, 8
    lat = rng.standard_normal((T, r)).astype(np.float32)
    rope = rng.standard_normal((T, dr)).astype(np.float32)
    q_lat = rng.standard_normal((H, r))
    q_rope = rng.standard_normal((H, dr))
    w_uv = rng.standard_normal((H * dv, r)) / np.sqrt(r)
    w_o = rng.standard_normal((D, H * dv)) / np.sqrt(H * dv)
    sm = 0.3
    packed, scales, _ = ko.write_cache(lat, rope, d, bits)
    o = ko.decode_layer(q_lat, q_rope, packed, scales, d, dr, bits, sm, T)
    v, y = ko.latent_epilogue(o[None], w_uv, w_o, dv)
    xhat = ko.dequantize_rows(ko.unpack_rows(packed, bits, d + dr), scales)
    keys = xhat                                                       # [c[:d] || k^R]
    y_ref = np.zeros(D)
    vs = []
    for h in range(H):
        qh = np.concatenate([q_lat[h, :d], q_rope[h]])
        p = softmax(sm * (keys @ qh))
        vals = xhat[:, :d] @ w_uv[h * dv:(h + 1) * dv, :d].T           # [T, dv] per-token values
        vh = p @ vals
        vs.append(vh)
        y_ref += w_o[:, h * dv:(h + 1) * dv] @ vh
    np.testing.assert_allclose(v[0], np.stack(vs), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[0], y_ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# grouped-query (non-MLA) variant: precision + depth
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4, 8, 16])
def test_gqa_decode_matches_sdpa_with_grouped_heads(bits):
    """Against torch's fp64 scaled_dot_product_attention with each KV head
    repeated for its query group, on the dequantized cache."""
    rng = np.random.default_rng(20 + bits)
    T, nkv, G, dh = 37, 2, 3, 16
    k = rng.standard_normal((T, nkv, dh)).astype(np.float32) * 2
    v = rng.standard_normal((T, nkv, dh)).astype(np.float32)
    q = rng.standard_normal((nkv * G, dh))
    ck, cv, sc = ko.gqa_write_cache(k, v, bits)
    sm = 0.2
    o = ko.gqa_decode_layer(q, ck, cv, sc, sm, T)
    kh = torch.from_numpy(ck.astype(np.float64) * sc.astype(np.float64)[:, None, None])
    vh = torch.from_numpy(cv.astype(np.float64) * sc.astype(np.float64)[:, None, None])
    kq = kh.permute(1, 0, 2).repeat_interleave(G, dim=0)            # [H, T, dh]
    vq = vh.permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], kq, vq, scale=sm)
    np.testing.assert_allclose(o, ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def test_gqa_one_scale_per_token_over_keys_and_values():
    rng = np.random.default_rng(31)
    T, nkv, dh, bits = 9, 3, 8, 4
    k = rng.standard_normal((T, nkv, dh)).astype(np.float32)
    v = rng.standard_normal((T, nkv, dh)).astype(np.float32) * 0.1
    v[4, 2, 5] = 9.0                                                 # the token's largest value is a V entry
    k[6] = 0
    v[6] = 0                                                         # an all-zero token
    ck, cv, sc = ko.gqa_write_cache(k, v, bits)
    qm = ko.qmax(bits)
    for t in range(T):
        amax = max(np.abs(k[t]).max(), np.abs(v[t]).max())
        assert sc[t] == np.float32(amax) / np.float32(qm)
        if amax > 0:
            assert max(np.abs(ck[t]).max(), np.abs(cv[t]).max()) == qm
    assert cv[4, 2, 5] == qm and sc[6] == 0 and not ck[6].any() and not cv[6].any()


def test_gqa_rows_hold_values_then_keys_and_reduce_to_latent_attention():
    """The library's row per (token, KV head) is [V codes || K codes]; with
    the query [0 || q_h] and values = the first d_h fields, the latent
    attention of the MLA path computes the grouped-query output."""
    rng = np.random.default_rng(32)
    T, nkv, G, dh, bits = 21, 2, 2, 16, 8
    k = rng.standard_normal((T, nkv, dh)).astype(np.float32)
    v = rng.standard_normal((T, nkv, dh)).astype(np.float32)
    q = rng.standard_normal((nkv * G, dh))
    ck, cv, sc = ko.gqa_write_cache(k, v, bits)
    rows = ko.gqa_pack_kv_rows(ck, cv, bits)
    o = ko.gqa_decode_layer(q, ck, cv, sc, 0.3, T)
    for g in range(nkv):
        codes = ko.unpack_rows(rows[:, g, :], bits, 2 * dh)
        assert np.array_equal(codes[:, :dh], cv[:, g]) and np.array_equal(codes[:, dh:], ck[:, g])
        xhat = ko.dequantize_rows(codes, sc)
        qv = np.concatenate([np.zeros((G, dh)), q[g * G:(g + 1) * G]], axis=1)
        np.testing.assert_allclose(ko.attend(qv, xhat, dh, 0.3), o[g * G:(g + 1) * G], rtol=1e-12, atol=1e-12)


def test_gqa_accounting_and_table_fixture():
    import importlib.util
    here = os.path.dirname(os.path.abspath(__file__))
    # C0 of the 14B shape: 48 * 2 * 8 * 128 * 16 bits = 192 KiB per token
    assert ko.c0_bits(48, 8, 128) == 192 * 1024 * 8
    # 8-bit anchors on every other layer: 2x from precision times 2x from depth
    half = [ko.Layer(l if l % 2 == 0 else l - 1, 128, 8, 1.0) for l in range(48)]
    assert abs(ko.c0_bits(48, 8, 128) / ko.gqa_table_bits_per_token(half, 8, 128) - 4) < 0.01
    spec = importlib.util.spec_from_file_location("mkg", os.path.join(here, "golden", "make_table_14b_gqa.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    fixture = json.load(open(os.path.join(here, "golden", "table_14b_gqa.json")))
    t, draws, bits = mk.freeze()
    assert (t, draws, bits) == (fixture["table"], fixture["draws"], fixture["bits_per_token"])
    assert abs(bits / (ko.c0_bits(48, 8, 128) / 4) - 1) <= 0.01
    for l, (a, d, b) in enumerate(t):
        assert a <= l and t[a][0] == a
        if a == l:
            assert d == 128 and b in (2, 4, 8, 16)


# ----------------------------------------------------------------------------
# fixtures and generators
# ----------------------------------------------------------------------------

def test_mixed_table_fixture_is_reproducible_and_valid():
    import importlib.util
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("mk", os.path.join(here, "golden", "make_table_14b_mixed.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    fixture = json.load(open(os.path.join(here, "golden", "table_14b_mixed.json")))
    rng = np.random.default_rng(7)
    full = 48 * ((512 + 64) * 16 + 32)
    for _ in range(fixture["draws"]):
        t = mk.draw(rng)
    assert t == fixture["table"]
    assert mk.bits_of(t) == fixture["bits_per_token"]
    assert abs(fixture["bits_per_token"] / (full / 4) - 1) <= 0.01
    assert t[0][0] == 0
    for l, (a, d, b) in enumerate(t):
        assert a <= l and t[a][0] == a
        if a != l:
            assert all(t[x][0] != x for x in range(a + 1, l + 1))    # nearest preceding anchor
    inh = sum(1 for l, (a, _, _) in enumerate(t) if a != l)
    assert 0.2 <= inh / 48 <= 0.45


def test_hetero_tables_fixture_is_reproducible_and_valid():
    import importlib.util
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("mk", os.path.join(here, "golden", "make_table_14b_mixed.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    fixture = json.load(open(os.path.join(here, "golden", "tables_14b_hetero.json")))
    single = json.load(open(os.path.join(here, "golden", "table_14b_mixed.json")))
    assert [x["seed"] for x in fixture["tables"]] == list(mk.HETERO_SEEDS)
    assert fixture["tables"][0]["table"] == single["table"]
    full = 48 * ((512 + 64) * 16 + 32)
    seen = set()
    for x in fixture["tables"]:
        t, draws, bits = mk.freeze(x["seed"])
        assert (t, draws, bits) == (x["table"], x["draws"], x["bits_per_token"])
        assert abs(bits / (full / 4) - 1) <= 0.01
        ko.resolve_table([ko.Layer(a, d, b, 1.0) for a, d, b in t], 512)    # a valid table
        seen.add(json.dumps(t))
    assert len(seen) == 4                                                   # four different tables


def test_eviction_positions():
    s = synth.gen_scores(4, 0, 65536)
    pos = synth.keep_positions(s, 8192)
    assert pos.numel() == 8192 and torch.all(pos[1:] > pos[:-1])
    kept = torch.zeros(65536, dtype=torch.bool)
    kept[pos.long()] = True
    assert s[kept].min() >= s[~kept].max()


def test_generators_are_seeded_and_shaped():
    a = synth.gen_latent(3, 5, (4, 2000), 512)
    b = synth.gen_latent(3, 5, (4, 2000), 512)
    c = synth.gen_latent(3, 6, (4, 2000), 512)
    assert torch.equal(a, b) and not torch.equal(a, c)
    var = a.reshape(-1, 512).double().var(0)
    expect = 1 / (1 + torch.arange(512, dtype=torch.float64) / 8)
    assert torch.all((var / expect - 1).abs() < 0.1)
    ql, qr = synth.queries(synth.workload(0))
    assert ql.shape == (1, 1, 4, 64) and qr.shape == (1, 1, 4, 16) and ql.dtype == torch.float32
