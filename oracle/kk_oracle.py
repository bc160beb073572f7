"""Plain CPU oracle for KV-Kaizen compressed decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no common helpers, tables or constants); both sides follow the
same written layout specification independently.

What it computes, and from where (web pages on KV-Kaizen, arXiv 2609.37988;
page "KV-Kaizen: Learning Context-Adaptive Cache Compression Choices",
the picx.dev whiteboard summary, is the only one with method detail):

* Depth axis (section "Three Non-Eviction Compression Axes", item 1): an
  anchor layer owns a cache, later layers inherit the cache of an anchor.
* Rank axis (same section, item 2): the MLA cache holds a latent c^KV in R^r
  and a decoupled RoPE key k^R in R^{d_R}; only the first d <= r latent
  coordinates are kept.
* Precision axis (same section, item 3): cached tensors are stored at b <= 16
  bits with symmetric uniform quantization and one scale per token.
* Action set and cost (section "Action Space and Cost Model", the action-set
  equation and the per-token cost equation c(a)): inherit costs 0 bits,
  (d, b) costs (d + d_R) * b bits per token; rho = C0 / sum_l c(a_l) with
  C0 = L * 2 * n_kv * d_h * 16 (bf16 non-MLA cache).
* Decode reads the whole cache of every layer at every generated token
  (section "Background: The KV Cache Bottleneck").

Readings where the pages are silent:

* One scale covers the concatenation [c[:d] || k^R] of one anchor layer for
  one token; scale = amax / qmax in IEEE fp32 division, qmax = 2^(b-1) - 1,
  code = clamp(rint_half_even(fl32(v / scale)), -qmax, qmax); an all-zero
  token has scale 0 and codes 0.  b = 16 is also an integer code with a scale.
* A scale costs 32 bits per anchor layer per token on top of c(a).
* Codes are b-bit two's-complement fields, field j at bit offset j*b of the
  row (little-endian bytes), rows zero-padded to a multiple of 16 bytes.
  b = 16 is stored as two byte planes: the K high bytes (field order), then
  the K low bytes with bit 7 flipped (offset binary).
* Absorbed-MLA attention per head h: z_t = sm_scale * (q_lat[:d] . c_t[:d] +
  q_rope . k^R_t) on the dequantized cache, softmax over the cached tokens,
  o = sum_t p_t c_t[:d].  An empty cache gives o = 0.
* Latent epilogue (the MLA value path after attention; the pages name the
  shared latent and its truncation, section "Three Non-Eviction Compression
  Axes", item 2, but not the projections): head h's value is its block of
  the value up-projection W_UV [H * d_v, r] applied to o restricted to the
  kept coordinates, v_h = W_UV[h*d_v:(h+1)*d_v, :d] o_h, and the layer output
  is y = W_O [v_1; ...; v_H] with W_O [D, H * d_v].  Because attention is
  linear in the values, this equals attention over the per-token values
  W_UV[h] c_t[:d] (the non-absorbed form), which pins it.

* Non-MLA variant (precision and depth on a grouped-query cache; the
  configuration of the "Precision + depth" rows of Table 1 and the KVK 4x
  row of Table 2): an anchor layer caches keys K and values V per KV head,
  [n_kv, d_h] each per token, at b bits; inheriting layers read it.  One
  scale per token covers everything the anchor stores for that token (K and
  V of all KV heads, as for the MLA row).  Query head h reads KV head
  h // (H / n_kv): z_t = sm_scale * q_h . K_t, o_h = sum_t softmax(z)_t V_t.
  The cost of a (b) action is 2 * n_kv * d_h * b bits per token.

Floating point: the quantizer runs in numpy float32 (its decisions are
defined in fp32); dequantization and attention run in float64.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BITS_SET = (2, 4, 8, 16)          # section "Action Space and Cost Model": the bit-width set
SCALE_BITS = 32                   # one fp32 scale per token per anchor layer (reading)


# ----------------------------------------------------------------------------
# Quantization (precision axis)
# ----------------------------------------------------------------------------

def qmax(bits: int) -> int:
    """Largest symmetric code magnitude for b-bit two's complement, 2^(b-1) - 1."""
    return (1 << (bits - 1)) - 1


def quantize_rows(v: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric uniform quantization with one scale per row (per token).

    Follows the precision item of "Three Non-Eviction Compression Axes":
    every value of the row shares one scale; codes are symmetric integers.
    ``v`` is [N, K]; it is taken as float32 exactly (bf16 sources widen
    exactly).  Returns int32 codes [N, K] and float32 scales [N].
    """
    if bits not in BITS_SET:
        raise ValueError(f"bits must be one of {BITS_SET}")
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("v must be [N, K]")
    amax = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    qm = np.float32(qmax(bits))
    scale = (amax / qm).astype(np.float32)                 # IEEE fp32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = v / scale[:, None]                           # fp32 / fp32, rounded once
    codes = np.clip(np.rint(quot), -qm, qm)                 # ties to even, then clamp
    codes[amax == 0] = 0.0
    return codes.astype(np.int32), scale


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x_hat = code * scale, exact in float64 (at most 15 + 24 significant bits)."""
    return codes.astype(np.float64) * scale.astype(np.float64)[:, None]


# ----------------------------------------------------------------------------
# Bit packing (layout reading: b-bit two's-complement fields, LSB first)
# ----------------------------------------------------------------------------

def row_bytes(k: int, bits: int) -> int:
    if (k * bits) % 8:
        raise ValueError("row of k fields at b bits is not a whole number of bytes")
    return k * bits // 8


def row_stride(k: int, bits: int) -> int:
    """Row bytes rounded up to a multiple of 16."""
    return (row_bytes(k, bits) + 15) // 16 * 16


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack int codes [N, K] into uint8 rows [N, row_stride]."""
    codes = np.asarray(codes, dtype=np.int64)
    n, k = codes.shape
    nb = row_bytes(k, bits)
    out = np.zeros((n, row_stride(k, bits)), dtype=np.uint8)
    mask = (1 << bits) - 1
    u = (codes & mask).astype(np.uint64)                    # two's-complement field value
    if bits == 16:                                        # byte planes
        out[:, :k] = (u >> np.uint64(8)).astype(np.uint8)
        out[:, k:2 * k] = ((u & np.uint64(0xFF)) ^ np.uint64(0x80)).astype(np.uint8)
        return out
    per_byte = 8 // bits
    u = u.reshape(n, nb, per_byte)
    byte = np.zeros((n, nb), dtype=np.uint64)
    for i in range(per_byte):
        byte |= u[:, :, i] << np.uint64(i * bits)
    out[:, :nb] = byte.astype(np.uint8)
    return out


def unpack_rows(packed: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Inverse of pack_rows: uint8 rows -> sign-extended int32 codes [N, K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    nb = row_bytes(k, bits)
    b = packed[:, :nb].astype(np.int64)
    if bits == 16:
        u = (b[:, k:2 * k] ^ 0x80) | (b[:, :k] << 8)
    else:
        per_byte = 8 // bits
        mask = (1 << bits) - 1
        u = np.stack([(b >> (i * bits)) & mask for i in range(per_byte)], axis=2).reshape(n, k)
    sign = 1 << (bits - 1)
    return np.where(u >= sign, u - (1 << bits), u).astype(np.int32)


# ----------------------------------------------------------------------------
# Per-layer table (depth / rank / precision actions)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Layer:
    anchor: int          # == own index: anchor; < own index: inherits that anchor's cache
    d: int               # kept latent width (anchors)
    bits: int            # bit width (anchors)
    sm_scale: float      # softmax scale of this layer


def resolve_table(layers: list[Layer], r: int) -> list[tuple[int, int, int]]:
    """For every layer return (anchor, d_eff, b_eff).

    Depth item of "Three Non-Eviction Compression Axes": an anchor produces a
    cache and later layers inherit from an anchor; an inheritor reads its
    anchor's cache, so its d and b are the anchor's.
    """
    out = []
    for l, lay in enumerate(layers):
        a = lay.anchor
        if a == l:
            if not (0 < lay.d <= r) or lay.bits not in BITS_SET:
                raise ValueError(f"layer {l}: bad anchor action")
            out.append((l, lay.d, lay.bits))
        else:
            if not (0 <= a < l) or layers[a].anchor != a:
                raise ValueError(f"layer {l}: anchor {a} is not an earlier anchor")
            out.append((a, layers[a].d, layers[a].bits))
    return out


# ----------------------------------------------------------------------------
# Cache write and decode attention
# ----------------------------------------------------------------------------

def write_cache(latent: np.ndarray, rope: np.ndarray, d: int, bits: int):
    """Quantize and pack rows [c[:d] || k^R] of one anchor layer.

    latent [N, >= d], rope [N, d_R] (float32 or exactly-widened bf16).
    Returns (packed uint8 [N, stride], scales float32 [N], codes int32 [N, d + d_R]).
    """
    v = np.concatenate([np.asarray(latent, np.float32)[:, :d], np.asarray(rope, np.float32)], axis=1)
    codes, scales = quantize_rows(v, bits)
    return pack_rows(codes, bits), scales, codes


def attend(qv: np.ndarray, xhat: np.ndarray, d: int, sm_scale: float) -> np.ndarray:
    """Softmax attention of H query rows over T cached rows, values = xhat[:, :d].

    qv [H, K], xhat [T, K] (float64); z = sm_scale * qv . xhat_t; returns [H, d].
    An empty cache (T = 0) returns zeros (reading: empty sum).
    """
    qv = np.asarray(qv, np.float64)
    xhat = np.asarray(xhat, np.float64)
    if xhat.shape[0] == 0:
        return np.zeros((qv.shape[0], d), np.float64)
    z = float(sm_scale) * (qv @ xhat.T)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    return (w @ xhat[:, :d]) / w.sum(axis=1, keepdims=True)


def decode_layer(q_lat: np.ndarray, q_rope: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                 d: int, d_rope: int, bits: int, sm_scale: float, seq_len: int) -> np.ndarray:
    """Absorbed-MLA decode for one layer and one sequence.

    q_lat [H, >= d], q_rope [H, d_R]; packed/scales: the anchor cache rows of
    this sequence.  Only the first ``seq_len`` rows are attended.
    """
    k = d + d_rope
    codes = unpack_rows(packed[:seq_len], bits, k)
    xhat = dequantize_rows(codes, scales[:seq_len])
    qv = np.concatenate([np.asarray(q_lat, np.float64)[:, :d], np.asarray(q_rope, np.float64)], axis=1)
    return attend(qv, xhat, d, sm_scale)


def latent_epilogue(o_lat: np.ndarray, w_uv: np.ndarray, w_o: np.ndarray, d_v: int):
    """Value up-projection and output projection of one layer.

    o_lat [B, H, d] (attention output in the kept latent coordinates),
    w_uv [H * d_v, r] with r >= d (columns d.. are not used), w_o [D, H * d_v].
    Returns (v [B, H, d_v], y [B, D]) in float64:
      v[b, h, j] = sum_{i<d} w_uv[h*d_v + j, i] * o_lat[b, h, i]
      y[b, n]    = sum_{h, j} w_o[n, h*d_v + j] * v[b, h, j]
    """
    o = np.asarray(o_lat, np.float64)
    bsz, heads, d = o.shape
    wu = np.asarray(w_uv, np.float64)
    wo = np.asarray(w_o, np.float64)
    v = np.empty((bsz, heads, d_v), np.float64)
    for h in range(heads):
        v[:, h, :] = o[:, h, :] @ wu[h * d_v:(h + 1) * d_v, :d].T
    y = v.reshape(bsz, heads * d_v) @ wo.T
    return v, y


def gqa_write_cache(k: np.ndarray, v: np.ndarray, bits: int):
    """Quantize one anchor layer of a grouped-query cache.

    k, v [N, n_kv, d_h] (float32 or exactly-widened bf16).  One scale per
    token over all of that token's K and V values.  Returns (codes_k, codes_v
    int32 [N, n_kv, d_h], scales float32 [N])."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    n, nkv, dh = k.shape
    codes, scales = quantize_rows(np.concatenate([k.reshape(n, nkv * dh), v.reshape(n, nkv * dh)], axis=1), bits)
    return codes[:, :nkv * dh].reshape(n, nkv, dh), codes[:, nkv * dh:].reshape(n, nkv, dh), scales


def gqa_pack_kv_rows(codes_k: np.ndarray, codes_v: np.ndarray, bits: int) -> np.ndarray:
    """The library's row layout: per (token, KV head) one packed row of
    2 d_h fields, values first then keys, [N, n_kv, stride] uint8."""
    n, nkv, dh = codes_k.shape
    rows = np.concatenate([codes_v, codes_k], axis=2).reshape(n * nkv, 2 * dh)
    packed = pack_rows(rows, bits)
    return packed.reshape(n, nkv, packed.shape[1])


def gqa_decode_layer(q: np.ndarray, codes_k: np.ndarray, codes_v: np.ndarray, scales: np.ndarray,
                     sm_scale: float, seq_len: int) -> np.ndarray:
    """Grouped-query decode for one layer and one sequence: q [H, d_h];
    codes [T, n_kv, d_h] with scales [T].  Returns o [H, d_h] (float64)."""
    q = np.asarray(q, np.float64)
    h_total, dh = q.shape
    nkv = codes_k.shape[1]
    group = h_total // nkv
    sc = np.asarray(scales[:seq_len], np.float64)[:, None]
    out = np.zeros((h_total, dh), np.float64)
    if seq_len == 0:
        return out
    for g in range(nkv):
        kh = codes_k[:seq_len, g, :].astype(np.float64) * sc
        vh = codes_v[:seq_len, g, :].astype(np.float64) * sc
        for j in range(group):
            h = g * group + j
            z = float(sm_scale) * (kh @ q[h])
            w = np.exp(z - z.max())
            out[h] = (w @ vh) / w.sum()
    return out


def gqa_table_bits_per_token(layers: list[Layer], n_kv: int, d_head: int, scale_bits: int = SCALE_BITS) -> int:
    """Stored bits per token of a grouped-query table: per anchor
    2 * n_kv * d_h * b + one scale."""
    return sum(2 * n_kv * d_head * lay.bits + scale_bits for l, lay in enumerate(layers) if lay.anchor == l)


def partial_state(qv, xhat, d, sm_scale):
    """Flash-decoding partial over a token subset: (m [H], l [H], O [H, d]) with
    O = sum_t exp(z_t - m) xhat_t[:d] (unnormalized).  Used to check the
    split-and-merge reading of online softmax."""
    if xhat.shape[0] == 0:
        h = qv.shape[0]
        return np.full(h, -np.inf), np.zeros(h), np.zeros((h, d))
    z = float(sm_scale) * (np.asarray(qv, np.float64) @ np.asarray(xhat, np.float64).T)
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    return m, w.sum(axis=1), w @ xhat[:, :d]


def merge_states(states):
    """Merge partials: m* = max m_j; l* = sum l_j e^(m_j - m*); o = sum O_j e^(m_j - m*) / l*."""
    ms = np.stack([s[0] for s in states])
    finite = np.isfinite(ms)
    mstar = np.where(finite, ms, -np.inf).max(axis=0)
    lsum = 0.0
    osum = 0.0
    for (m, l, o) in states:
        w = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(mstar), mstar, 0.0)), 0.0)
        lsum = lsum + l * w
        osum = osum + o * w[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(lsum[:, None] > 0, osum / np.where(lsum > 0, lsum, 1.0)[:, None], 0.0)
    return out


# ----------------------------------------------------------------------------
# Accounting (cost model)
# ----------------------------------------------------------------------------

def actions(r: int) -> list:
    """Action set A = {inherit} U {(d, b) : d in {r/8, r/4, r/2, r}, b in {2,4,8,16}}."""
    return ["inherit"] + [(d, b) for d in (r // 8, r // 4, r // 2, r) for b in BITS_SET]


def action_cost_bits(action, d_rope: int) -> int:
    """Per-token cost c(a): 0 for inherit, (d + d_R) * b otherwise."""
    if action == "inherit":
        return 0
    d, b = action
    return (d + d_rope) * b


def c0_bits(n_layers: int, n_kv: int, d_head: int) -> int:
    """Uncompressed bf16 non-MLA cost per token: C0 = L * 2 * n_kv * d_h * 16."""
    return n_layers * 2 * n_kv * d_head * 16


def table_bits_per_token(layers: list[Layer], d_rope: int, scale_bits: int = SCALE_BITS) -> int:
    """Stored bits per token: sum over anchors of (d + d_R) * b + scale bits."""
    total = 0
    for l, lay in enumerate(layers):
        if lay.anchor == l:
            total += action_cost_bits((lay.d, lay.bits), d_rope) + scale_bits
    return total


def anchor_cache_bytes(d: int, d_rope: int, bits: int, batch: int, t_cap: int) -> int:
    """Bytes one anchor cache occupies: batch * t_cap * (row stride + 4 scale bytes)."""
    return batch * t_cap * (row_stride(d + d_rope, bits) + 4)


# ----------------------------------------------------------------------------
# Whole decode step over a table (all layers, all sequences)
# ----------------------------------------------------------------------------

def decode_step(layers: list[Layer], r: int, d_rope: int, caches: dict, q_lat: np.ndarray,
                q_rope: np.ndarray, seq_lens, layer_ids=None, seq_ids=None) -> dict:
    """Run decode attention for the given layers and sequences.

    caches: anchor index -> (packed [B, T_cap, stride], scales [B, T_cap]).
    q_lat [L, B, H, r], q_rope [L, B, H, d_R].  Returns {(l, s): o [H, d_eff]}.
    """
    res = resolve_table(layers, r)
    layer_ids = range(len(layers)) if layer_ids is None else layer_ids
    seq_ids = range(len(seq_lens)) if seq_ids is None else seq_ids
    out = {}
    for l in layer_ids:
        a, d, b = res[l]
        packed, scales = caches[a]
        for s in seq_ids:
            out[(l, s)] = decode_layer(q_lat[l, s], q_rope[l, s], packed[s], scales[s], d, d_rope, b,
                                       layers[l].sm_scale, int(seq_lens[s]))
    return out
