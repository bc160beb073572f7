"""Seeded generators and workload descriptions.

Distributions (the workload recipe):
  * latent c^KV coordinate i (0-based) ~ N(0, variance 1 / (1 + i / 8)),
  * RoPE key k^R ~ N(0, 1),
  * q_lat, q_rope ~ N(0, 1); float32 in the tiny workload, rounded to bf16
    (round-to-nearest-even) in the others,
  * eviction scores ~ U[0, 1), one draw per (sequence, original position).

Every tensor comes from its own torch.Generator, seeded from
(workload, layer, kind, extra) through numpy's SeedSequence, so any tensor can
be regenerated on its own.  Generation runs on the requested device (the
large workloads are drawn on the GPU; CPU and GPU streams differ, and every
consumer takes the tensors from here, never from the other side).
"""

from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np
import torch

KIND_LATENT, KIND_ROPE, KIND_QLAT, KIND_QROPE, KIND_SCORES, KIND_WUV, KIND_WO, KIND_K, KIND_V, KIND_Q = range(10)

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")


def seed_for(workload: int, layer: int, kind: int, extra: int = 0, data_seed: int = 0) -> int:
    ss = np.random.SeedSequence(data_seed, spawn_key=(workload, layer, kind, extra))
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def latent_std(r: int, device="cpu") -> torch.Tensor:
    i = torch.arange(r, dtype=torch.float64)
    return (1.0 / torch.sqrt(1.0 + i / 8.0)).to(torch.float32).to(device)


def gen_latent(workload: int, layer: int, shape, r: int, device="cpu", extra: int = 0) -> torch.Tensor:
    """[..., r] float32 latent rows with the decaying per-coordinate spread."""
    g = _gen(device, seed_for(workload, layer, KIND_LATENT, extra))
    x = torch.randn(*shape, r, generator=g, device=device, dtype=torch.float32)
    return x * latent_std(r, device)


def gen_rope(workload: int, layer: int, shape, d_rope: int, device="cpu", extra: int = 0) -> torch.Tensor:
    g = _gen(device, seed_for(workload, layer, KIND_ROPE, extra))
    return torch.randn(*shape, d_rope, generator=g, device=device, dtype=torch.float32)


def gen_q(workload: int, layer: int, kind: int, shape, width: int, dtype, device="cpu") -> torch.Tensor:
    g = _gen(device, seed_for(workload, layer, kind))
    x = torch.randn(*shape, width, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def gen_epilogue_weights(workload: int, layer: int, n_heads: int, d_v: int, r: int, d_model: int, device="cpu"):
    """Synthetic projection weights of one layer, rounded to bf16:
    W_UV [n_heads * d_v, r] ~ N(0, 1/r), W_O [d_model, n_heads * d_v] ~ N(0, 1/(n_heads * d_v))."""
    g = _gen(device, seed_for(workload, layer, KIND_WUV))
    w_uv = torch.randn(n_heads * d_v, r, generator=g, device=device, dtype=torch.float32) / math.sqrt(r)
    g = _gen(device, seed_for(workload, layer, KIND_WO))
    w_o = torch.randn(d_model, n_heads * d_v, generator=g, device=device, dtype=torch.float32) / math.sqrt(n_heads * d_v)
    return w_uv.to(torch.bfloat16), w_o.to(torch.bfloat16)


def gen_scores(workload: int, seq: int, n: int, device="cpu") -> torch.Tensor:
    g = _gen(device, seed_for(workload, 0, KIND_SCORES, seq))
    return torch.rand(n, generator=g, device=device, dtype=torch.float32)


def keep_positions(scores: torch.Tensor, keep: int) -> torch.Tensor:
    """Positions of the `keep` highest scores (ties to the lower position),
    returned ascending.  This is the stand-in eviction policy's selection,
    not part of the compressed-cache method."""
    order = torch.argsort(-scores, stable=True)[:keep]
    return torch.sort(order).values.to(torch.int32)


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclass
class LayerSpec:
    anchor: int
    d: int
    bits: int
    sm_scale: float


@dataclass
class Workload:
    wid: int
    name: str
    n_layers: int
    n_heads: int
    batch: int
    seq_len: int            # cached tokens per sequence (after eviction if any)
    r: int
    d_rope: int
    q_dtype: torch.dtype
    layers: list = field(default_factory=list)
    nominal_context: int = 0   # >0: rows kept from this many positions per sequence

    def anchors(self):
        return [l for l, s in enumerate(self.layers) if s.anchor == l]

    def d_eff(self, l):
        return self.layers[self.layers[l].anchor].d

    def bits_eff(self, l):
        return self.layers[self.layers[l].anchor].bits


def _uniform_layers(n, d, bits, d_rope):
    sm = 1.0 / math.sqrt(d + d_rope)
    return [LayerSpec(l, d, bits, sm) for l in range(n)]


def layers_from_table(table, d_rope):
    """table: list of [anchor, d, bits] (inheritors may carry d = bits = 0)."""
    out = []
    for l, (a, d, b) in enumerate(table):
        da = table[a][1]
        out.append(LayerSpec(int(a), int(d), int(b), 1.0 / math.sqrt(da + d_rope)))
    return out


def mixed_table_14b():
    """The frozen per-layer table of the 14B-shaped mixed workload."""
    with open(os.path.join(GOLDEN_DIR, "table_14b_mixed.json")) as f:
        return json.load(f)["table"]


def workload(wid: int) -> Workload:
    """The five workloads: 0 tiny, 1 7B-shaped uncompressed, 2 7B uniform d=256 b=8,
    3 14B-shaped mixed 4x, 4 14B-shaped mixed 4x with eviction keeping 1/8."""
    if wid == 0:
        return Workload(0, "tiny", 1, 4, 1, 256, 64, 16, torch.float32, _uniform_layers(1, 32, 8, 16))
    if wid == 1:
        return Workload(1, "7b_uncompressed", 28, 28, 32, 8192, 512, 64, torch.bfloat16,
                        _uniform_layers(28, 512, 16, 64))
    if wid == 2:
        return Workload(2, "7b_uniform_d256_b8", 28, 28, 32, 8192, 512, 64, torch.bfloat16,
                        _uniform_layers(28, 256, 8, 64))
    if wid == 3:
        return Workload(3, "14b_mixed_4x", 48, 40, 32, 8192, 512, 64, torch.bfloat16,
                        layers_from_table(mixed_table_14b(), 64))
    if wid == 4:
        return Workload(4, "14b_mixed_4x_evict8", 48, 40, 8, 8192, 512, 64, torch.bfloat16,
                        layers_from_table(mixed_table_14b(), 64), nominal_context=65536)
    raise ValueError(wid)


@dataclass
class GqaWorkload:
    """A grouped-query (non-MLA) model with a precision + depth table."""
    wid: int
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    batch: int
    seq_len: int
    q_dtype: torch.dtype
    layers: list = field(default_factory=list)

    def anchors(self):
        return [l for l, s in enumerate(self.layers) if s.anchor == l]

    def bits_eff(self, l):
        return self.layers[self.layers[l].anchor].bits


GQA_WID = 9


def gqa_layers_from_table(table, d_head):
    """table rows [anchor, d, bits]; softmax scale 1/sqrt(d_head) for every layer."""
    sm = 1.0 / math.sqrt(d_head)
    return [LayerSpec(int(a), int(d_head) if a == l else 0, int(b), sm) for l, (a, _, b) in enumerate(table)]


def gqa_table_14b():
    with open(os.path.join(GOLDEN_DIR, "table_14b_gqa.json")) as f:
        return json.load(f)["table"]


def gqa_workload(batch: int = 16, seq_len: int = 16384) -> GqaWorkload:
    """Qwen2.5-14B-shaped grouped-query model (48 layers, 40 query heads, 8 KV
    heads of 128) with the frozen 4x precision + depth table, at the 16k
    context of the long-context evaluation."""
    return GqaWorkload(GQA_WID, "14b_gqa_4x", 48, 40, 8, 128, batch, seq_len, torch.bfloat16,
                       gqa_layers_from_table(gqa_table_14b(), 128))


def small_gqa_workload(wid: int, table, n_q_heads: int, n_kv_heads: int, d_head: int, batch: int, seq_len: int,
                       q_dtype=torch.bfloat16) -> GqaWorkload:
    return GqaWorkload(wid, "small_gqa", len(table), n_q_heads, n_kv_heads, d_head, batch, seq_len, q_dtype,
                       gqa_layers_from_table(table, d_head))


def gqa_source(w: GqaWorkload, layer: int, device="cpu"):
    """K and V source rows of one anchor layer, float32 [B, T, n_kv, d_head], both N(0, 1)."""
    shape = (w.batch, w.seq_len, w.n_kv_heads, w.d_head)
    g = _gen(device, seed_for(w.wid, layer, KIND_K))
    k = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    g = _gen(device, seed_for(w.wid, layer, KIND_V))
    v = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return k, v


def gqa_queries(w: GqaWorkload, device="cpu"):
    """q [L, B, H, d_head] ~ N(0, 1) in the workload's q dtype."""
    qs = []
    for l in range(w.n_layers):
        g = _gen(device, seed_for(w.wid, l, KIND_Q))
        qs.append(torch.randn(w.batch, w.n_q_heads, w.d_head, generator=g, device=device).to(w.q_dtype))
    return torch.stack(qs)


HETERO_WID = 5   # data seeds of run k of the heterogeneous batch: workload HETERO_WID + k


def hetero_tables_14b():
    """The four frozen tables of the heterogeneous-batch workload."""
    with open(os.path.join(GOLDEN_DIR, "tables_14b_hetero.json")) as f:
        return [x["table"] for x in json.load(f)["tables"]]


def hetero_workloads(batch_per_table: int = 8, seq_len: int = 8192, tables=None, n_heads: int = 40,
                     r: int = 512, d_rope: int = 64):
    """14B-shaped heterogeneous batch: run k (k = 0..3) holds batch_per_table
    sequences that use table k, with its own data seeds.  Returns one
    Workload per run; the runs follow one another in the batch."""
    tables = hetero_tables_14b() if tables is None else tables
    return [Workload(HETERO_WID + k, f"14b_hetero_run{k}", len(t), n_heads, batch_per_table, seq_len, r, d_rope,
                     torch.bfloat16, layers_from_table(t, d_rope)) for k, t in enumerate(tables)]


def depth_variant(w: Workload, mode: str) -> Workload:
    """The workload with its depth sharing changed, for measuring what sharing
    costs and saves.  "own_cache": every inheriting layer becomes an anchor with
    its former anchor's width and bit width (the same query rows and work; each
    layer's bytes are read from a cache of its own).  "anchors_only": the
    inheriting layers are left out.  "shared" returns w."""
    if mode == "shared":
        return w
    if mode == "own_cache":
        layers = [LayerSpec(l, w.layers[s.anchor].d, w.layers[s.anchor].bits, s.sm_scale)
                  for l, s in enumerate(w.layers)]
    elif mode == "anchors_only":
        layers = [LayerSpec(i, w.layers[a].d, w.layers[a].bits, w.layers[a].sm_scale)
                  for i, a in enumerate(w.anchors())]
    else:
        raise ValueError(f"depth mode {mode!r}: shared, own_cache or anchors_only")
    return replace(w, name=f"{w.name}_{mode}", n_layers=len(layers), layers=layers)


def uniform_workload(d: int, bits: int, n_layers: int = 8) -> Workload:
    """n_layers anchors of one (d, b) in the 14B shape (40 heads, B = 32,
    T = 8192, r = 512, d_R = 64), drawn from the 14B workload's generators:
    the cost of one layer at each kept width and bit width."""
    return Workload(3, f"uniform_{n_layers}x_d{d}_b{bits}", n_layers, 40, 32, 8192, 512, 64, torch.bfloat16,
                    _uniform_layers(n_layers, d, bits, 64))


def small_workload(wid: int, n_layers: int, n_heads: int, batch: int, seq_len: int, r: int, d_rope: int,
                   table, q_dtype=torch.bfloat16, name="small") -> Workload:
    return Workload(wid, name, n_layers, n_heads, batch, seq_len, r, d_rope, q_dtype,
                    layers_from_table(table, d_rope))


# ----------------------------------------------------------------------------
# Source rows for one anchor layer
# ----------------------------------------------------------------------------

def source_rows(w: Workload, layer: int, device="cpu", seqs=None):
    """fp32 source rows of one anchor layer.

    Returns (latent [B', T, r], rope [B', T, d_R], positions or None).  With
    eviction, T is the number of kept rows and the rows are those of the kept
    positions (drawn from the full nominal context, then gathered).
    """
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    if not w.nominal_context:
        lat = gen_latent(w.wid, layer, (w.batch, w.seq_len), w.r, device)
        rope = gen_rope(w.wid, layer, (w.batch, w.seq_len), w.d_rope, device)
        return lat[seqs], rope[seqs], None
    lats, ropes, poss = [], [], []
    for s in seqs:
        full_lat = gen_latent(w.wid, layer, (w.nominal_context,), w.r, device, extra=s + 1)
        full_rope = gen_rope(w.wid, layer, (w.nominal_context,), w.d_rope, device, extra=s + 1)
        pos = keep_positions(gen_scores(w.wid, s, w.nominal_context, device), w.seq_len)
        lats.append(full_lat[pos.long()])
        ropes.append(full_rope[pos.long()])
        poss.append(pos)
    return torch.stack(lats), torch.stack(ropes), torch.stack(poss)


def full_context_rows(w: Workload, layer: int, seq: int, device="cpu"):
    """Eviction workloads only: the un-evicted source rows of one sequence
    [nominal_context, r] / [nominal_context, d_R] and the kept positions."""
    lat = gen_latent(w.wid, layer, (w.nominal_context,), w.r, device, extra=seq + 1)
    rope = gen_rope(w.wid, layer, (w.nominal_context,), w.d_rope, device, extra=seq + 1)
    pos = keep_positions(gen_scores(w.wid, seq, w.nominal_context, device), w.seq_len)
    return lat, rope, pos


def queries(w: Workload, device="cpu"):
    """q_lat [L, B, H, r], q_rope [L, B, H, d_R] in the workload's q dtype."""
    ql = torch.stack([gen_q(w.wid, l, KIND_QLAT, (w.batch, w.n_heads), w.r, w.q_dtype, device)
                      for l in range(w.n_layers)])
    qr = torch.stack([gen_q(w.wid, l, KIND_QROPE, (w.batch, w.n_heads), w.d_rope, w.q_dtype, device)
                      for l in range(w.n_layers)])
    return ql.contiguous(), qr.contiguous()
