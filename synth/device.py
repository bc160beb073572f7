"""Fill a workload's anchor caches on the GPU through the library writer.

Marshalling only: draws the seeded source rows on the device and hands them to
``kk_quantize_write``; all quantization and packing happens in the library.
"""

from __future__ import annotations

import torch

from . import gen


def build_caches(kk, model, w: gen.Workload, t_cap: int | None = None, device="cuda", seq_lens=None):
    """Returns {anchor: (codes, scales)} for every anchor layer of `w`.

    Rows t < seq_lens[s] of sequence s are written (all rows by default).
    With eviction (w.nominal_context > 0) each sequence's full context is drawn
    and the kept positions are gathered by the writer's src_index path.
    """
    t_cap = t_cap or w.seq_len
    lens = [w.seq_len] * w.batch if seq_lens is None else [int(x) for x in seq_lens]
    caches = {}
    for a in w.anchors():
        codes, scales = kk.alloc_cache(model, a, w.batch, t_cap, device)
        codes.zero_()
        scales.zero_()
        if w.nominal_context:
            for s in range(w.batch):
                lat, rope, pos = gen.full_context_rows(w, a, s, device)
                n = lens[s]
                dst = s * t_cap + torch.arange(n, device=device, dtype=torch.int64)
                kk.quantize_write(model, a, lat, rope, codes, scales, dst, src_index=pos[:n].contiguous())
                del lat, rope
        else:
            lat, rope, _ = gen.source_rows(w, a, device)
            for s in range(w.batch):
                n = lens[s]
                dst = s * t_cap + torch.arange(n, device=device, dtype=torch.int64)
                kk.quantize_write(model, a, lat[s], rope[s], codes, scales, dst)
            del lat, rope
        caches[a] = (codes, scales)
    return caches


def build_gqa_caches(kk, model, w: gen.GqaWorkload, t_cap: int | None = None, device="cuda", seq_lens=None):
    """{anchor: (codes, scales)} of a grouped-query workload through the
    library writer; rows t < seq_lens[s] of sequence s are written."""
    t_cap = t_cap or w.seq_len
    lens = [w.seq_len] * w.batch if seq_lens is None else [int(x) for x in seq_lens]
    caches = {}
    for a in w.anchors():
        codes, scales = kk.gqa_alloc_cache(model, a, w.batch, t_cap, device)
        codes.zero_()
        scales.zero_()
        k, v = gen.gqa_source(w, a, device)
        for s in range(w.batch):
            n = lens[s]
            dst = s * t_cap + torch.arange(n, device=device, dtype=torch.int64)
            kk.gqa_quantize_write(model, a, k[s, :n].contiguous(), v[s, :n].contiguous(), codes, scales, dst)
        del k, v
        caches[a] = (codes, scales)
    return caches
