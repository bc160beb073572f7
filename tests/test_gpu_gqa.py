"""GPU parity of the grouped-query (non-MLA) precision + depth path
(kk_gqa_quantize_write, kk_gqa_decode_attn) against the CPU oracle.

Bar as for the latent cache: codes and scales bit-exact, each (layer,
sequence) output within max-abs 2e-3 * max|o_oracle|.  The oracle computes
grouped-query attention directly on separate K and V; the library runs it as
latent attention over rows [V_g || K_g], so the comparison also checks that
reformulation.
"""

import numpy as np
import pytest
import torch

from oracle import kk_oracle as ko
import synth
from synth.device import build_gqa_caches

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def kk():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def run(kk, w, lens, t_cap, split_tokens=0):
    model = kk.GqaModel(w.layers, w.n_q_heads, w.n_kv_heads, w.d_head)
    caches = build_gqa_caches(kk, model, w, t_cap, seq_lens=lens)
    q = synth.gqa_queries(w, "cuda")
    dec = kk.GqaDecoder(model, caches, w.batch, t_cap, max(lens), split_tokens=split_tokens)
    dec(q, torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return model, caches, q, dec


def check(w, caches, q, dec, l, s, seq_len, src):
    a = w.layers[l].anchor
    b = w.bits_eff(l)
    k, v = src[a]
    ck, cv, sc = ko.gqa_write_cache(k[:seq_len], v[:seq_len], b)
    codes_gpu, scales_gpu = caches[a]
    rows = ko.gqa_pack_kv_rows(ck, cv, b)                        # [T, n_kv, stride]
    got_rows = codes_gpu[s, :, :seq_len].permute(1, 0, 2).cpu().numpy()
    assert np.array_equal(got_rows, rows), f"codes differ: anchor {a} seq {s}"
    got_sc = scales_gpu[s, :, :seq_len].cpu().numpy()
    for g in range(w.n_kv_heads):
        assert np.array_equal(got_sc[g].view(np.uint32), sc.view(np.uint32)), f"scales differ: anchor {a} head {g}"
    ref = ko.gqa_decode_layer(q[l, s].float().cpu().numpy(), ck, cv, sc, w.layers[l].sm_scale, seq_len)
    got = dec.out[l, s].cpu().numpy().astype(np.float64)
    if seq_len == 0:
        assert np.all(got == 0)
        return 0.0
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    assert err <= TOL * scale, f"layer {l} seq {s}: ratio {err / scale:.2e}"
    return err / scale


# every bit width, groups of 1-3 layers
TABLE = [[0, 0, 8], [0, 0, 0], [2, 0, 2], [3, 0, 16], [3, 0, 0], [3, 0, 0], [6, 0, 4]]


@pytest.mark.parametrize("d_head,n_q,n_kv,split", [(64, 6, 2, 0), (128, 6, 2, 64), (64, 8, 8, 0),
                                                   (128, 16, 2, 0), (64, 32, 1, 96)])
def test_small_tables_ragged(kk, d_head, n_q, n_kv, split):
    """Group sizes 3, 1 (one query head per KV head), 8 and 32 (two row blocks),
    d_h 64 and 128, ragged lengths with an empty sequence, with and without
    forced splits."""
    w = synth.small_gqa_workload(70 + d_head + n_q, TABLE, n_q, n_kv, d_head, 3, 300)
    lens = [300, 0, 77]
    model, caches, q, dec = run(kk, w, lens, 320, split)
    worst = 0.0
    for s in range(w.batch):
        src = {}
        for a in w.anchors():
            k, v = synth.gqa_source(w, a, "cuda")
            src[a] = (k[s].cpu().numpy(), v[s].cpu().numpy())
        for l in range(w.n_layers):
            worst = max(worst, check(w, caches, q, dec, l, s, lens[s], src))
    print(f"gqa d_h {d_head} H {n_q} n_kv {n_kv} split {split}: worst err ratio {worst:.2e}")


def test_fp32_queries_and_inheritor_equals_anchor_call(kk):
    """fp32 queries; an inheriting layer's output equals a one-layer call on
    its anchor's cache with the inheritor's queries, bit for bit."""
    w = synth.small_gqa_workload(90, TABLE, 6, 2, 64, 2, 200, q_dtype=torch.float32)
    lens = [200, 150]
    model, caches, q, dec = run(kk, w, lens, 200, 64)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for l in (1, 4, 5):
        a = w.layers[l].anchor
        one = kk.GqaModel([kk.LayerSpec(0, w.d_head, w.layers[a].bits, w.layers[l].sm_scale)], 6, 2, 64)
        d1 = kk.GqaDecoder(one, {0: caches[a]}, 2, 200, 200, split_tokens=64)
        d1(q[l:l + 1].contiguous(), sl)
        torch.cuda.synchronize()
        assert torch.equal(d1.out[0], dec.out[l]), f"inheritor {l}"
    src = {}
    for s in range(2):
        for a in w.anchors():
            k, v = synth.gqa_source(w, a, "cuda")
            src[a] = (k[s].cpu().numpy(), v[s].cpu().numpy())
        for l in range(w.n_layers):
            check(w, caches, q, dec, l, s, lens[s], src)


def test_full_size_14b_sampled(kk):
    """The 14B grouped-query 4x table (48 layers, 40 query / 8 KV heads of 128)
    at 16 sequences x 16384 tokens, in the launch configuration the benchmark
    times; one layer of every bit width and an inheritor, first and last
    sequence."""
    w = synth.gqa_workload()
    model, caches, q, dec = run(kk, w, [w.seq_len] * w.batch, w.seq_len)
    picks = [next(l for l in range(w.n_layers) if w.bits_eff(l) == b) for b in (2, 4, 8, 16)]
    picks.append(next(l for l in range(w.n_layers) if w.layers[l].anchor != l))
    worst, n = 0.0, 0
    for l in picks:
        a = w.layers[l].anchor
        k, v = synth.gqa_source(w, a, "cuda")
        for s in (0, w.batch - 1):
            src = {a: (k[s].cpu().numpy(), v[s].cpu().numpy())}
            worst = max(worst, check(w, caches, q, dec, l, s, w.seq_len, src))
            n += 1
        del k, v
    print(f"gqa 14B: worst err ratio {worst:.2e} over {n} samples")


def _random_gqa_case(i):
    """Seeded random grouped-query table and step: d_h 64 or 128, 1-8 KV
    heads with groups of 1-32 query heads, 1-6 layers with random inheritance
    and code widths, 1-3 sequences of 0-300 tokens, automatic or fixed
    splits, bf16 or fp32 queries."""
    rng = np.random.default_rng(2000 + i)
    d_head = int(rng.choice([64, 128]))
    n_kv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 32]))
    L = int(rng.integers(1, 7))
    table, anchors = [], []
    for l in range(L):
        if l > 0 and rng.random() < 0.35:
            table.append([int(rng.choice(anchors)), 0, 0])
        else:
            table.append([l, 0, int(rng.choice([2, 4, 8, 16]))])
            anchors.append(l)
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(0, 301, B)]
    split = int(rng.choice([0, 0, 32, 96]))
    q_dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    return table, d_head, G * n_kv, n_kv, B, lens, split, q_dtype


@pytest.mark.parametrize("case", range(12))
def test_random_gqa_tables(kk, case):
    """Randomized sweep of the grouped-query path: every (layer, sequence)
    against the oracle's direct grouped-query attention."""
    table, d_head, n_q, n_kv, B, lens, split, q_dtype = _random_gqa_case(case)
    print(f"gqa case {case}: d_h {d_head}, H {n_q}, n_kv {n_kv}, table {table}, lens {lens}, split {split}, "
          f"q {q_dtype}", flush=True)
    w = synth.small_gqa_workload(300 + case, table, n_q, n_kv, d_head, B, 300, q_dtype=q_dtype)
    model, caches, q, dec = run(kk, w, lens, 320, split)
    worst = 0.0
    for s in range(w.batch):
        src = {}
        for a in w.anchors():
            k, v = synth.gqa_source(w, a, "cuda")
            src[a] = (k[s].cpu().numpy(), v[s].cpu().numpy())
        for l in range(w.n_layers):
            worst = max(worst, check(w, caches, q, dec, l, s, lens[s], src))
    print(f"gqa case {case}: worst err ratio {worst:.2e}")
