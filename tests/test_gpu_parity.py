"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bar: codes and scales bit-exact; decode output per layer (and here per
sampled (layer, sequence)) within max-abs 2e-3 * max|o_oracle|.
"""


import numpy as np
import pytest
import torch

from oracle import kk_oracle as ko
import synth
from synth.device import build_caches

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def kk():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def source_cpu(w, a, s):
    """fp32 source rows of anchor a, sequence s, exactly as the GPU side drew them."""
    if w.nominal_context:
        lat, rope, pos = synth.full_context_rows(w, a, s, "cuda")
        return lat[pos.long()].cpu().numpy(), rope[pos.long()].cpu().numpy()
    lat, rope, _ = synth.source_rows(w, a, "cuda")
    return lat[s].cpu().numpy(), rope[s].cpu().numpy()


def run_gpu(kk, w, seq_lens=None, t_cap=None, split_tokens=0):
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    t_cap = t_cap or w.seq_len
    lens = [w.seq_len] * w.batch if seq_lens is None else list(seq_lens)
    caches = build_caches(kk, model, w, t_cap, seq_lens=[min(x, t_cap) for x in lens])
    ql, qr = synth.queries(w, "cuda")
    dec = kk.Decoder(model, caches, w.batch, t_cap, max(min(max(lens), t_cap), 0), split_tokens=split_tokens)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dec(ql, qr, sl)
    torch.cuda.synchronize()
    return model, caches, dec, ql, qr


def check_layer_seq(w, dec, caches, ql, qr, l, s, seq_len, src_cache=None):
    a = w.layers[l].anchor
    d, b = w.d_eff(l), w.bits_eff(l)
    if src_cache is not None and a in src_cache:
        lat, rope = src_cache[a]
    else:
        lat, rope = source_cpu(w, a, s)
    packed, scales, _ = ko.write_cache(lat[:seq_len], rope[:seq_len], d, b)
    # writer parity (bit-exact) on the rows this sequence holds
    codes_gpu, scales_gpu = caches[a]
    assert np.array_equal(codes_gpu[s, :seq_len].cpu().numpy(), packed), f"codes differ: anchor {a} seq {s}"
    assert np.array_equal(scales_gpu[s, :seq_len].cpu().numpy().view(np.uint32), scales.view(np.uint32))
    q_lat = ql[l, s].float().cpu().numpy().astype(np.float64)
    q_rope = qr[l, s].float().cpu().numpy().astype(np.float64)
    ref = ko.decode_layer(q_lat, q_rope, packed, scales, d, w.d_rope, b, w.layers[l].sm_scale, seq_len)
    got = dec.layer_out(l)[s].cpu().numpy().astype(np.float64)
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if scale == 0:
        assert err == 0
    else:
        assert err <= TOL * scale, f"layer {l} seq {s}: err {err:.3e} vs {TOL} * {scale:.3e} (ratio {err / scale:.2e})"
    return err / scale if scale else 0.0


def test_tiny_workload_full(kk):
    w = synth.workload(0)
    model, caches, dec, ql, qr = run_gpu(kk, w)
    r = check_layer_seq(w, dec, caches, ql, qr, 0, 0, 256)
    print(f"tiny: err ratio {r:.2e}")


# A mixed table that spans every bit width, widths from 64 to 256, inheriting
# groups of 1-3 layers (group rows 40..120 span 1-2 row chunks).
MIXED_SMALL = [[0, 128, 8], [0, 0, 0], [2, 64, 2], [3, 256, 16], [3, 0, 0], [3, 0, 0], [6, 192, 4],
               [7, 256, 2], [8, 64, 16], [8, 0, 0]]


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_mixed_small_ragged_full(kk, split_tokens):
    w = synth.small_workload(10, len(MIXED_SMALL), 40, 4, 1000, 256, 32, MIXED_SMALL)
    lens = [1000, 517, 33, 1]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=1024, split_tokens=split_tokens)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"mixed small split={split_tokens}: worst err ratio {worst:.2e}")


def test_edge_lengths_and_empty(kk):
    table = [[0, 64, 4], [1, 32, 8], [1, 0, 0]]
    w = synth.small_workload(11, 3, 24, 6, 70, 64, 16, table)
    lens = [0, 1, 31, 32, 33, 70]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=72)
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(3):
            if lens[s] == 0:
                assert torch.all(dec.layer_out(l)[s] == 0)
            else:
                check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src)


def test_max_seq_len_is_a_hint_and_lengths_clamp(kk):
    """max_seq_len only sets the split count: with a hint below the real
    lengths (or 0) every token is still attended; seq_lens above t_cap are
    clamped to t_cap (the caches hold t_cap rows)."""
    table = [[0, 64, 8], [0, 0, 0], [2, 96, 16], [3, 64, 2]]
    w = synth.small_workload(18, 4, 16, 3, 256, 128, 32, table)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = build_caches(kk, model, w, 256)
    ql, qr = synth.queries(w, "cuda")
    lens = [256, 200, 1000]                         # the last one clamps to t_cap = 256
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for hint in (0, 64, 256):
        dec = kk.Decoder(model, caches, 3, 256, hint)
        dec(ql, qr, sl)
        torch.cuda.synchronize()
        for s_ in range(3):
            src = {a: source_cpu(w, a, s_) for a in w.anchors()}
            for l in range(w.n_layers):
                check_layer_seq(w, dec, caches, ql, qr, l, s_, min(lens[s_], 256), src)


def test_deterministic_and_split_invariant(kk):
    w = synth.small_workload(12, len(MIXED_SMALL), 40, 2, 700, 256, 32, MIXED_SMALL)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = build_caches(kk, model, w)
    ql, qr = synth.queries(w, "cuda")
    sl = torch.full((w.batch,), 700, dtype=torch.int32, device="cuda")
    outs = []
    for st in (0, 0, 96, 32):
        dec = kk.Decoder(model, caches, w.batch, 700, 700, split_tokens=st)
        dec(ql, qr, sl)
        outs.append(dec.out.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    # different split choices round P' differently (per-split maxima and scale
    # exponents); each is within the bar of the oracle, so they agree within it
    for o in outs[2:]:
        rel = (o - outs[0]).abs().max() / outs[0].abs().max()
        assert rel < TOL


def test_inheritor_equals_one_layer_call_on_anchor_cache(kk):
    w = synth.small_workload(13, len(MIXED_SMALL), 40, 2, 300, 256, 32, MIXED_SMALL)
    model, caches, dec, ql, qr = run_gpu(kk, w, split_tokens=64)
    sl = torch.full((w.batch,), 300, dtype=torch.int32, device="cuda")
    for l in (1, 4, 5, 9):
        a = w.layers[l].anchor
        spec = w.layers[a]
        one = kk.Model([kk.LayerSpec(0, spec.d, spec.bits, w.layers[l].sm_scale)], w.n_heads, w.r, w.d_rope)
        d1 = kk.Decoder(one, {0: caches[a]}, w.batch, 300, 300, split_tokens=64)
        d1(ql[l:l + 1].contiguous(), qr[l:l + 1].contiguous(), sl)
        torch.cuda.synchronize()
        assert torch.equal(d1.layer_out(0), dec.layer_out(l)), f"inheritor {l}"


@pytest.mark.parametrize("heads", [64, 100, 128])
def test_many_heads_row_chunks(kk, heads):
    """More heads than one item's 48 rows: 48-row chunks that cross layer
    boundaries inside an inheriting group (64 heads: 48 + 16 rows per layer;
    100 and 128 heads: chunks straddling layers of a 3-layer group)."""
    table = [[0, 256, 4], [0, 0, 0], [2, 128, 16], [3, 192, 8], [3, 0, 0], [3, 0, 0]]
    w = synth.small_workload(16, len(table), heads, 2, 300, 256, 64, table)
    lens = [300, 77]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=320)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"heads {heads}: worst err ratio {worst:.2e}")


def limits_table():
    """64 layers (the table limit) in four anchor groups of 20, 11, 10 and 23
    layers; widths 448 and 256 with d_R = 128, so K = 576 (the K limit) for
    the wide anchors; every bit width."""
    table = [[0, 448, 4]] + [[0, 0, 0]] * 19
    table += [[20, 448, 16]] + [[20, 0, 0]] * 10
    table += [[31, 256, 2]] + [[31, 0, 0]] * 9
    table += [[41, 448, 8]] + [[41, 0, 0]] * 22
    assert len(table) == 64
    return table


@pytest.mark.parametrize("heads", [1, 3])
def test_limits_64_layers_rope_128_k_576(kk, heads):
    """The largest table and RoPE width: 64 layers, d_R = 128 with d = 448
    (K = 576), r = 512 > d; one or three heads, so that a group's inheriting
    layers fill 48-row chunks across layer boundaries (1 head: 20 layers in one
    chunk; 3 heads: 69 rows of the last group in chunks of 48 + 21)."""
    table = limits_table()
    w = synth.small_workload(19, len(table), heads, 2, 100, 512, 128, table)
    lens = [100, 33]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=128)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"limits, {heads} heads: worst err ratio {worst:.2e}")


def test_fp32_queries_at_full_k(kk):
    """fp32 queries (every chunk's query loaded in one round trip) at the
    largest K = 512 + 64 with 40 heads (three row blocks), every bit width,
    an inheriting layer; ragged lengths."""
    table = [[0, 512, 16], [1, 512, 8], [2, 448, 4], [2, 0, 0], [4, 512, 2]]
    w = synth.small_workload(21, len(table), 40, 2, 200, 512, 64, table, q_dtype=torch.float32)
    lens = [200, 45]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=224)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"fp32 queries, K = 576: worst err ratio {worst:.2e}")


def test_most_splits_per_sequence(kk):
    """Two long sequences and few rows: the planner cuts each sequence into
    the most splits it allows (64, checked through the workspace size), so the
    merge combines 64 partials per output; the second length is ragged."""
    table = [[0, 64, 4], [1, 32, 8]]
    w = synth.small_workload(22, len(table), 4, 2, 16384, 64, 16, table)
    lens = [16384, 9001]
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    slot_bytes = lambda d: (32 * d + 192) * 4       # fp16 O/l of 64 rows, then m, l and the unit
    assert kk.workspace_bytes(model, w.batch, 16384) == 64 * w.batch * (slot_bytes(64) + slot_bytes(32))
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"64 splits: worst err ratio {worst:.2e}")


def test_softmax_scale_sign_zero_and_extremes(kk):
    """Per-layer softmax scales that are negative (the logits flip sign), zero
    (uniform weights), tiny, and large (close to an argmax), on ragged lengths
    so that the masked last tile meets each of them."""
    from synth.gen import LayerSpec
    table = [[0, 64, 4], [0, 0, 0], [0, 0, 0], [3, 128, 16], [3, 0, 0], [5, 96, 2]]
    w = synth.small_workload(13, len(table), 24, 2, 300, 128, 32, table)
    scales = [-0.09, 0.0, 0.9, -1.5, 1e-30, -0.2]
    w.layers = [LayerSpec(x.anchor, x.d, x.bits, sc) for x, sc in zip(w.layers, scales)]
    lens = [300, 45]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=320)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"softmax scales: worst err ratio {worst:.2e}")


def test_append_then_attend(kk):
    """kk_append_decode writes each sequence's next token into every anchor
    cache (row seq_lens[s] - 1 of the lengths after the append) and decodes: the
    caches equal the plain writer's for the new lengths, the output equals a
    separate kk_decode_attn on them bit for bit, and both match the oracle.
    A sequence of length 0 after the append writes nothing and gives zeros."""
    table = [[0, 96, 4], [0, 0, 0], [2, 64, 16], [3, 128, 2], [3, 0, 0], [5, 64, 8]]
    w = synth.small_workload(14, len(table), 24, 5, 128, 128, 32, table, q_dtype=torch.float32)
    before, after = [100, 31, 0, 127, 0], [101, 32, 1, 128, 0]
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = build_caches(kk, model, w, 128, seq_lens=before)
    new_lat = torch.zeros(w.n_layers, w.batch, w.r, dtype=torch.float32, device="cuda")
    new_rope = torch.zeros(w.n_layers, w.batch, w.d_rope, dtype=torch.float32, device="cuda")
    for a in w.anchors():
        lat, rope, _ = synth.source_rows(w, a, "cuda")
        for s in range(w.batch):
            if after[s] > 0:
                new_lat[a, s] = lat[s, after[s] - 1]
                new_rope[a, s] = rope[s, after[s] - 1]
    ql, qr = synth.queries(w, "cuda")
    sl = torch.tensor(after, dtype=torch.int32, device="cuda")
    dec = kk.Decoder(model, caches, w.batch, 128, 128)
    dec.append(new_lat, new_rope, ql, qr, sl)
    torch.cuda.synchronize()
    ref_caches = build_caches(kk, model, w, 128, seq_lens=after)
    for a in w.anchors():
        assert torch.equal(caches[a][0], ref_caches[a][0]), f"codes of anchor {a}"
        assert torch.equal(caches[a][1].view(torch.int32), ref_caches[a][1].view(torch.int32)), f"scales of anchor {a}"
    ref = kk.Decoder(model, ref_caches, w.batch, 128, 128)
    ref(ql, qr, sl)
    torch.cuda.synchronize()
    assert torch.equal(dec.out, ref.out)
    worst = 0.0
    for s in range(w.batch):
        if after[s] == 0:
            for l in range(w.n_layers):
                assert torch.all(dec.layer_out(l)[s] == 0)
            continue
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, after[s], src))
    print(f"append then attend: worst err ratio {worst:.2e}")


def test_append_then_attend_full_size_sampled(kk):
    """The 14B mixed table at full size in the configuration bench.py --append
    times: caches hold 8191 tokens, kk_append_decode writes token 8191 of
    every sequence into every anchor and decodes over 8192; the new rows are
    bit-exact and sampled outputs match the oracle over the full context."""
    w = synth.workload(3)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    T = w.seq_len
    caches = build_caches(kk, model, w, T, seq_lens=[T - 1] * w.batch)
    new_lat = torch.zeros(w.n_layers, w.batch, w.r, dtype=torch.float32, device="cuda")
    new_rope = torch.zeros(w.n_layers, w.batch, w.d_rope, dtype=torch.float32, device="cuda")
    for a in w.anchors():
        lat, rope, _ = synth.source_rows(w, a, "cuda")
        new_lat[a] = lat[:, T - 1]
        new_rope[a] = rope[:, T - 1]
        del lat, rope
    ql, qr = synth.queries(w, "cuda")
    sl = torch.full((w.batch,), T, dtype=torch.int32, device="cuda")
    dec = kk.Decoder(model, caches, w.batch, T, T)
    dec.append(new_lat, new_rope, ql, qr, sl)
    torch.cuda.synchronize()
    picks = [next(l for l in range(w.n_layers) if w.bits_eff(l) == b) for b in (2, 4, 8, 16)]
    worst = 0.0
    for i, l in enumerate(picks):
        s_ = 0 if i % 2 == 0 else w.batch - 1
        worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s_, T))
    print(f"append full size: worst err ratio {worst:.2e}")


def test_outliers_and_zero_tokens(kk):
    table = [[0, 128, 2], [1, 128, 4], [2, 128, 8], [3, 128, 16]]
    w = synth.small_workload(14, 4, 16, 1, 200, 128, 32, table)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = {}
    src = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    for a in w.anchors():
        lat = torch.randn(200, 128, generator=g, device="cuda")
        rope = torch.randn(200, 32, generator=g, device="cuda")
        mask = torch.rand(200, 128, generator=g, device="cuda") < 1e-3
        lat = torch.where(mask, lat * 20, lat)
        lat[5] = 0
        rope[5] = 0                                    # an all-zero token: scale 0, codes 0
        lat[7] *= 1e-20                                # a tiny-magnitude token
        codes, scales = kk.alloc_cache(model, a, 1, 200)
        kk.quantize_write(model, a, lat, rope, codes, scales, torch.arange(200, device="cuda"))
        caches[a] = (codes, scales)
        src[a] = (lat.cpu().numpy(), rope.cpu().numpy())
    ql, qr = synth.queries(w, "cuda")
    ql[2, 0, 3] = 0
    qr[2, 0, 3] = 0                                    # a head with q = 0: uniform weights
    dec = kk.Decoder(model, caches, 1, 200, 200)
    dec(ql, qr, torch.tensor([200], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for l in range(4):
        check_layer_seq(w, dec, caches, ql, qr, l, 0, 200, src)


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_largest_integer_scores(kk, split_tokens):
    """The largest integer Q.K scores the kernel can meet: d = 512 with d_R = 64
    (K = 576), every cache element +-1 (so every code is +-qmax) and every query
    element 1 (so every fixed-point query element is at its maximum, 16256),
    40 heads (three row blocks), each bit width.  The latent score then reaches
    about 2^30 in int32 (|256 hi + lo| summed over 512 features), half the
    int32 range.  Tokens carry a seeded sign, so the logits are +-24 and the
    softmax sits on the positive tokens; 200 tokens span several tiles and a
    ragged tail.  Compared with the oracle like every other case."""
    table = [[0, 512, 2], [1, 512, 4], [2, 512, 8], [3, 512, 16]]
    T = 200
    w = synth.small_workload(15, 4, 40, 1, T, 512, 64, table)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    sign = torch.where(torch.rand(T, 1, generator=g, device="cuda") < 0.5, -1.0, 1.0)
    lat = sign.expand(T, 512).contiguous()
    rope = sign.expand(T, 64).contiguous()
    caches, src = {}, {}
    for a in w.anchors():
        codes, scales = kk.alloc_cache(model, a, 1, T)
        kk.quantize_write(model, a, lat, rope, codes, scales, torch.arange(T, device="cuda"))
        caches[a] = (codes, scales)
        src[a] = (lat.cpu().numpy(), rope.cpu().numpy())
    ql = torch.ones(4, 1, 40, 512, dtype=torch.bfloat16, device="cuda")
    qr = torch.ones(4, 1, 40, 64, dtype=torch.bfloat16, device="cuda")
    dec = kk.Decoder(model, caches, 1, T, T, split_tokens=split_tokens)
    dec(ql, qr, torch.tensor([T], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    worst = 0.0
    for l in range(4):
        worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, 0, T, src))
    print(f"largest integer scores, split_tokens {split_tokens}: worst err ratio {worst:.2e}")


def test_zero_tokens_at_item_start_and_all_zero_sequences(kk):
    """Tokens whose stored values are all zero have scale 0 and score 0; they
    still weigh in the softmax.  Sequence 0 is all zero tokens (the output is
    0), sequence 1 starts with 40 of them (the first tile of an item is all
    zero), sequence 2 has them at the end; every bit width, with and without
    splits."""
    table = [[0, 128, 2], [1, 128, 4], [2, 128, 8], [3, 128, 16], [3, 0, 0]]
    w = synth.small_workload(17, 5, 16, 3, 300, 128, 32, table)
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    caches, src = {}, {}
    for a in w.anchors():
        lat = torch.randn(3, 300, 128, generator=g, device="cuda")
        rope = torch.randn(3, 300, 32, generator=g, device="cuda")
        lat[0] = 0
        rope[0] = 0
        lat[1, :40] = 0
        rope[1, :40] = 0
        lat[2, 250:] = 0
        rope[2, 250:] = 0
        codes, scales = kk.alloc_cache(model, a, 3, 300)
        for s_ in range(3):
            kk.quantize_write(model, a, lat[s_].contiguous(), rope[s_].contiguous(), codes, scales,
                              s_ * 300 + torch.arange(300, device="cuda"))
        caches[a] = (codes, scales)
        src[a] = [(lat[s_].cpu().numpy(), rope[s_].cpu().numpy()) for s_ in range(3)]
    ql, qr = synth.queries(w, "cuda")
    sl = torch.full((3,), 300, dtype=torch.int32, device="cuda")
    for st in (0, 64):
        dec = kk.Decoder(model, caches, 3, 300, 300, split_tokens=st)
        dec(ql, qr, sl)
        torch.cuda.synchronize()
        assert torch.isfinite(dec.out).all(), f"split {st}: non-finite output"
        for s_ in range(3):
            for l in range(w.n_layers):
                a = w.layers[l].anchor
                if s_ == 0:
                    assert torch.all(dec.layer_out(l)[0] == 0)
                    continue
                check_layer_seq(w, dec, caches, ql, qr, l, s_, 300, {a: src[a][s_]})


def test_b16_full_rank_matches_unquantized_attention(kk):
    table = [[0, 256, 16]]
    w = synth.small_workload(15, 1, 28, 2, 2048, 256, 64, table)
    model, caches, dec, ql, qr = run_gpu(kk, w)
    for s in range(2):
        lat, rope = source_cpu(w, 0, s)
        src = np.concatenate([lat, rope], 1).astype(np.float64)
        q = np.concatenate([ql[0, s].float().cpu().numpy(), qr[0, s].float().cpu().numpy()], 1).astype(np.float64)
        ref = ko.attend(q, src, 256, w.layers[0].sm_scale)
        got = dec.layer_out(0)[s].cpu().numpy()
        assert np.max(np.abs(got - ref)) <= TOL * np.max(np.abs(ref))


# Queries whose latent and RoPE parts differ widely in size (or that carry one
# outlier coordinate per row): the kernel rounds each part of a row to a 15-bit
# fixed-point number with its own prescale, so the bar holds across this range.
QRANGE_TABLE = [[0, 512, 2], [1, 384, 4], [1, 0, 0], [3, 256, 8], [4, 128, 16], [4, 0, 0], [6, 512, 16]]


def _scale_queries(kind, ql, qr):
    """Power-of-two scalings (exact in bf16) of seeded N(0, 1) queries."""
    ql, qr = ql.clone(), qr.clone()
    L, B, H, r = ql.shape
    if kind == "rope_x64":
        qr *= 64
    elif kind == "rope_x256":
        qr *= 256
    elif kind == "lat_x64":
        ql *= 64
    elif kind == "lat_outlier_x64":
        for l in range(L):
            for h in range(H):
                ql[l, :, h, (7 * h + 3 * l) % 128] *= 64
    elif kind == "rope_outlier_x64":
        for l in range(L):
            for h in range(H):
                qr[l, :, h, (5 * h + l) % qr.shape[-1]] *= 64
    return ql.contiguous(), qr.contiguous()


@pytest.mark.parametrize("split_tokens", [0, 256])
@pytest.mark.parametrize("kind", ["rope_x64", "rope_x256", "lat_x64", "lat_outlier_x64", "rope_outlier_x64"])
def test_query_dynamic_range(kk, kind, split_tokens):
    w = synth.small_workload(23, len(QRANGE_TABLE), 40, 2, 2048, 512, 64, QRANGE_TABLE)
    lens = [2048, 1333]
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = build_caches(kk, model, w, 2048, seq_lens=lens)
    ql, qr = _scale_queries(kind, *synth.queries(w, "cuda"))
    dec = kk.Decoder(model, caches, w.batch, 2048, 2048, split_tokens=split_tokens)
    dec(ql, qr, torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"query range {kind}, split_tokens {split_tokens}: worst err ratio {worst:.2e}")


@pytest.mark.parametrize("split_tokens", [0, 64])
@pytest.mark.parametrize("d_rope,table", [
    (32, [[0, 48, 2], [1, 80, 4], [2, 208, 8], [2, 0, 0], [4, 48, 16], [5, 80, 16]]),
    (80, [[0, 64, 2], [1, 448, 4], [2, 16, 8], [3, 448, 16], [3, 0, 0]]),
])
def test_widths_off_the_64_grid(kk, d_rope, table, split_tokens):
    """Kept widths that are odd multiples of 16 (the last 32-wide P.V unit half
    filled) and RoPE widths that are not multiples of 64 (the RoPE chunk reads
    past the row), every bit width, split and unsplit, ragged lengths."""
    w = synth.small_workload(24, len(table), 40, 2, 300, 512, d_rope, table)
    lens = [300, 97]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=320, split_tokens=split_tokens)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"widths off the 64 grid (d_R {d_rope}, split {split_tokens}): worst err ratio {worst:.2e}")


# Every bit width in one table.  NARROW keeps d <= 256, so 16- and 28-head
# tables run the lean register budget; WIDE has d = 512 anchors, which need
# the full one.
ROWS_NARROW = [[0, 256, 16], [1, 128, 8], [1, 0, 0], [3, 192, 4], [4, 64, 2]]
ROWS_WIDE = [[0, 512, 2], [1, 512, 16], [2, 256, 8], [3, 128, 4], [3, 0, 0]]


@pytest.mark.parametrize("split_tokens", [0, 64])
@pytest.mark.parametrize("r,table", [(256, ROWS_NARROW), (512, ROWS_WIDE)], ids=["narrow", "wide"])
@pytest.mark.parametrize("heads", [16, 28, 40])
def test_row_blocks_by_bit_width(kk, heads, r, table, split_tokens):
    """One, two and three 16-row Q.K blocks per item (16, 28 and 40 heads),
    each with every bit width: the tile copies are shared out between the
    Q.K and P.V waves differently for each block count and for narrow
    (b <= 4) and wide codes.  Ragged lengths, one a single token."""
    w = synth.small_workload(25, len(table), heads, 3, 300, r, 64, table)
    lens = [300, 97, 1]
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=320, split_tokens=split_tokens)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"row blocks ({heads} heads, r {r}, split {split_tokens}): worst err ratio {worst:.2e}")


def _random_case(i):
    """Seeded random table and step: head count (1 to 72, across the one-,
    two- and three-block items and the 48-row chunks that cross layers),
    1-6 layers with random inheritance, any d <= r (multiple of 16), every
    code width, d_R in {16, 32, 64, 128}, 1-4 sequences of 0-300 tokens,
    automatic or fixed splits, bf16 or fp32 queries."""
    rng = np.random.default_rng(1000 + i)
    H = int(rng.choice([1, 2, 5, 8, 13, 16, 20, 24, 31, 32, 36, 40, 47, 48, 56, 64, 72]))
    L = int(rng.integers(1, 7))
    d_rope = int(rng.choice([16, 32, 64, 128]))
    r = int(rng.choice([256, 512]))
    table, anchors = [], []
    for l in range(L):
        if l > 0 and rng.random() < 0.35:
            table.append([int(rng.choice(anchors)), 0, 0])
        else:
            d = 16 * int(rng.integers(1, min(r, 576 - d_rope) // 16 + 1))
            table.append([l, d, int(rng.choice([2, 4, 8, 16]))])
            anchors.append(l)
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 301, B)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.choice([0, 1, 31, 32, 33]))
    split = int(rng.choice([0, 0, 32, 64, 128]))
    q_dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    return table, H, r, d_rope, B, lens, split, q_dtype


@pytest.mark.parametrize("case", range(24))
def test_random_tables(kk, case):
    """Randomized sweep: every (layer, sequence) of a seeded random table
    against the oracle, codes and scales bit-exact."""
    table, H, r, d_rope, B, lens, split, q_dtype = _random_case(case)
    print(f"case {case}: H {H}, table {table}, r {r}, d_R {d_rope}, lens {lens}, split {split}, q {q_dtype}",
          flush=True)
    w = synth.small_workload(40 + case, len(table), H, B, 300, r, d_rope, table, q_dtype=q_dtype)
    model, caches, dec, ql, qr = run_gpu(kk, w, seq_lens=lens, t_cap=320, split_tokens=split)
    worst = 0.0
    for s in range(w.batch):
        src = {a: source_cpu(w, a, s) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, lens[s], src))
    print(f"case {case}: worst err ratio {worst:.2e}")


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_full_size_workloads_every_anchor_and_layer(kk, wid):
    """The four full-size workloads in the configuration bench.py times
    (automatic splits): every anchor's codes and scales bit-exact on the first
    and the last sequence, and every layer's output within the bar on one
    sequence (layer l on sequence l mod B, so the layers of a group meet
    different sequences)."""
    w = synth.workload(wid)
    model, caches, dec, ql, qr = run_gpu(kk, w)
    anchors = w.anchors()
    seqs_for_codes = (0, w.batch - 1)
    src = {}
    for a in anchors:
        for s in seqs_for_codes:
            src[(a, s)] = source_cpu(w, a, s)
    n_codes = 0
    for a in anchors:
        for s in seqs_for_codes:
            lat, rope = src[(a, s)]
            packed, scales, _ = ko.write_cache(lat, rope, w.layers[a].d, w.layers[a].bits)
            codes_gpu, scales_gpu = caches[a]
            assert np.array_equal(codes_gpu[s].cpu().numpy(), packed), f"codes differ: anchor {a} seq {s}"
            assert np.array_equal(scales_gpu[s].cpu().numpy().view(np.uint32), scales.view(np.uint32)), \
                f"scales differ: anchor {a} seq {s}"
            n_codes += 1
    worst, n_out = 0.0, 0
    for l in range(w.n_layers):
        s = l % w.batch
        a = w.layers[l].anchor
        lat_rope = src.get((a, s)) or source_cpu(w, a, s)
        worst = max(worst, check_layer_seq(w, dec, caches, ql, qr, l, s, w.seq_len, {a: lat_rope}))
        n_out += 1
    assert n_codes == 2 * len(anchors) and n_out == w.n_layers
    print(f"workload {wid} ({w.name}): codes and scales of {len(anchors)} anchors x 2 sequences bit-exact; "
          f"{n_out} of {w.n_layers} layers within the bar, worst err ratio {worst:.2e}")
