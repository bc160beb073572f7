"""GPU parity of kk_multi_decode_attn: one batch whose runs of sequences use
different tables (a context-adaptive selector picks a table per prompt), in
one fused launch, against the CPU oracle per (run, layer, sequence).

Bar as for kk_decode_attn: the caches bit-exact, each output row within
max-abs 2e-3 * max|o_oracle|.
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


def run_multi(kk, ws, lens, t_cap, split_tokens=0, max_seq_len=None):
    """ws: one Workload per run; lens: per-run lists of sequence lengths."""
    runs, qs = [], []
    for w, ln in zip(ws, lens):
        model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
        caches = build_caches(kk, model, w, t_cap, seq_lens=ln)
        runs.append((model, caches, w.batch))
        qs.append(synth.queries(w, "cuda"))
    ql = torch.cat([q[0] for q in qs], 1).contiguous()
    qr = torch.cat([q[1] for q in qs], 1).contiguous()
    flat = [x for ln in lens for x in ln]
    msl = max(flat) if max_seq_len is None else max_seq_len
    dec = kk.MultiDecoder(runs, t_cap, msl, split_tokens=split_tokens)
    dec(ql, qr, torch.tensor(flat, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return runs, dec, qs


def source_cpu(w, a, s):
    lat, rope, _ = synth.source_rows(w, a, "cuda")
    return lat[s].cpu().numpy(), rope[s].cpu().numpy()


def check(w, got, caches, q, l, s, seq_len, src):
    """Oracle for layer l, sequence s of one run (its own table and caches)."""
    a = w.layers[l].anchor
    d, b = w.d_eff(l), w.bits_eff(l)
    lat, rope = src[a]
    packed, scales, _ = ko.write_cache(lat[:seq_len], rope[:seq_len], d, b)
    codes_gpu, scales_gpu = caches[a]
    assert np.array_equal(codes_gpu[s, :seq_len].cpu().numpy(), packed)
    assert np.array_equal(scales_gpu[s, :seq_len].cpu().numpy().view(np.uint32), scales.view(np.uint32))
    q_lat = q[0][l, s].float().cpu().numpy().astype(np.float64)
    q_rope = q[1][l, s].float().cpu().numpy().astype(np.float64)
    ref = ko.decode_layer(q_lat, q_rope, packed, scales, d, w.d_rope, b, w.layers[l].sm_scale, seq_len)
    got = got.cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    if seq_len == 0:
        assert np.all(got == 0)
        return 0.0
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    if scale == 0:
        assert err == 0
        return 0.0
    assert err <= TOL * scale, f"layer {l} seq {s}: ratio {err / scale:.2e}"
    return err / scale


# Three tables of one 6-layer, 24-head model: different anchors, group sizes,
# widths and every bit width.
TABLES = [
    [[0, 64, 4], [0, 0, 0], [2, 128, 16], [3, 96, 2], [3, 0, 0], [5, 64, 8]],
    [[0, 128, 16], [1, 32, 2], [1, 0, 0], [1, 0, 0], [4, 64, 8], [5, 96, 4]],
    [[0, 96, 8], [0, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0], [5, 128, 2]],
]


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_three_tables_ragged(kk, split_tokens):
    ws = [synth.small_workload(40 + k, 6, 24, b, 320, 128, 32, t) for k, (t, b) in enumerate(zip(TABLES, (2, 1, 3)))]
    lens = [[300, 45], [1], [0, 257, 33]]
    runs, dec, qs = run_multi(kk, ws, lens, 320, split_tokens)
    worst = 0.0
    for k, w in enumerate(ws):
        for s in range(w.batch):
            src = {a: source_cpu(w, a, s) for a in w.anchors()}
            for l in range(w.n_layers):
                worst = max(worst, check(w, dec.layer_out(k, l)[s], runs[k][1], qs[k], l, s, lens[k][s], src))
    print(f"three tables split={split_tokens}: worst err ratio {worst:.2e}")


def test_runs_agree_with_single_table_calls(kk):
    """Each run's output agrees with kk_decode_attn on that run alone (same
    caches and queries) to the bar; with the same split length they agree bit
    for bit (same items, same order of arithmetic)."""
    ws = [synth.small_workload(43 + k, 6, 24, 2, 256, 128, 32, t) for k, t in enumerate(TABLES)]
    lens = [[256, 200], [130, 256], [64, 1]]
    runs, dec, qs = run_multi(kk, ws, lens, 256, split_tokens=64, max_seq_len=256)
    for k, (model, caches, b) in enumerate(runs):
        one = kk.Decoder(model, caches, b, 256, 256, split_tokens=64)
        one(qs[k][0], qs[k][1], torch.tensor(lens[k], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        for l in range(model.n_layers):
            assert torch.equal(one.layer_out(l), dec.layer_out(k, l)), f"run {k} layer {l}"


def test_one_table_per_sequence(kk):
    """n_tables = batch: every sequence has its own table (five sequences)."""
    tabs = TABLES + [[[0, 32, 16], [1, 64, 4], [2, 128, 8], [2, 0, 0], [2, 0, 0], [2, 0, 0]],
                     [[0, 128, 2], [0, 0, 0], [0, 0, 0], [3, 128, 2], [3, 0, 0], [3, 0, 0]]]
    ws = [synth.small_workload(50 + k, 6, 24, 1, 200, 128, 32, t) for k, t in enumerate(tabs)]
    lens = [[200], [17], [96], [0], [199]]
    runs, dec, qs = run_multi(kk, ws, lens, 200)
    worst = 0.0
    for k, w in enumerate(ws):
        src = {a: source_cpu(w, a, 0) for a in w.anchors()}
        for l in range(w.n_layers):
            worst = max(worst, check(w, dec.layer_out(k, l)[0], runs[k][1], qs[k], l, 0, lens[k][0], src))
    print(f"one table per sequence: worst err ratio {worst:.2e}")


def test_hetero_full_size_sampled(kk):
    """The 14B-shaped heterogeneous batch (four frozen tables, 8 sequences
    each, 8192 tokens) in the launch configuration the benchmark times; one
    layer of every bit width of every run, first and last sequence."""
    ws = synth.hetero_workloads()
    lens = [[w.seq_len] * w.batch for w in ws]
    runs, dec, qs = run_multi(kk, ws, lens, ws[0].seq_len)
    worst, n = 0.0, 0
    for k, w in enumerate(ws):
        picks = []
        for b in (2, 4, 8, 16):
            ls = [l for l in range(w.n_layers) if w.bits_eff(l) == b]
            if ls:
                picks.append(ls[(k * 7) % len(ls)])
        lat_all = {}
        for l in picks:
            a = w.layers[l].anchor
            if a not in lat_all:
                lat, rope, _ = synth.source_rows(w, a, "cuda")
                lat_all[a] = (lat[[0, w.batch - 1]].cpu().numpy(), rope[[0, w.batch - 1]].cpu().numpy())
                del lat, rope
        for l in picks:
            a = w.layers[l].anchor
            for i, s in enumerate((0, w.batch - 1)):
                src = {a: (lat_all[a][0][i], lat_all[a][1][i])}
                worst = max(worst, check(w, dec.layer_out(k, l)[s], runs[k][1], qs[k], l, s, w.seq_len, src))
                n += 1
    print(f"heterogeneous 14B batch: worst err ratio {worst:.2e} over {n} samples")


def _random_hetero_case(i):
    """Seeded random heterogeneous batch: one model shape (1-6 layers, 1-64
    heads, d_R 16-128), 2-4 runs each with its own random table (inheritance,
    widths, code widths), 1-3 sequences per run of 0-300 tokens, automatic or
    fixed splits."""
    rng = np.random.default_rng(3000 + i)
    L = int(rng.integers(1, 7))
    H = int(rng.choice([1, 4, 13, 16, 24, 32, 40, 48, 64]))
    d_rope = int(rng.choice([16, 32, 64, 128]))
    r = 256
    tables = []
    for _ in range(int(rng.integers(2, 5))):
        t, anchors = [], []
        for l in range(L):
            if l > 0 and rng.random() < 0.35:
                t.append([int(rng.choice(anchors)), 0, 0])
            else:
                t.append([l, 16 * int(rng.integers(1, min(r, 576 - d_rope) // 16 + 1)), int(rng.choice([2, 4, 8, 16]))])
                anchors.append(l)
        tables.append(t)
    batches = [int(rng.integers(1, 4)) for _ in tables]
    lens = [[int(x) for x in rng.integers(0, 301, b)] for b in batches]
    split = int(rng.choice([0, 0, 32, 128]))
    return L, H, r, d_rope, tables, batches, lens, split


@pytest.mark.parametrize("case", range(8))
def test_random_hetero_batches(kk, case):
    """Randomized sweep of kk_multi_decode_attn: every (run, layer, sequence)
    against the oracle with that run's table."""
    L, H, r, d_rope, tables, batches, lens, split = _random_hetero_case(case)
    print(f"hetero case {case}: L {L}, H {H}, d_R {d_rope}, tables {tables}, lens {lens}, split {split}", flush=True)
    ws = [synth.small_workload(400 + 10 * case + k, L, H, b, 300, r, d_rope, t)
          for k, (t, b) in enumerate(zip(tables, batches))]
    runs, dec, qs = run_multi(kk, ws, lens, 320, split)
    worst = 0.0
    for k, w in enumerate(ws):
        for s in range(w.batch):
            src = {a: source_cpu(w, a, s) for a in w.anchors()}
            for l in range(w.n_layers):
                worst = max(worst, check(w, dec.layer_out(k, l)[s], runs[k][1], qs[k], l, s, lens[k][s], src))
    print(f"hetero case {case}: worst err ratio {worst:.2e}")
