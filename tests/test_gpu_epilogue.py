"""GPU parity of kk_latent_epilogue (per-head W_UV on the kept latent
coordinates, then W_O) against the CPU oracle.

The epilogue is checked on its own input: the oracle takes the library's
decode output o_lat, so the comparison measures only the epilogue's
arithmetic.  Bar: max-abs error <= 1e-4 * max|ref| for v and y.  Derivation:
the bf16 weights enter exactly; an fp32 activation enters as hi + lo (two
round-to-nearest bf16 parts), off by at most 2^-18 of its magnitude; products
are exact in fp32 and the sums (K <= 5120 terms) accumulate in fp32, whose
rounding over such sums stays near 1e-6 of the result for these random
inputs.  1e-4 leaves a wide margin, yet a dropped head, a transposed block, a
wrong truncation or a lost low part of the activations (2^-9 error) fails it.
An end-to-end check (oracle decode + oracle epilogue against the library's
two calls) uses the decode bar, 2e-3.
"""

import numpy as np
import pytest
import torch

from oracle import kk_oracle as ko
import synth
from synth.device import build_caches

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_E2E = 2e-3


@pytest.fixture(scope="module")
def kk():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def decode_and_project(kk, w, d_v, d_model, seq_lens=None, t_cap=None):
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    t_cap = t_cap or w.seq_len
    lens = [w.seq_len] * w.batch if seq_lens is None else list(seq_lens)
    caches = build_caches(kk, model, w, t_cap, seq_lens=lens)
    ql, qr = synth.queries(w, "cuda")
    dec = kk.Decoder(model, caches, w.batch, t_cap, max(lens))
    dec(ql, qr, torch.tensor(lens, dtype=torch.int32, device="cuda"))
    wts = [synth.gen_epilogue_weights(w.wid, l, w.n_heads, d_v, w.r, d_model, "cuda") for l in range(w.n_layers)]
    v = torch.empty(w.n_layers, w.batch, w.n_heads * d_v, dtype=torch.float32, device="cuda")
    y = torch.empty(w.n_layers, w.batch, d_model, dtype=torch.float32, device="cuda")
    kk.latent_epilogue(model, w.batch, dec.out, [a for a, _ in wts], [b for _, b in wts], v, y)
    torch.cuda.synchronize()
    return model, caches, dec, ql, qr, wts, v, y


def check_layer(w, dec, wts, v, y, l, d_v):
    o = dec.layer_out(l).cpu().numpy().astype(np.float64)
    wu, wo = (t.float().cpu().numpy().astype(np.float64) for t in wts[l])
    v_ref, y_ref = ko.latent_epilogue(o, wu, wo, d_v)
    got_v = v[l].cpu().numpy().astype(np.float64).reshape(v_ref.shape)
    got_y = y[l].cpu().numpy().astype(np.float64)
    ev = np.max(np.abs(got_v - v_ref)) / max(np.max(np.abs(v_ref)), 1e-300)
    ey = np.max(np.abs(got_y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-300)
    assert ev <= TOL, f"layer {l}: v error ratio {ev:.2e}"
    assert ey <= TOL, f"layer {l}: y error ratio {ey:.2e}"
    return max(ev, ey)


def test_small_ragged_shapes(kk):
    """d_v and d_model not multiples of the 64-row wave tile, a batch that is
    not a multiple of 16, widths 32..128 (k-steps with a partial last step),
    inheriting layers with weights of their own."""
    table = [[0, 64, 4], [0, 0, 0], [2, 48, 16], [3, 128, 2], [3, 0, 0], [5, 32, 8]]
    w = synth.small_workload(60, len(table), 12, 5, 200, 128, 32, table)
    d_v, d_model = 40, 72
    model, caches, dec, ql, qr, wts, v, y = decode_and_project(kk, w, d_v, d_model, seq_lens=[200, 3, 77, 1, 150])
    worst = max(check_layer(w, dec, wts, v, y, l, d_v) for l in range(w.n_layers))
    print(f"epilogue small: worst error ratio {worst:.2e}")


@pytest.mark.parametrize("batch", [16, 40, 64, 70])
def test_batch_blocks(kk, batch):
    """One to four 16-row batch blocks per pass, and a second pass (batch > 64)."""
    table = [[0, 96, 8], [1, 128, 4]]
    w = synth.small_workload(61, 2, 8, batch, 64, 128, 32, table)
    d_v, d_model = 64, 136
    model, caches, dec, ql, qr, wts, v, y = decode_and_project(kk, w, d_v, d_model)
    worst = max(check_layer(w, dec, wts, v, y, l, d_v) for l in range(w.n_layers))
    print(f"epilogue batch {batch}: worst error ratio {worst:.2e}")


def test_end_to_end_against_oracle_decode(kk):
    """Oracle decode then oracle epilogue against the library's two calls."""
    table = [[0, 64, 8], [0, 0, 0], [2, 96, 2]]
    w = synth.small_workload(62, 3, 8, 2, 120, 128, 32, table)
    d_v, d_model = 32, 48
    model, caches, dec, ql, qr, wts, v, y = decode_and_project(kk, w, d_v, d_model)
    for l in range(w.n_layers):
        a = w.layers[l].anchor
        d, b = w.d_eff(l), w.bits_eff(l)
        lat, rope, _ = synth.source_rows(w, a, "cuda")
        wu, wo = (t.float().cpu().numpy().astype(np.float64) for t in wts[l])
        for s in range(w.batch):
            packed, scales, _ = ko.write_cache(lat[s].cpu().numpy(), rope[s].cpu().numpy(), d, b)
            o = ko.decode_layer(ql[l, s].float().cpu().numpy(), qr[l, s].float().cpu().numpy(), packed, scales,
                                d, w.d_rope, b, w.layers[l].sm_scale, w.seq_len)
            _, y_ref = ko.latent_epilogue(o[None], wu, wo, d_v)
            got = y[l, s].cpu().numpy().astype(np.float64)
            assert np.max(np.abs(got - y_ref[0])) <= TOL_E2E * np.max(np.abs(y_ref))


def test_full_size_14b_sampled(kk):
    """The 14B mixed table at full size (B = 32, T = 8192) with 14B-shaped
    projections (40 heads x d_v = 128, d_model = 5120) in the launch
    configuration the benchmark times; four layers of different widths checked
    over the whole batch."""
    w = synth.workload(3)
    d_v, d_model = 128, 5120
    model, caches, dec, ql, qr, wts, v, y = decode_and_project(kk, w, d_v, d_model)
    del caches
    picks = []
    for d in (128, 256, 384, 512):
        picks.append(next(l for l in range(w.n_layers) if w.d_eff(l) == d))
    worst = max(check_layer(w, dec, wts, v, y, l, d_v) for l in picks)
    print(f"epilogue 14B: worst error ratio {worst:.2e} over layers {picks}")
