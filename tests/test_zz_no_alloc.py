"""kk_decode_attn_noalloc (split partials in the library's static device
array) against kk_decode_attn (caller workspace), through the C ABI.

Both run the same plan and kernels, so the outputs must agree bit for bit
(stricter than the 2e-3 * max|out| bar that kk_decode_attn itself is held to
against the oracle).  Two calls in a row, the second smaller, so the second
runs over what the first left in the array.
"""

import pytest
import torch

import synth
from synth.device import build_caches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kk():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def _setup(kk, w, lens, t_cap, split_tokens):
    model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
    caches = build_caches(kk, model, w, t_cap, seq_lens=lens)
    ql, qr = synth.queries(w, "cuda")
    dec = kk.Decoder(model, caches, w.batch, t_cap, max(lens), split_tokens=split_tokens)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return dec, ql, qr, sl


def _both(dec, ql, qr, sl):
    ref = dec(ql, qr, sl).clone()
    dec.out.fill_(float("nan"))          # the no-alloc call must write every output
    got = dec.noalloc(ql, qr, sl).clone()
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_point_two_calls(kk):
    # call 1: the 14B mixed table (48 layers, 40 heads), 32 sequences of 8192
    # tokens, automatic splits (159 MiB of partials)
    w1 = synth.workload(3)
    print("noalloc call 1: 14b_mixed_4x B=32 T=8192 auto splits", flush=True)
    dec1, ql1, qr1, sl1 = _setup(kk, w1, [w1.seq_len] * w1.batch, w1.seq_len, 0)
    assert dec1.ws_bytes <= kk.KK_NOALLOC_SCRATCH_BYTES
    ref1, got1 = _both(dec1, ql1, qr1, sl1)
    assert torch.equal(ref1, got1), f"call 1 differs: max |diff| {(ref1 - got1).abs().max().item():.3e}"
    del dec1, ql1, qr1, sl1
    torch.cuda.empty_cache()

    # call 2: a smaller mixed table, ragged lengths, 64-token splits, after call 1
    table = [[0, 128, 8], [0, 0, 0], [2, 64, 2], [3, 256, 16], [3, 0, 0], [5, 192, 4]]
    w2 = synth.small_workload(21, len(table), 40, 4, 1000, 256, 32, table)
    lens2 = [1000, 517, 33, 1]
    print("noalloc call 2: 6-layer mixed table B=4 lens [1000, 517, 33, 1] split 64", flush=True)
    dec2, ql2, qr2, sl2 = _setup(kk, w2, lens2, 1024, 64)
    assert 0 < dec2.ws_bytes < w1.batch * 1024 * 1024
    ref2, got2 = _both(dec2, ql2, qr2, sl2)
    assert torch.equal(ref2, got2), f"call 2 differs: max |diff| {(ref2 - got2).abs().max().item():.3e}"
    print(f"noalloc: both calls bit-identical to kk_decode_attn ({ref1.numel()} and {ref2.numel()} outputs)")


def test_noalloc_refuses_steps_beyond_the_array(kk):
    # two d = 512 anchors, 32 sequences of 8192 tokens in 32-token splits (64
    # per sequence) need 518 MiB of partials: refused on the host before
    # anything is enqueued, the output left as it was
    table = [[0, 512, 4], [0, 0, 0], [2, 512, 4], [2, 0, 0]]
    w = synth.small_workload(22, len(table), 40, 32, 8192, 512, 64, table)
    print("noalloc refusal: 4-layer d512 b4 B=32 T=8192 split 32", flush=True)
    dec, ql, qr, sl = _setup(kk, w, [w.seq_len] * w.batch, w.seq_len, 32)
    assert dec.ws_bytes > kk.KK_NOALLOC_SCRATCH_BYTES
    dec.out.fill_(7.0)
    with pytest.raises(kk.KKError) as e:
        dec.noalloc(ql, qr, sl)
    assert e.value.status == kk.KK_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(dec.out == 7.0)
    # the same step through kk_decode_attn with its workspace still runs
    dec(ql, qr, sl)
    torch.cuda.synchronize()
    assert torch.isfinite(dec.out).all()
