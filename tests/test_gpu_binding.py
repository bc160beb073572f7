"""The binding's extent checks: device buffers that are too short or shaped
unlike the table are rejected with ValueError before the library is called
(the C ABI sees pointers only, so these checks are what keeps a short buffer
away from the kernels)."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kk():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def small_model(kk):
    # an anchor (d = 64, 8 bits) and one layer inheriting it; 4 heads, r = 64, d_R = 16
    return kk.Model([kk.LayerSpec(0, 64, 8, 0.1), kk.LayerSpec(0, 0, 0, 0.1)], 4, 64, 16)


def test_short_or_missing_cache_rejected(kk):
    m = small_model(kk)
    codes, scales = kk.alloc_cache(m, 0, 2, 64)
    with pytest.raises(ValueError):
        kk.Decoder(m, {0: (codes[:1], scales)}, 2, 64, 64)
    with pytest.raises(ValueError):
        kk.Decoder(m, {0: (codes, scales[:, :32])}, 2, 64, 64)
    with pytest.raises(ValueError):
        kk.Decoder(m, {}, 2, 64, 64)


def test_write_extents_rejected(kk):
    m = small_model(kk)
    codes, scales = kk.alloc_cache(m, 0, 2, 64)
    lat = torch.zeros(8, 64, device="cuda")
    rope = torch.zeros(8, 16, device="cuda")
    slots = torch.arange(8, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):       # rope rows fewer than latent rows
        kk.quantize_write(m, 0, lat, rope[:7], codes, scales, slots)
    with pytest.raises(ValueError):       # latent narrower than d
        kk.quantize_write(m, 0, lat[:, :32], rope, codes, scales, slots)
    with pytest.raises(ValueError):       # cache shorter than [batch][t_cap]
        kk.quantize_write(m, 0, lat, rope, codes[:, :32].contiguous(), scales, slots)
    with pytest.raises(ValueError):       # src_index of another length
        kk.quantize_write(m, 0, lat, rope, codes, scales, slots, src_index=torch.zeros(7, dtype=torch.int32,
                                                                                       device="cuda"))
    kk.quantize_write(m, 0, lat, rope, codes, scales, slots)   # the well-formed call goes through
    torch.cuda.synchronize()


def test_query_and_output_shapes_rejected(kk):
    m = small_model(kk)
    codes, scales = kk.alloc_cache(m, 0, 2, 64)
    dec = kk.Decoder(m, {0: (codes, scales)}, 2, 64, 64)
    ql = torch.zeros(2, 2, 4, 64, device="cuda", dtype=torch.bfloat16)
    qr = torch.zeros(2, 2, 4, 16, device="cuda", dtype=torch.bfloat16)
    sl = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dec(ql[:, :1].contiguous(), qr, sl)
    with pytest.raises(ValueError):       # q_lat and q_rope of different dtypes
        dec(ql, qr.float(), sl)
    with pytest.raises(ValueError):
        dec(ql, qr, sl[:1])
    dec(ql, qr, sl)                       # zero lengths: zeros
    torch.cuda.synchronize()
    assert torch.all(dec.out == 0)
    wu = [torch.zeros(32, 64, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    wo = [torch.zeros(8, 32, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    v = torch.empty(2, 2, 32, device="cuda")
    y = torch.empty(2, 2, 8, device="cuda")
    with pytest.raises(ValueError):       # o_lat is not the packed decode output
        kk.latent_epilogue(m, 2, dec.out[:-1], wu, wo, v, y)
    with pytest.raises(ValueError):       # W_UV of the wrong width
        kk.latent_epilogue(m, 2, dec.out, [w[:, :32].contiguous() for w in wu], wo, v, y)
    kk.latent_epilogue(m, 2, dec.out, wu, wo, v, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
