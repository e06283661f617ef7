"""INT4 with fp16 scales on the GPU (lpnh.cn/news/2042373 §2.1 run in fp16; §2.2's 16-bit
scale accounting: 4.25 bits per element for K groups of 64, 4.125 for V groups of 128).

Bar: codes and fp16 scales bit-exact against the oracle's ``quantize_int4_fp16_scale``
(prefill and append, zero groups, scales that underflow fp16, the largest fp16); dequant
bit-exact (code * scale is exact in fp32); decode attention over the cache within max abs
2e-3 and relative L2 1e-4 of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, quant
from tests.kvq_testutil import append_decode, assert_attn_close, cache_arrays, decode, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _edge_rows(k):
    """Plant the edge cases in a [B, H, S, D] fp16 tensor (in place)."""
    k[0, 0, 3] = 0.0                                   # all-zero groups
    k[0, 1, 5] = 6e-8                                  # amax / 7 underflows fp16 -> scale 1
    k[1, 0, 7, 0] = 65504.0                            # the largest fp16
    k[1, 1, 9] *= 1e-4                                 # subnormal-range scales


@pytest.mark.parametrize("D,gk,gv", [(128, 64, 128), (64, 32, 64), (256, 128, 256)])
def test_codes_and_scales_bit_exact(D, gk, gv):
    B, H, S = 2, 2, 200
    k = synth.kv_source((B, H, S, D), 181, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, S, D), 182, DEV)
    _edge_rows(k)
    desc = kvq.make_desc("int4h", B, H, D, S + 8, gk, gv)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :S - 8].contiguous(), v[:, :, :S - 8].contiguous(), 0, S - 8)
    for t in range(S - 8, S):                          # the last rows one at a time
        kvq.kvq_append(desc, dc.c, k[:, :, t].contiguous(), v[:, :, t].contiguous(), [t] * B)
    kc, ks, vc, vs = cache_arrays(dc, "int4h")
    for codes, scales, x, g in ((kc, ks, k, gk), (vc, vs, v, gv)):
        q, s = quant.quantize_int4_fp16_scale(np16(x), g)
        assert np.array_equal(scales[:, :, :S].view(np.uint16), s.view(np.uint16))
        assert np.array_equal(quant.unpack_nibbles(codes[:, :, :S]), q)
    # dequant: code * scale, exact in fp32
    out = torch.empty((B, H, S, D), dtype=torch.float32, device=DEV)
    kvq.kvq_dequant(desc, dc.c, 0, 0, S, out)
    torch.cuda.synchronize()
    q, s = quant.quantize_int4_fp16_scale(np16(k), gk)
    assert np.array_equal(out.cpu().numpy(), quant.dequantize_int4_exact(q, s, gk).astype(np.float32))


CASES = [
    # D, G, gk, gv, lens, window, num_splits
    (128, 4, 64, 128, [1000, 700], 0, 0),
    (64, 8, 32, 64, [600, 1], 0, 0),
    (256, 2, 128, 256, [900, 333], 256, 0),
    (128, 1, 64, 128, [700, 700], 0, 40),
]


@pytest.mark.parametrize("case", CASES, ids=[f"h{i}" for i in range(len(CASES))])
def test_decode_attention(case):
    D, G, gk, gv, lens, W, ns = case
    B, H = len(lens), 2
    L = max(lens)
    k = synth.kv_source((B, H, L, D), 191 + D, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, L, D), 192 + D, DEV, outlier_channels=2)
    q = synth.query((B, H * G, D), 193 + D, DEV)
    desc = kvq.make_desc("int4h", B, H, D, L, gk, gv)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, L)
    qk, sk = quant.quantize_int4_fp16_scale(np16(k), gk)
    qv, sv = quant.quantize_int4_fp16_scale(np16(v), gv)
    ref = attention.decode_attention(np16(q), quant.dequantize_int4_exact(qk, sk, gk),
                                     quant.dequantize_int4_exact(qv, sv, gv), lens, W)
    out = decode(desc, dc, q, H * G, lens, W, 0.0, ns)
    assert_attn_close(out.cpu().numpy(), ref, f"{case}")


@pytest.mark.parametrize("D,G,gk,gv", [(128, 4, 64, 128), (64, 8, 32, 64), (256, 2, 128, 256), (128, 1, 32, 32)])
def test_append_decode_step(D, G, gk, gv):
    B, H, L = 2, 2, 800
    k = synth.kv_source((B, H, L, D), 201, DEV)
    v = synth.kv_source((B, H, L, D), 202, DEV)
    q = synth.query((B, H * G, D), 203, DEV)
    desc = kvq.make_desc("int4h", B, H, D, L, gk, gv)
    dc, du = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(desc, DEV)
    for c_ in (dc, du):
        kvq.kvq_quantize_prefill(desc, c_.c, k[:, :, :L - 1].contiguous(), v[:, :, :L - 1].contiguous(), 0, L - 1)
    kn, vn = k[:, :, L - 1].contiguous(), v[:, :, L - 1].contiguous()
    out = append_decode(desc, dc, kn, vn, q, H * G, [L, L])
    # the fused step (the split-K kernel codes the new row) leaves the cache bytes of the
    # append kernel
    kvq.kvq_append(desc, du.c, kn, vn, [L - 1, L - 1])
    torch.cuda.synchronize()
    for x, y in ((dc.k_codes, du.k_codes), (dc.k_scales, du.k_scales), (dc.v_codes, du.v_codes),
                 (dc.v_scales, du.v_scales)):
        assert torch.equal(x, y)
    qk, sk = quant.quantize_int4_fp16_scale(np16(k), gk)
    qv, sv = quant.quantize_int4_fp16_scale(np16(v), gv)
    ref = attention.decode_attention(np16(q), quant.dequantize_int4_exact(qk, sk, gk),
                                     quant.dequantize_int4_exact(qv, sv, gv), [L, L])
    assert_attn_close(out.cpu().numpy(), ref, f"int4h append + decode D={D} G={G}")
