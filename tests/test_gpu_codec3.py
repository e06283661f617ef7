"""GPU parity of the WHT + Lloyd-Max codec at 3 bits ("长上下文内存大瘦身：LARQL 四大 KV 缓存
引擎原理与横向对比", pwwt.cn/news/5725003, engine three: 3 or 4 bits) against the oracle.

Rows hold the 3-bit indices packed back to back (index i in bits 3i .. 3i + 2 of the row
as a little-endian bit string, 3D/8 bytes).  Bar as for the 4-bit codec: index mismatches only where y/s
lies within 1e-5 of a decision threshold; scales and decoded values within 1e-5
relative; attention over the same codes within max abs 2e-3 and relative L2 1e-4.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, codec
from tests.kvq_testutil import (append_decode, assert_attn_close, cache_arrays, codec_hat_from_device,
                                decode, np16, pack3, unpack3)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _encode(k, v, cap=None):
    B, H, S, D = k.shape
    desc = kvq.make_desc("codec3", B, H, D, cap or S)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, S)
    return desc, dc


def _check_codes(got_codes, got_scales, x16):
    idx, s, u = codec.encode(x16, bits=3)
    g_idx = unpack3(got_codes)
    assert np.allclose(got_scales[..., 0], s, rtol=1e-5, atol=0)
    mism = g_idx != idx
    if mism.any():
        _, thr, _ = codec.codebook(3)
        d = np.min(np.abs(u[mism][:, None] - thr[None, :]), axis=1)
        assert np.all(d <= 1e-5), f"{int((d > 1e-5).sum())} codes differ away from a threshold"
    assert g_idx.max() <= 7
    return int(mism.sum())


@pytest.mark.parametrize("D", [64, 128, 256])
def test_encode_boundary_rule_3bit(D):
    k = synth.kv_source((2, 4, 300, D), 151, DEV)
    v = synth.kv_source((2, 4, 300, D), 152, DEV, outlier_channels=2, zero_groups=((1, 3, 7, 0, D),))
    desc, dc = _encode(k, v)
    kc, ks, vc, vs = cache_arrays(dc, "codec3")
    _check_codes(kc, ks, np16(k))
    _check_codes(vc, vs, np16(v))
    assert vs[1, 3, 7, 0] == 0.0


def test_dequant_3bit():
    D = 128
    k = synth.kv_source((2, 4, 100, D), 153, DEV)
    v = synth.kv_source((2, 4, 100, D), 154, DEV)
    desc, dc = _encode(k, v)
    kc, ks, _, _ = cache_arrays(dc, "codec3")
    out = torch.empty((2, 4, 100, D), dtype=torch.float32, device=DEV)
    kvq.kvq_dequant(desc, dc.c, 0, 0, 100, out)
    torch.cuda.synchronize()
    ref = codec.decode(unpack3(kc), ks[..., 0], bits=3)
    got = out.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    # coarser than the 4-bit codec's ~0.9954, as the 3-bit distortion is larger
    cos = codec.row_cosine(np16(k).astype(np.float64), got).mean()
    assert 0.97 < cos < 0.99, cos


def _inject(dc, kidx, ks, vidx, vs):
    dc.k_codes.copy_(torch.from_numpy(pack3(kidx).reshape(-1)).to(DEV))
    dc.v_codes.copy_(torch.from_numpy(pack3(vidx).reshape(-1)).to(DEV))
    dc.k_scales.copy_(torch.from_numpy(np.ascontiguousarray(ks).reshape(-1)).to(DEV))
    dc.v_scales.copy_(torch.from_numpy(np.ascontiguousarray(vs).reshape(-1)).to(DEV))


@pytest.mark.parametrize("window,L,cap,D,G,ns", [(0, 700, 700, 256, 2, 0), (256, 700, 256, 128, 4, 0),
                                                 (1024, 4097, 1024, 256, 2, 0), (0, 900, 900, 64, 8, 40)])
def test_attention_over_oracle_codes_3bit(window, L, cap, D, G, ns):
    """Decode attention on a cache holding the oracle's own 3-bit codes, global and in
    window rings, merged in-kernel and (40 splits) by the merge kernel."""
    B, H = 2, 2
    k = synth.kv_source((B, H, L, D), 160 + L, DEV)
    v = synth.kv_source((B, H, L, D), 161 + L, DEV)
    q = synth.query((B, H * G, D), 162 + L, DEV)
    kidx, ks, _ = codec.encode(np16(k), bits=3)
    vidx, vs, _ = codec.encode(np16(v), bits=3)
    desc = kvq.make_desc("codec3", B, H, D, cap)
    dc = kvq.DeviceCache(desc, DEV)
    slots = np.arange(L) % cap
    keep = np.arange(max(0, L - cap), L)
    ring = lambda a: a[:, :, keep][:, :, np.argsort(slots[keep])]  # noqa: E731
    _inject(dc, ring(kidx), ring(ks), ring(vidx), ring(vs))
    out = decode(desc, dc, q, H * G, [L, L], window, 0.0, ns)
    ref = attention.decode_attention(np16(q), codec.decode(kidx, ks, bits=3),
                                     codec.decode(vidx, vs, bits=3), [L, L], window)
    assert_attn_close(out.cpu().numpy(), ref, f"codec3 w={window} D={D}")


@pytest.mark.parametrize("D,G,window", [(256, 2, 0), (128, 4, 512)])
def test_fused_append_decode_3bit(D, G, window):
    """The split-K kernel codes the new row (as the encode kernel does), stores its packed bits
    and attends it; against the oracle and against the unfused pair."""
    B, H, L = 2, 2, 1500
    cap = window or L
    k = synth.kv_source((B, H, L, D), 171, DEV)
    v = synth.kv_source((B, H, L, D), 172, DEV)
    q = synth.query((B, H * G, D), 173, DEV)
    desc = kvq.make_desc("codec3", B, H, D, cap)
    dc, du = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(desc, DEV)
    lo = max(0, L - 1 - cap)
    for c_ in (dc, du):
        kvq.kvq_quantize_prefill(desc, c_.c, k[:, :, lo:L - 1].contiguous(), v[:, :, lo:L - 1].contiguous(),
                                 lo, L - 1 - lo)
    kn, vn = k[:, :, L - 1].contiguous(), v[:, :, L - 1].contiguous()
    out = append_decode(desc, dc, kn, vn, q, H * G, [L, L], window)
    kvq.kvq_append(desc, du.c, kn, vn, [L - 1, L - 1])
    out_u = decode(desc, du, q, H * G, [L, L], window)
    torch.cuda.synchronize()
    for x, y in ((dc.k_codes, du.k_codes), (dc.v_codes, du.v_codes), (dc.k_scales, du.k_scales),
                 (dc.v_scales, du.v_scales)):
        assert torch.equal(x, y)
    assert_attn_close(out.cpu().numpy(), out_u.cpu().numpy().astype(np.float64), "fused vs unfused")
    # the oracle over the rows the fused call stored (each held to the codec rule first)
    kh, vh, _ = codec_hat_from_device(dc, "codec3", np16(k), np16(v), [L, L], window)
    ref = attention.decode_attention(np16(q), kh, vh, [L, L], window)
    assert_attn_close(out.cpu().numpy(), ref, f"codec3 fused D={D} w={window}")
