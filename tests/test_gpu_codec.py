"""GPU parity of the WHT + Lloyd-Max 4-bit codec ("长上下文内存大瘦身：LARQL 四大 KV 缓存
引擎原理与横向对比", pwwt.cn/news/5725003, engine three) against the oracle.

Bar: code mismatches only where the pre-quantization value y/s lies within 1e-5 of a
decision threshold; scales and rotated (decoded) values within 1e-5 relative;
attention over the same codes within max abs 2e-3 and relative L2 1e-4.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, codec, quant
from tests.kvq_testutil import (append_decode, assert_attn_close, cache_arrays, codec_hat_from_device,
                                decode, np16)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _encode(k, v, cap=None):
    B, H, S, D = k.shape
    desc = kvq.make_desc("codec", B, H, D, cap or S)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, S)
    return desc, dc


def _check_codes(got_codes, got_scales, x16):
    idx, s, u = codec.encode(x16)
    g_idx = quant.unpack_nibbles(got_codes, signed=False)
    g_s = got_scales[..., 0]
    assert np.allclose(g_s, s, rtol=1e-5, atol=0)
    mism = g_idx != idx
    if mism.any():
        _, thr, _ = codec.codebook(4)
        d = np.min(np.abs(u[mism][:, None] - thr[None, :]), axis=1)
        assert np.all(d <= 1e-5), f"{int((d > 1e-5).sum())} codes differ away from a threshold"
    return int(mism.sum()), idx.size


@pytest.mark.parametrize("D", [64, 128, 256])
def test_encode_boundary_rule(D):
    k = synth.kv_source((2, 4, 300, D), 51, DEV)
    v = synth.kv_source((2, 4, 300, D), 52, DEV, outlier_channels=2,
                        zero_groups=((1, 3, 7, 0, D),))
    desc, dc = _encode(k, v)
    kc, ks, vc, vs = cache_arrays(dc, "codec")
    _check_codes(kc, ks, np16(k))
    _check_codes(vc, vs, np16(v))
    assert vs[1, 3, 7, 0] == 0.0


def test_dequant_rotated_values():
    D = 256
    k = synth.kv_source((2, 4, 100, D), 53, DEV)
    v = synth.kv_source((2, 4, 100, D), 54, DEV)
    desc, dc = _encode(k, v)
    kc, ks, _, _ = cache_arrays(dc, "codec")
    out = torch.empty((2, 4, 100, D), dtype=torch.float32, device=DEV)
    kvq.kvq_dequant(desc, dc.c, 0, 0, 100, out)
    torch.cuda.synchronize()
    # the oracle decodes the same codes and scales the GPU stored (a decode-only check)
    ref = codec.decode(quant.unpack_nibbles(kc, signed=False), ks[..., 0])
    got = out.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    cos = codec.row_cosine(np16(k).astype(np.float64), got)
    assert abs(cos.mean() - 0.9954) < 0.0015


def _inject(dc, kidx, ks, vidx, vs):
    """Write oracle-encoded codes/scales into the device cache buffers."""
    dc.k_codes.copy_(torch.from_numpy(quant.pack_nibbles(kidx).reshape(-1)).to(DEV))
    dc.v_codes.copy_(torch.from_numpy(quant.pack_nibbles(vidx).reshape(-1)).to(DEV))
    dc.k_scales.copy_(torch.from_numpy(np.ascontiguousarray(ks).reshape(-1)).to(DEV))
    dc.v_scales.copy_(torch.from_numpy(np.ascontiguousarray(vs).reshape(-1)).to(DEV))


@pytest.mark.parametrize("window,L,cap", [(0, 700, 700), (256, 700, 256), (1024, 4097, 1024)])
def test_attention_over_oracle_codes(window, L, cap):
    """Decode attention on a cache holding the oracle's own codes (so both sides attend
    over identical dequantized values), in a global layer and in window rings."""
    B, H, G, D = 2, 4, 2, 256
    k = synth.kv_source((B, H, L, D), 60 + L, DEV)
    v = synth.kv_source((B, H, L, D), 61 + L, DEV)
    q = synth.query((B, H * G, D), 62 + L, DEV)
    kn, vn = np16(k), np16(v)
    kidx, ks, _ = codec.encode(kn)
    vidx, vs, _ = codec.encode(vn)
    desc = kvq.make_desc("codec", B, H, D, cap)
    dc = kvq.DeviceCache(desc, DEV)
    slots = np.arange(L) % cap
    keep = np.arange(max(0, L - cap), L)
    ring = lambda a: a[:, :, keep][:, :, np.argsort(slots[keep])]  # noqa: E731
    _inject(dc, ring(kidx), ring(ks), ring(vidx), ring(vs))
    out = decode(desc, dc, q, H * G, [L, L], window)
    ref = attention.decode_attention(np16(q), codec.decode(kidx, ks), codec.decode(vidx, vs),
                                     [L, L], window)
    assert_attn_close(out.cpu().numpy(), ref, f"codec w={window}")


@pytest.mark.parametrize("D,G", [(64, 8), (128, 1), (128, 4), (256, 4), (256, 8)])
def test_attention_over_oracle_codes_head_shapes(D, G):
    """The same check over head dims and GQA groups: q is rotated once per workgroup by
    the last G row groups, whose placement depends on D (lanes per row) and G."""
    B, H, L = 2, 2, 300
    k = synth.kv_source((B, H, L, D), 70 + D + G, DEV)
    v = synth.kv_source((B, H, L, D), 71 + D + G, DEV)
    q = synth.query((B, H * G, D), 72 + D + G, DEV)
    kn, vn = np16(k), np16(v)
    kidx, ks, _ = codec.encode(kn)
    vidx, vs, _ = codec.encode(vn)
    desc = kvq.make_desc("codec", B, H, D, L)
    dc = kvq.DeviceCache(desc, DEV)
    _inject(dc, kidx, ks, vidx, vs)
    out = decode(desc, dc, q, H * G, [L, L - 37], 0)
    ref = attention.decode_attention(np16(q), codec.decode(kidx, ks), codec.decode(vidx, vs),
                                     [L, L - 37], 0)
    assert_attn_close(out.cpu().numpy(), ref, f"codec D={D} G={G}")


@pytest.mark.parametrize("fmt,wid", [("codec", 4), ("codec3", 8)])
def test_gemma_shape_end_to_end_window_and_global(fmt, wid):
    """The Gemma-3-4B-shaped codec decode step as the benchmark runs it (batch 4, 4 KV
    heads x 256, 8 query heads; the library's split plan): one sliding-window layer (ring
    of 1024 rows) and one global layer, each prefilled to 4096 positions, then the one-launch
    kvq_append_decode_attn of position 4096 (the kernel codes the new row), eager and
    replayed from a HIP graph.  The new row's bytes equal those kvq_append stores."""
    w = synth.WORKLOADS[wid]
    for layer in (0, w.layers - 1):
        W = w.layer_window(layer)
        k, v, q, kn, vn = synth.layer_inputs(w, layer, DEV)
        L = w.context + 1
        cap = W if W else L
        desc = kvq.make_desc(fmt, w.batch, w.kv_heads, w.head_dim, cap)
        dc, du = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(desc, DEV)
        for start in range(0, w.context, cap):
            n = min(cap, w.context - start)
            for c_ in (dc, du):
                kvq.kvq_quantize_prefill(desc, c_.c, k[:, :, start:start + n].contiguous(),
                                         v[:, :, start:start + n].contiguous(), start, n)
        ws = kvq.decode_workspace(desc, w.q_heads, L, W, device=DEV)
        out = append_decode(desc, dc, kn, vn, q, w.q_heads, [L] * w.batch, W, ws=ws).cpu().numpy()
        kvq.kvq_append(desc, du.c, kn, vn, [w.context] * w.batch)
        torch.cuda.synchronize()
        for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
            assert torch.equal(getattr(dc, name), getattr(du, name)), name
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        replayed = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
        with torch.cuda.graph(g, stream=st):   # (re-appends the same row: same bytes)
            kvq.kvq_append_decode_attn(desc, dc.c, kn, vn, q, w.q_heads, [L] * w.batch, W, 0.0, 0,
                                       replayed, ws)
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        kall = np.concatenate([np16(k), np16(kn)[:, :, None]], axis=2)
        vall = np.concatenate([np16(v), np16(vn)[:, :, None]], axis=2)
        # every attended row read back from the cache and held to the codec rule, then
        # the oracle's attention over those rows
        kh, vh, _ = codec_hat_from_device(dc, fmt, kall, vall, [L] * w.batch, W)
        ref = attention.decode_attention(np16(q), kh, vh, [L] * w.batch, W)
        assert_attn_close(out, ref, f"gemma {fmt} layer {layer}")
        assert_attn_close(replayed.cpu().numpy(), ref, f"gemma {fmt} layer {layer}, graph")
