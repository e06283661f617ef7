"""Attention sinks over a window ring, on the GPU.

"AI 推理性能调优：KV Cache 优化与显存管理的工程实践" (bxzpzcl.cn/news/2871434),
section 3.2 ``SlidingWindowAttention``: a windowed query also attends the first
``num_sink_tokens`` positions.  The cache keeps them in S slots ahead of a ring of
C - S slots (position p < S in slot p, else in slot S + (p - S) mod (C - S)); a decode
step attends ``[0, min(S, len - W)) U [len - W, len)``.  Checked here: the layout
(dequantized slots equal the oracle's rows of those positions, bit for bit), appends
equal to prefills, and decode attention against the oracle's
``decode_attention(..., window, sinks)`` on every format, with and without the fused
append.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, codec, quant
from tests.kvq_testutil import append_decode, assert_attn_close, codec_hat_from_device, decode, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fill_ring(desc, k, v, upto):
    """Prefill positions [0, upto) chunk by chunk: the sinks and a ring's worth first,
    then ring-sized chunks (each write fits the ring)."""
    dc = kvq.DeviceCache(desc, DEV)
    S, R = desc.sinks, desc.capacity - desc.sinks
    start = 0
    while start < upto:
        n = min(upto - start, (S + R) if start == 0 else R)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
        start += n
    return dc


def _hat(fmt, k16, v16):
    if fmt == "int4":
        D = k16.shape[-1]
        gk, gv = min(64, D), min(128, D)
        qk, sk = quant.quantize_int4(k16, gk)
        qv, sv = quant.quantize_int4(v16, gv)
        return quant.dequantize_int4_exact(qk, sk, gk), quant.dequantize_int4_exact(qv, sv, gv)
    if fmt == "int8":
        qk, sk = quant.quantize_int8(k16)
        qv, sv = quant.quantize_int8(v16)
        return quant.dequantize_int8_exact(qk, sk), quant.dequantize_int8_exact(qv, sv)
    if fmt == "int4h":
        D = k16.shape[-1]
        gk, gv = min(64, D), min(128, D)
        qk, sk = quant.quantize_int4_fp16_scale(k16, gk)
        qv, sv = quant.quantize_int4_fp16_scale(v16, gv)
        return quant.dequantize_int4_exact(qk, sk, gk), quant.dequantize_int4_exact(qv, sv, gv)
    kidx, ksc, _ = codec.encode(k16)
    vidx, vsc, _ = codec.encode(v16)
    return codec.decode(kidx, ksc), codec.decode(vidx, vsc)


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_layout_sinks_and_ring_bit_exact(fmt):
    B, H, D, S, R, L = 2, 2, 128, 4, 60, 333
    k = synth.kv_source((B, H, L, D), 71, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, L, D), 72, DEV, outlier_channels=2)
    desc = kvq.make_desc(fmt, B, H, D, S + R, sinks=S)
    dc = _fill_ring(desc, k, v, L)
    kh, vh = _hat(fmt, np16(k), np16(v))
    for kv, ref in ((0, kh), (1, vh)):
        for start, n in ((0, S), (L - R, R)):          # the sinks, then the ring's rows
            out = torch.empty((B, H, n, D), dtype=torch.float32, device=DEV)
            kvq.kvq_dequant(desc, dc.c, kv, start, n, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref[:, :, start:start + n].astype(np.float32))
    # one position at a time lands in the same bytes
    da = kvq.DeviceCache(desc, DEV)
    for t in range(L):
        kvq.kvq_append(desc, da.c, k[:, :, t].contiguous(), v[:, :, t].contiguous(), [t] * B)
    torch.cuda.synchronize()
    for x, y in ((da.k_codes, dc.k_codes), (da.k_scales, dc.k_scales), (da.v_codes, dc.v_codes),
                 (da.v_scales, dc.v_scales)):
        assert torch.equal(x, y)


CASES = [
    # fmt, D, G, sinks, ring, window, lens, num_splits
    ("int4", 128, 4, 4, 256, 200, [1000, 700], 0),
    ("int4", 128, 1, 4, 256, 256, [1000, 257], 5),
    ("int8", 128, 4, 4, 128, 100, [900, 50], 0),       # sequence 1: window reaches the sinks
    ("int4", 64, 2, 16, 96, 96, [500, 140], 0),
    ("codec", 256, 2, 4, 256, 256, [1500, 600], 0),
    ("codec", 128, 4, 8, 128, 100, [700, 20], 40),      # merge kernel; a short sequence
    ("int4h", 128, 4, 4, 256, 200, [1000, 700], 0),     # fp16 scales with sinks: split-K kernel
    # one split, so its 32-position tiles start at lo - 4 (sequence 0: lo = 792): the first
    # holds the sinks, the next ones lie past the window start in consecutive ring slots,
    # and the one at 1012 wraps the ring (slots 244 .. 259, then 4 ..); in sequence 1
    # (lo = 712) the tile at 740 ends exactly at the last slot (228 .. 259)
    ("int4", 128, 4, 4, 256, 256, [1048, 968], 1),
    ("int4", 128, 4, 4, 256, 256, [1048, 968], 3),
]


@pytest.mark.parametrize("case", CASES, ids=[f"sinks{i}" for i in range(len(CASES))])
def test_decode_window_with_sinks(case):
    fmt, D, G, S, R, W, lens, ns = case
    B, Hkv = len(lens), 2
    L = max(lens)
    k = synth.kv_source((B, Hkv, L, D), 81 + L, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 82 + L, DEV, outlier_channels=2)
    q = synth.query((B, Hkv * G, D), 83 + L, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, S + R, min(64, D), min(128, D), sinks=S)
    kh, vh = _hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, lens, W, sinks=S)
    # every sequence prefilled to its own length: sequences shorter than L get their own
    # cache rows filled up to L too (the rows past len_b are never attended)
    dc = _fill_ring(desc, k, v, L)
    # the ring holds positions up to L - 1 for every sequence; for a shorter sequence
    # the attended positions are rewritten below (prefill of its window at its own end)
    for b, ln in enumerate(lens):
        if ln < L:
            lo = max(S, ln - R)
            one = kvq.make_desc(fmt, 1, Hkv, D, S + R, min(64, D), min(128, D), sinks=S)
            sub = kvq.kvq_cache(*[t.view(B, -1)[b].data_ptr() for t in
                                  (dc.k_codes, dc.k_scales, dc.v_codes, dc.v_scales)])
            kvq.kvq_quantize_prefill(one, sub, k[b:b + 1, :, lo:ln].contiguous(),
                                     v[b:b + 1, :, lo:ln].contiguous(), lo, ln - lo)
    out = decode(desc, dc, q, Hkv * G, lens, W, 0.0, ns)
    if fmt == "codec":   # over the rows the GPU coded (each held to the codec rule)
        kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), lens, W)
        ref = attention.decode_attention(np16(q), kh, vh, lens, W, sinks=S)
    assert_attn_close(out.cpu().numpy(), ref, f"{case}")


@pytest.mark.parametrize("fmt,D,G", [("int4", 128, 4), ("codec", 256, 2), ("int4h", 128, 4)])
def test_append_decode_with_sinks(fmt, D, G):
    """The step's new row (position len - 1) lands in its ring slot and is attended."""
    B, Hkv, S, R, W, L = 2, 2, 4, 128, 128, 700
    k = synth.kv_source((B, Hkv, L, D), 91, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 92, DEV, outlier_channels=2)
    q = synth.query((B, Hkv * G, D), 93, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, S + R, min(64, D), min(128, D), sinks=S)
    dc = _fill_ring(desc, k, v, L - 1)
    out = append_decode(desc, dc, k[:, :, L - 1].contiguous(), v[:, :, L - 1].contiguous(), q,
                        Hkv * G, [L, L], W)
    if fmt == "codec":   # over the rows the GPU coded, the new one included
        kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), [L, L], W)
    else:
        kh, vh = _hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, [L, L], W, sinks=S)
    assert_attn_close(out.cpu().numpy(), ref, f"{fmt} append + decode")
    # the new row sits in slot S + (L - 1 - S) mod R
    ref_cache = _fill_ring(desc, k, v, L)
    slot = S + (L - 1 - S) % R
    torch.cuda.synchronize()
    sc = (lambda t: t.view(torch.float16)) if fmt == "int4h" else (lambda t: t)   # fp16 scales
    for x, y in ((dc.k_codes, ref_cache.k_codes), (dc.v_codes, ref_cache.v_codes),
                 (sc(dc.k_scales), sc(ref_cache.k_scales)), (sc(dc.v_scales), sc(ref_cache.v_scales))):
        xs = x.view(B, Hkv, S + R, -1)[:, :, slot]
        ys = y.view(B, Hkv, S + R, -1)[:, :, slot]
        assert torch.equal(xs, ys)
