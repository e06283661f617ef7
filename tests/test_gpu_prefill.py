"""Chunked-prefill (multi-query, causal) attention over the INT4 cache on the GPU
(lpnh.cn/news/2042373 section 1.1: the prefill computes every position of the prompt at
once, where decode computes one).

A chunk of nq tokens per sequence sits at positions [len - nq, len) of the cache and
attends causally (with a window, each query its own window).  Held against the fp64
oracle (``attention.prefill_attention`` over the oracle's dequantized values; the cache
codes are bit-exact with the oracle's elsewhere) at max abs 2e-3 and relative L2 1e-4,
for chunk sizes 1 .. 512, ragged lengths, GQA groups 1, 2, 4, 8, K groups 64 and 128,
windows, a window ring and the paged layout.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, quant
from tests.kvq_testutil import assert_attn_close, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # G, gk, nq, lens, window, cap (None: max len), page size
    (4, 64, 16, [8193, 2000], 0, None, 0),
    (4, 64, 100, [1000, 1000], 0, None, 0),     # chunk not a multiple of the query block
    (1, 128, 64, [3000], 0, None, 0),
    (8, 64, 37, [500, 37], 0, None, 0),          # the whole prompt as one chunk (sequence 1)
    (2, 64, 512, [4096, 4096], 0, None, 0),
    (4, 64, 64, [2048, 1500], 256, None, 0),     # window
    (4, 64, 200, [3000, 3000], 256, 512, 0),     # window ring (capacity >= window + chunk - 1)
    (4, 64, 48, [1999, 777], 0, None, 16),       # paged, pages of 16
    (2, 128, 96, [2500, 900], 300, None, 64),    # paged, window
    (4, 64, 1, [100, 200], 0, None, 0),          # one-token chunks
]


def _fill(desc, dc, k, v, L, cap):
    for start in range(0, L, cap):
        n = min(cap, L - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)


@pytest.mark.parametrize("case", CASES, ids=[f"prefill{i}" for i in range(len(CASES))])
def test_prefill_attention(case):
    G, gk, nq, lens, W, cap, P = case
    B, Hkv, D = len(lens), 2, 128
    L = max(lens)
    k = synth.kv_source((B, Hkv, L, D), 4200 + nq, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 4300 + nq, DEV, outlier_channels=3,
                        zero_groups=((0, 1, L - 1, 0, D),))
    q = synth.query((B, Hkv * G, nq, D), 4400 + nq, DEV)
    if P:
        C = (L + P - 1) // P * P
        table, pages = synth.block_table(B, C, P, 4500 + nq)
        desc = kvq.make_desc("int4", B, Hkv, D, C, gk, 128, page_size=P, num_pages=pages)
        dc = kvq.DeviceCache(desc, DEV, block_table=table.to(DEV))
        _fill(desc, dc, k, v, L, C)
    else:
        C = cap or L
        desc = kvq.make_desc("int4", B, Hkv, D, C, gk, 128)
        dc = kvq.DeviceCache(desc, DEV)
        _fill(desc, dc, k, v, L, C)
    out = torch.full((B, Hkv * G, nq, D), float("nan"), dtype=torch.float32, device=DEV)
    kvq.kvq_prefill_attn(desc, dc.c, q, Hkv * G, nq, lens, W, 0.0, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "an output was not written"
    qk, sk = quant.quantize_int4(np16(k), gk)
    qv, sv = quant.quantize_int4(np16(v), 128)
    kh = quant.dequantize_int4_exact(qk, sk, gk)
    vh = quant.dequantize_int4_exact(qv, sv, 128)
    ref = attention.prefill_attention(np16(q), kh, vh, lens, W)
    assert_attn_close(out.cpu().numpy(), ref, f"prefill {case}")


H16_CASES = [
    # G, gk, nq, lens, window, cap, page size
    (4, 64, 100, [1000, 1000], 0, None, 0),
    (2, 128, 333, [2000, 700], 0, None, 0),
    (8, 64, 64, [1500, 1200], 256, None, 0),
    (4, 64, 48, [1999, 777], 0, None, 16),
]


@pytest.mark.parametrize("case", H16_CASES, ids=[f"h16_{i}" for i in range(len(H16_CASES))])
def test_prefill_attention_fp16_scales(case):
    """The same chunked prefill over an INT4 cache with fp16 scales (the kernel's 2-byte
    scale transfers), against the oracle over the fp16-scale format's dequantized values."""
    G, gk, nq, lens, W, cap, P = case
    B, Hkv, D = len(lens), 2, 128
    L = max(lens)
    k = synth.kv_source((B, Hkv, L, D), 4700 + nq, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 4800 + nq, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, nq, D), 4900 + nq, DEV)
    if P:
        C = (L + P - 1) // P * P
        table, pages = synth.block_table(B, C, P, 5000 + nq)
        desc = kvq.make_desc("int4h", B, Hkv, D, C, gk, 128, page_size=P, num_pages=pages)
        dc = kvq.DeviceCache(desc, DEV, block_table=table.to(DEV))
    else:
        C = cap or L
        desc = kvq.make_desc("int4h", B, Hkv, D, C, gk, 128)
        dc = kvq.DeviceCache(desc, DEV)
    _fill(desc, dc, k, v, L, C)
    out = torch.full((B, Hkv * G, nq, D), float("nan"), dtype=torch.float32, device=DEV)
    kvq.kvq_prefill_attn(desc, dc.c, q, Hkv * G, nq, lens, W, 0.0, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "an output was not written"
    qk, sk = quant.quantize_int4_fp16_scale(np16(k), gk)
    qv, sv = quant.quantize_int4_fp16_scale(np16(v), 128)
    kh = quant.dequantize_int4_exact(qk, sk, gk)
    vh = quant.dequantize_int4_exact(qv, sv, 128)
    ref = attention.prefill_attention(np16(q), kh, vh, lens, W)
    assert_attn_close(out.cpu().numpy(), ref, f"prefill fp16 scales {case}")


def test_prefill_then_decode_agree():
    """A one-token chunk is the decode step: kvq_prefill_attn with n_query = 1 and
    kvq_decode_attn give the same output within the bar."""
    B, Hkv, G, D, L = 3, 2, 4, 128, 1500
    k = synth.kv_source((B, Hkv, L, D), 4600, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 4601, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 4602, DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, L)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, L)
    lens = [L, 999, 33]
    out = torch.empty((B, Hkv * G, 1, D), dtype=torch.float32, device=DEV)
    kvq.kvq_prefill_attn(desc, dc.c, q[:, :, None].contiguous(), Hkv * G, 1, lens, 0, 0.0, out)
    ws = kvq.decode_workspace(desc, Hkv * G, L, device=DEV)
    dec = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=DEV)
    kvq.kvq_decode_attn(desc, dc.c, q, Hkv * G, lens, 0, 0.0, 0, dec, ws)
    torch.cuda.synchronize()
    assert_attn_close(out[:, :, 0].cpu().numpy(), dec.cpu().numpy().astype(np.float64), "prefill vs decode")


def test_benched_chunk_full_size_sampled():
    """The chunk the benchmark times, at full size: the Llama-3-8B-shaped layer (8
    sequences, 8 KV heads, 32 query heads) prefilled to 7680 positions, the 512-token chunk
    quantized into positions 7680 .. 8191, then kvq_prefill_attn of its 512 queries, eager
    and replayed from a HIP graph.  The oracle checks sampled outputs one by one (a query
    of the chunk is the decode query at its own length): first, middle and last queries of
    corner (sequence, head) pairs."""
    w = synth.WORKLOADS[2]
    B, Hq, Hkv, D, L, NQ = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.context, 512
    P0 = L - NQ
    k, v, _, _, _ = synth.layer_inputs(w, 1, DEV)
    q = synth.query((B, Hq, NQ, D), synth.seed_of(w.wid, 1, 6), DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, L, w.group_k, w.group_v)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :P0].contiguous(), v[:, :, :P0].contiguous(), 0, P0)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, P0:].contiguous(), v[:, :, P0:].contiguous(), P0, NQ)
    out = torch.full((B, Hq, NQ, D), float("nan"), dtype=torch.float32, device=DEV)
    kvq.kvq_prefill_attn(desc, dc.c, q, Hq, NQ, [L] * B, 0, 0.0, out)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    replayed = torch.full_like(out, float("nan"))
    with torch.cuda.graph(g, stream=s):
        kvq.kvq_prefill_attn(desc, dc.c, q, Hq, NQ, [L] * B, 0, 0.0, replayed)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.equal(out, replayed)
    got = out.cpu().numpy()
    q16 = np16(q)
    for b in (0, B - 1):
        kh_b, vh_b = {}, {}
        for h in (0, 5, Hq - 1):
            kvh = h // (Hq // Hkv)
            if kvh not in kh_b:
                qk, sk = quant.quantize_int4(np16(k[b:b + 1, kvh:kvh + 1]), w.group_k)
                qv, sv = quant.quantize_int4(np16(v[b:b + 1, kvh:kvh + 1]), w.group_v)
                kh_b[kvh] = quant.dequantize_int4_exact(qk, sk, w.group_k)
                vh_b[kvh] = quant.dequantize_int4_exact(qv, sv, w.group_v)
            for i in (0, 1, 255, NQ - 1):
                ref = attention.prefill_attention(q16[b:b + 1, h:h + 1, i:i + 1], kh_b[kvh], vh_b[kvh],
                                                  [P0 + i + 1])
                assert_attn_close(got[b:b + 1, h:h + 1, i:i + 1], ref, f"chunk b={b} h={h} query {i}")
