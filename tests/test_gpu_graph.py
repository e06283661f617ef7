"""HIP-graph replay of a decode step.

A captured ``kvq_append_decode_attn`` call replays to the eager result, replay after
replay, with eager library work and synchronizations in between, and leaves the split
arrival counters at zero each time.  Paths: the INT4 matrix-core kernel (in-kernel
merge, append fused in the prologue) and its instances for attention sinks, for
recent fp16 rows and for fp16 scales, the codec's split-K kernel with the in-kernel merge, and the codec's
split-K kernel followed by the merge kernel.  The eager result
is itself checked against the oracle ("长上下文内存大瘦身" engine three for the codec;
lpnh.cn/news/2042373 section 2.1 and the plain softmax definition for INT4).
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, codec, quant
from tests.kvq_testutil import assert_attn_close, codec_hat_from_device, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # fmt, head_dim, q heads per kv head, num_splits (0: planned), sinks, recent, window
    ("int4", 128, 4, 0, 0, 0, 0),     # matrix-core kernel, 4 splits merged in-kernel
    ("codec", 256, 2, 0, 0, 0, 0),    # split-K, in-kernel merge (append in a split of its own)
    ("codec", 256, 2, 40, 0, 0, 0),   # split-K + merge kernel
    ("int4", 128, 4, 0, 4, 0, 256),   # matrix-core sink instance, window 256 + 4 sinks
    ("int4", 128, 4, 0, 0, 64, 0),    # matrix-core recent-row instance, 64 fp16 rows
    ("int4h", 128, 4, 0, 0, 0, 0),    # matrix-core fp16-scale instance
]


@pytest.mark.parametrize("fmt,D,G,ns,S,R,W", CASES,
                         ids=[f"{c[0]}-{c[1]}-ns{c[3]}-s{c[4]}-r{c[5]}" for c in CASES])
def test_graph_replay_matches_eager(fmt, D, G, ns, S, R, W):
    B, Hkv, P = 2, 2, 700
    L = P + 1
    Hq = Hkv * G
    k = synth.kv_source((B, Hkv, L, D), 61, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 62, DEV, outlier_channels=2)
    q = synth.query((B, Hq, D), 63, DEV)
    q2 = synth.query((B, Hq, D), 64, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, L, min(64, D), min(128, D), sinks=S, recent=R)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :P].contiguous(), v[:, :, :P].contiguous(), 0, P)
    kn, vn = k[:, :, P].contiguous(), v[:, :, P].contiguous()
    ws = kvq.decode_workspace(desc, Hq, L, W, ns, DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    other = torch.empty_like(out)
    lens = [L, L]

    def step():
        kvq.kvq_append_decode_attn(desc, dc.c, kn, vn, q, Hq, lens, W, 0.0, ns, out, ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    if fmt == "codec":   # over the rows the GPU coded (each held to the codec rule)
        kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), lens, W)
        ref = attention.decode_attention(np16(q), kh, vh, lens, W)
        assert_attn_close(eager.cpu().numpy(), ref, f"{fmt} eager")
    else:
        quantize = quant.quantize_int4_fp16_scale if fmt == "int4h" else quant.quantize_int4
        qk, sk = quantize(np16(k), 64)
        qv, sv = quantize(np16(v), 128)
        kh, vh = quant.dequantize_int4_exact(qk, sk, 64), quant.dequantize_int4_exact(qv, sv, 128)
        if R:
            kh = attention.recent_fp16_rows(kh, np16(k), lens, R)
            vh = attention.recent_fp16_rows(vh, np16(v), lens, R)
        ref = attention.decode_attention(np16(q), kh, vh, lens, W, sinks=S)
        assert_attn_close(eager.cpu().numpy(), ref, f"{fmt} eager")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    counters = ws[: B * Hkv].view(torch.int32)
    for r in range(4):
        out.fill_(float("nan"))   # the replay must write every output
        g.replay()
        torch.cuda.synchronize()
        # (tiles and rows are shared out dynamically: the fp32 sums may differ from the
        # eager call in their last bits)
        assert torch.allclose(out, eager, rtol=1e-4, atol=1e-5), f"replay {r}"
        assert int(counters.abs().sum()) == 0, f"split counters after replay {r}"
        # eager work between replays, through the same workspace
        kvq.kvq_decode_attn(desc, dc.c, q2, Hq, lens, W, 0.0, ns, other, ws)
        torch.cuda.synchronize()
        assert int(counters.abs().sum()) == 0, f"split counters after eager call {r}"
        assert torch.isfinite(other).all()
