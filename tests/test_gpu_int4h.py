"""INT4 with fp16 scales on the GPU (lpnh.cn/news/2042373 §2.1 run in fp16; §2.2's 16-bit
scale accounting: 4.25 bits per element for K groups of 64, 4.125 for V groups of 128).

Bar: codes and fp16 scales bit-exact against the oracle's ``quantize_int4_fp16_scale``
(prefill and append, zero groups, scales that underflow fp16, the largest fp16); dequant
bit-exact (code * scale is exact in fp32); decode attention over the cache within max abs
2e-3 and relative L2 1e-4 of the fp64 oracle.

At head_dim 128 with V groups of 128 the matrix-core kernel serves the format (fp16 scale
transfers into its tiles, the fused append in its prologue with the format's fp16
arithmetic); other shapes, and caches with sinks, take the split-K kernel.
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
    # the fused step (the matrix-core kernel's prologue or the split-K kernel codes the new
    # row) leaves the cache bytes of the append kernel
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


MFMA_CASES = [
    # G, gk, lens, window, cap (None: max len), num_splits (0: planned), V multiplier
    (1, 128, [3000, 900], 0, None, 0, 1.0),      # one K group
    (2, 64, [2500, 1], 0, None, 0, 1.0),         # a one-position sequence
    (4, 32, [4000, 2000], 0, None, 3, 1.0),      # four K groups
    (8, 64, [3000, 3000], 0, None, 0, 1.0),      # 16 columns (one position set)
    (4, 64, [5000, 4000], 1024, 1100, 0, 1.0),   # window ring
    (4, 64, [6000, 6000], 0, None, 24, 1.0),     # many splits
    (4, 64, [3000, 1500], 0, None, 0, 1e-3),     # small V scales
    (2, 64, [3000, 1500], 0, None, 0, 1e-5),     # V scales in fp16's subnormal range
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=[f"mfma{i}" for i in range(len(MFMA_CASES))])
def test_matrix_core_instance(case):
    """The matrix-core kernel's fp16-scale instance against the oracle: every K group
    count, GQA 1 .. 8, windows over a ring, split counts, and V scales down to fp16
    subnormals (the P' normalizer moves with them)."""
    G, gk, lens, W, cap, ns, vm = case
    B, H, D = len(lens), 2, 128
    L = max(lens)
    C = cap or L
    k = synth.kv_source((B, H, L, D), 2100 + G + gk, DEV, outlier_channels=3)
    v = (synth.kv_source((B, H, L, D), 2200 + G + gk, DEV, outlier_channels=3).float() * vm).to(torch.float16)
    q = synth.query((B, H * G, D), 2300 + G + gk, DEV)
    desc = kvq.make_desc("int4h", B, H, D, C, gk, 128)
    dc = kvq.DeviceCache(desc, DEV)
    for start in range(max(0, L - C), L, C):   # the last C positions (a ring holds those)
        n = min(C, L - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    # a ring shorter than the longest sequence holds that sequence's last positions in
    # every row: a shorter sequence gets its own last C positions back
    one = kvq.make_desc("int4h", 1, H, D, C, gk, 128)
    for b, ln in enumerate(lens):
        lo = max(0, ln - C)
        if ln < L and C < L:
            sub = kvq.kvq_cache(*[t.view(B, -1)[b].data_ptr() for t in
                                  (dc.k_codes, dc.k_scales, dc.v_codes, dc.v_scales)])
            kvq.kvq_quantize_prefill(one, sub, k[b:b + 1, :, lo:ln].contiguous(),
                                     v[b:b + 1, :, lo:ln].contiguous(), lo, ln - lo)
    assert kvq.kvq_plan_splits(desc, H * G, min(L, W) if W else L) >= 1
    out = decode(desc, dc, q, H * G, lens, W, 0.0, ns)
    qk, sk = quant.quantize_int4_fp16_scale(np16(k), gk)
    qv, sv = quant.quantize_int4_fp16_scale(np16(v), 128)
    ref = attention.decode_attention(np16(q), quant.dequantize_int4_exact(qk, sk, gk),
                                     quant.dequantize_int4_exact(qv, sv, 128), lens, W)
    assert_attn_close(out.cpu().numpy(), ref, f"int4h matrix-core {case}")


@pytest.mark.parametrize("G,gk", [(4, 64), (1, 128), (2, 32), (8, 64)])
def test_matrix_core_fused_step_edge_rows(G, gk):
    """The fused step's new row coded in the matrix-core kernel's prologue with the fp16
    arithmetic, over rows that hit the format's edges (zero groups, a scale that
    underflows fp16, the largest fp16, subnormal scales): the same cache bytes as the
    append kernel, and attention within the bar of the oracle."""
    B, H, D, L = 2, 2, 128, 1500
    k = synth.kv_source((B, H, L, D), 2400 + G, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, L, D), 2500 + G, DEV, outlier_channels=2)
    q = synth.query((B, H * G, D), 2600 + G, DEV)
    kn, vn = k[:, :, L - 1].clone(), v[:, :, L - 1].clone()
    kn[0, 0] = 0.0
    vn[0, 0] = 0.0
    kn[0, 1] = 6e-8
    vn[0, 1] = 6e-8
    kn[1, 0, 5] = 65504.0
    vn[1, 0, 5] = -65504.0
    kn[1, 1] *= 1e-4
    vn[1, 1] *= 1e-4
    k[:, :, L - 1] = kn
    v[:, :, L - 1] = vn
    desc = kvq.make_desc("int4h", B, H, D, L, gk, 128)
    dc, du = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(desc, DEV)
    for c_ in (dc, du):
        kvq.kvq_quantize_prefill(desc, c_.c, k[:, :, :L - 1].contiguous(), v[:, :, :L - 1].contiguous(), 0, L - 1)
    out = append_decode(desc, dc, kn.contiguous(), vn.contiguous(), q, H * G, [L, L - 700])
    kvq.kvq_append(desc, du.c, kn.contiguous(), vn.contiguous(), [L - 1, L - 701])
    torch.cuda.synchronize()
    for x, y in ((dc.k_codes, du.k_codes), (dc.k_scales, du.k_scales), (dc.v_codes, du.v_codes),
                 (dc.v_scales, du.v_scales)):
        assert torch.equal(x, y)
    # the oracle over each sequence's own rows: sequence 1 appended at position L - 701
    kk, vv = np16(k), np16(v)
    kk[1, :, L - 701] = kk[1, :, L - 1]
    vv[1, :, L - 701] = vv[1, :, L - 1]
    qk, sk = quant.quantize_int4_fp16_scale(kk, gk)
    qv, sv = quant.quantize_int4_fp16_scale(vv, 128)
    ref = attention.decode_attention(np16(q), quant.dequantize_int4_exact(qk, sk, gk),
                                     quant.dequantize_int4_exact(qv, sv, 128), [L, L - 700])
    assert_attn_close(out.cpu().numpy(), ref, f"int4h fused step G={G} gk={gk}")


def test_benched_step_full_size():
    """The fp16-scale decode step at the size the benchmark times (Llama-3-8B shape: 8
    sequences, 8 KV heads, 32 query heads, 8192 cached positions + the appended one, the
    library's split plan), eager and replayed from a HIP graph, against the oracle."""
    w = synth.WORKLOADS[9]
    k, v, q, kn, vn = synth.layer_inputs(w, 3, DEV)
    L = w.context + 1
    desc = kvq.make_desc("int4h", w.batch, w.kv_heads, w.head_dim, L, w.group_k, w.group_v)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, w.context)
    assert kvq.kvq_plan_splits(desc, w.q_heads, L) == 4
    ws = kvq.decode_workspace(desc, w.q_heads, L, device=DEV)
    snap = [getattr(dc, n).clone() for n in ("k_codes", "k_scales", "v_codes", "v_scales")]
    eager = append_decode(desc, dc, kn, vn, q, w.q_heads, [L] * w.batch, ws=ws)
    for t, n in zip(snap, ("k_codes", "k_scales", "v_codes", "v_scales")):   # back to the prefilled cache
        getattr(dc, n).copy_(t)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    replayed = torch.full_like(eager, float("nan"))
    with torch.cuda.graph(g, stream=s):
        kvq.kvq_append_decode_attn(desc, dc.c, kn, vn, q, w.q_heads, [L] * w.batch, 0, 0.0, 0,
                                   replayed, ws)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    kall = np.concatenate([np16(k), np16(kn)[:, :, None]], axis=2)
    vall = np.concatenate([np16(v), np16(vn)[:, :, None]], axis=2)
    del k, v
    qk, sk = quant.quantize_int4_fp16_scale(kall, w.group_k)
    kc, ks, vc, vs = cache_arrays(dc, "int4h")
    assert np.array_equal(ks[:, :, L - 1].view(np.uint16), sk[:, :, L - 1].view(np.uint16))
    assert np.array_equal(quant.unpack_nibbles(kc[:, :, L - 1]), qk[:, :, L - 1])
    kh = quant.dequantize_int4_exact(qk, sk, w.group_k)
    del qk, sk
    qv, sv = quant.quantize_int4_fp16_scale(vall, w.group_v)
    vh = quant.dequantize_int4_exact(qv, sv, w.group_v)
    ref = attention.decode_attention(np16(q), kh, vh, [L] * w.batch)
    assert_attn_close(eager.cpu().numpy(), ref, "int4h benched step, eager")
    assert_attn_close(replayed.cpu().numpy(), ref, "int4h benched step, graph")
