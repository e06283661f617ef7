"""Recent tokens kept in fp16 besides their INT4 codes, on the GPU.

"LLM长上下文推理优化：用INT4状态机管理KV Cache" (pwwt.cn/news/4219524), section 8.3: the
older tokens' K/V in INT4, the recent ones in FP16.  A cache with recent = R keeps the
last R positions written in fp16 rings [B, Hkv, R, D] (position p in row p mod R) and
still quantizes every position; decode reads [len - R, len) from the rings and older
positions from the codes.  Checked here: the rings after prefills and appends (bit for
bit), the codes unchanged by the rings, and decode attention against the oracle's
``decode_attention`` over ``recent_fp16_rows`` (plain and fused append, every GQA group
and K group of the matrix-core kernel, windows, split counts, a running decode loop).
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, quant
from tests.kvq_testutil import append_decode, assert_attn_close, decode, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _hat(x16, g):
    c, s = quant.quantize_int4(x16, g)
    return quant.dequantize_int4_exact(c, s, g)


def _sub_cache(dc, b):
    """The kvq_cache of sequence b alone (batch 1 views of every buffer)."""
    B = dc.desc.batch
    return kvq.kvq_cache(*[t.view(B, -1)[b].data_ptr() for t in
                           (dc.k_codes, dc.k_scales, dc.v_codes, dc.v_scales, dc.k_recent, dc.v_recent)])


def _one(desc):
    return kvq.make_desc("int4", 1, desc.kv_heads, desc.head_dim, desc.capacity, desc.group_k,
                         desc.group_v, recent=desc.recent)


def _rings(dc):
    d = dc.desc
    torch.cuda.synchronize()
    shape = (d.batch, d.kv_heads, d.recent, d.head_dim)
    return dc.k_recent.view(shape).cpu().numpy(), dc.v_recent.view(shape).cpu().numpy()


def test_rings_after_prefill_and_append_bit_exact():
    B, H, D, C, R = 2, 2, 128, 400, 100
    L = 330
    k = synth.kv_source((B, H, L, D), 101, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, L, D), 102, DEV, outlier_channels=2)
    desc = kvq.make_desc("int4", B, H, D, C, recent=R)
    plain = kvq.make_desc("int4", B, H, D, C)
    dc, dp = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(plain, DEV)
    k16, v16 = np16(k), np16(v)
    # a first chunk shorter than the ring: rows 0 .. 49 hold positions 0 .. 49
    for d_, c_ in ((desc, dc), (plain, dp)):
        kvq.kvq_quantize_prefill(d_, c_.c, k[:, :, :50].contiguous(), v[:, :, :50].contiguous(), 0, 50)
    kr, vr = _rings(dc)
    assert np.array_equal(kr[:, :, :50].view(np.uint16), k16[:, :, :50].view(np.uint16))
    assert np.array_equal(vr[:, :, :50].view(np.uint16), v16[:, :, :50].view(np.uint16))
    # then [50, 300): the ring keeps the call's last 100 positions
    for d_, c_ in ((desc, dc), (plain, dp)):
        kvq.kvq_quantize_prefill(d_, c_.c, k[:, :, 50:300].contiguous(), v[:, :, 50:300].contiguous(), 50, 250)
    # and one position at a time up to 330
    for t in range(300, L):
        for d_, c_ in ((desc, dc), (plain, dp)):
            kvq.kvq_append(d_, c_.c, k[:, :, t].contiguous(), v[:, :, t].contiguous(), [t] * B)
    kr, vr = _rings(dc)
    for p in range(L - R, L):
        assert np.array_equal(kr[:, :, p % R].view(np.uint16), k16[:, :, p].view(np.uint16)), p
        assert np.array_equal(vr[:, :, p % R].view(np.uint16), v16[:, :, p].view(np.uint16)), p
    # the codes and scales are those of a cache without rings
    for x, y in ((dc.k_codes, dp.k_codes), (dc.k_scales, dp.k_scales), (dc.v_codes, dp.v_codes),
                 (dc.v_scales, dp.v_scales)):
        assert torch.equal(x, y)


CASES = [
    # G, group_k, recent, lens, window, num_splits
    (4, 64, 128, [1000, 700], 0, 0),
    (4, 64, 128, [1000, 50], 0, 0),          # sequence 1 shorter than the recent span
    (1, 128, 1, [900, 333], 0, 0),           # one fp16 row: the last position only
    (2, 32, 300, [1200, 301], 0, 5),         # 5 splits share the 300 fp16 rows
    (8, 64, 64, [800, 640], 0, 1),           # one split takes every row
    (8, 128, 1024, [1500, 1024], 0, 0),      # 1024 = len: sequence 1 all fp16
    (4, 32, 256, [1100, 900], 500, 0),       # window longer than the recent span
    (2, 64, 300, [1000, 777], 200, 0),       # recent span longer than the window
    (4, 64, 100, [1000, 640], 0, 40),        # 40 splits, 3 fp16 rows each, merged in-kernel
    (4, 64, 3, [1000, 640], 0, 16),          # more splits than fp16 rows
]


@pytest.mark.parametrize("case", CASES, ids=[f"recent{i}" for i in range(len(CASES))])
def test_decode_with_recent_fp16_rows(case):
    G, gk, R, lens, W, ns = case
    B, Hkv, D = len(lens), 2, 128
    L = max(lens)
    k = synth.kv_source((B, Hkv, L, D), 111 + R, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 112 + R, DEV, outlier_channels=2)
    q = synth.query((B, Hkv * G, D), 113 + R, DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, L, gk, 128, recent=R)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, L)
    for b, ln in enumerate(lens):     # a shorter sequence's rings hold its own last R
        if ln < L:
            lo = max(0, ln - R)
            kvq.kvq_quantize_prefill(_one(desc), _sub_cache(dc, b), k[b:b + 1, :, lo:ln].contiguous(),
                                     v[b:b + 1, :, lo:ln].contiguous(), lo, ln - lo)
    k16, v16 = np16(k), np16(v)
    K = attention.recent_fp16_rows(_hat(k16, gk), k16, lens, R)
    V = attention.recent_fp16_rows(_hat(v16, 128), v16, lens, R)
    ref = attention.decode_attention(np16(q), K, V, lens, W)
    out = decode(desc, dc, q, Hkv * G, lens, W, 0.0, ns)
    assert_attn_close(out.cpu().numpy(), ref, f"{case}")
    # the same buffers under a descriptor without rings: every position from the codes
    plain = kvq.make_desc("int4", B, Hkv, D, L, gk, 128)
    ref_int4 = attention.decode_attention(np16(q), _hat(k16, gk), _hat(v16, 128), lens, W)
    out_plain = decode(plain, dc, q, Hkv * G, lens, W, 0.0, ns)
    assert_attn_close(out_plain.cpu().numpy(), ref_int4, f"{case} without rings")


@pytest.mark.parametrize("G,gk,R", [(4, 64, 128), (8, 128, 300), (1, 32, 1)])
def test_fused_append_decode_with_recent_rows(G, gk, R):
    """The step's new row is attended at its fp16 value, stored in ring row (len - 1) mod
    R and quantized into the codes; the unfused pair (append, then decode) agrees."""
    B, Hkv, D, L = 2, 2, 128, 900
    k = synth.kv_source((B, Hkv, L, D), 121, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 122, DEV, outlier_channels=2)
    q = synth.query((B, Hkv * G, D), 123, DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, L, gk, 128, recent=R)
    dc, du = kvq.DeviceCache(desc, DEV), kvq.DeviceCache(desc, DEV)
    for c_ in (dc, du):
        kvq.kvq_quantize_prefill(desc, c_.c, k[:, :, :L - 1].contiguous(), v[:, :, :L - 1].contiguous(), 0, L - 1)
    kn, vn = k[:, :, L - 1].contiguous(), v[:, :, L - 1].contiguous()
    out = append_decode(desc, dc, kn, vn, q, Hkv * G, [L, L])
    k16, v16 = np16(k), np16(v)
    K = attention.recent_fp16_rows(_hat(k16, gk), k16, [L, L], R)
    V = attention.recent_fp16_rows(_hat(v16, 128), v16, [L, L], R)
    ref = attention.decode_attention(np16(q), K, V, [L, L])
    assert_attn_close(out.cpu().numpy(), ref, f"fused G={G} gk={gk} R={R}")
    kvq.kvq_append(desc, du.c, kn, vn, [L - 1, L - 1])
    out_u = decode(desc, du, q, Hkv * G, [L, L])
    assert_attn_close(out_u.cpu().numpy(), ref, f"unfused G={G} gk={gk} R={R}")
    # both paths leave the same cache: codes, scales and rings
    torch.cuda.synchronize()
    for x, y in ((dc.k_codes, du.k_codes), (dc.k_scales, du.k_scales), (dc.v_codes, du.v_codes),
                 (dc.v_scales, du.v_scales), (dc.k_recent, du.k_recent), (dc.v_recent, du.v_recent)):
        assert torch.equal(x, y)
    kr, _ = _rings(dc)
    assert np.array_equal(kr[:, :, (L - 1) % R].view(np.uint16), k16[:, :, L - 1].view(np.uint16))


def test_recent_decode_loop():
    """Consecutive fused steps over one cache and one workspace, each checked against the
    oracle: positions move from the rings to the codes as the sequence grows."""
    B, Hkv, G, D, R = 2, 2, 4, 128, 64
    P, steps = 500, 6
    L = P + steps
    k = synth.kv_source((B, Hkv, L, D), 131, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 132, DEV, outlier_channels=2)
    desc = kvq.make_desc("int4", B, Hkv, D, L, 64, 128, recent=R)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :P].contiguous(), v[:, :, :P].contiguous(), 0, P)
    ws = kvq.decode_workspace(desc, Hkv * G, L, 0, 70, DEV)
    k16, v16 = np16(k), np16(v)
    kh, vh = _hat(k16, 64), _hat(v16, 128)
    for i, ns in enumerate((0, 1, 7, 16, 40, 70)):
        ln = P + i + 1
        q = synth.query((B, Hkv * G, D), 140 + i, DEV)
        out = append_decode(desc, dc, k[:, :, ln - 1].contiguous(), v[:, :, ln - 1].contiguous(), q,
                            Hkv * G, [ln, ln], 0, 0.0, ns, ws)
        ref = attention.decode_attention(np16(q), attention.recent_fp16_rows(kh, k16, [ln, ln], R),
                                         attention.recent_fp16_rows(vh, v16, [ln, ln], R), [ln, ln])
        assert_attn_close(out.cpu().numpy(), ref, f"step {i} splits {ns}")
        assert int(ws[: B * Hkv].view(torch.int32).abs().sum()) == 0
