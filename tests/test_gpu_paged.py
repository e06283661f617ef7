"""Paged KV cache on the GPU ("AI 推理性能调优：KV Cache 优化与显存管理的工程实践",
bxzpzcl.cn/news/2871434, section 3.1 KVCacheManager: fixed pages from a pool; section 4:
16-64 token pages).

Block tables come from the oracle's page manager over a shuffled free list, so a
sequence's pages are scattered over the pool in no order.  Checked: the rows the
library writes (prefill and appends), gathered through the table by the oracle, equal
the oracle's quantization of the same positions (bit for bit; codec indices by the
boundary rule); dequantization through the table; decode attention on every kernel
path (INT4 and INT8 matrix-core, codec and fp16-scale split-K, head_dim 64) against the
fp64 oracle at max abs 2e-3 / rel-L2 1e-4, windows, ragged lengths, split counts and the
fused append included; and the paged step against the contiguous one.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import attention, codec, paged, quant
from tests.kvq_testutil import (append_decode, assert_attn_close, check_codec_rows, codec_indices,
                                decode, np16)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _table(B, cap, P, lens, seed, spare=3):
    """Block table [B, cap / P] from the page manager over a shuffled free list; entries
    past a sequence's pages point at page 0 (never attended)."""
    pps = cap // P
    need = sum((ln + P - 1) // P for ln in lens)
    mgr = paged.PageManager(page_size=P, max_pages=need + spare)
    mgr.free_pages = list(np.random.default_rng(seed).permutation(mgr.max_pages))
    t = np.zeros((B, pps), np.int32)
    for b, ln in enumerate(lens):
        got = mgr.allocate(f"seq{b}", ln)
        t[b, :len(got)] = got
    return t, mgr.max_pages


def _paged_cache(fmt, B, H, D, cap, P, lens, seed, gk=64, gv=128):
    table, pages = _table(B, cap, P, lens, seed)
    desc = kvq.make_desc(fmt, B, H, D, cap, min(gk, D), min(gv, D), page_size=P, num_pages=pages)
    dc = kvq.DeviceCache(desc, DEV, block_table=torch.from_numpy(table).to(DEV))
    return desc, dc, table


def _pool(dc, fmt):
    """(k_codes, k_scales, v_codes, v_scales) of a paged cache as [pages, H, P, .]."""
    d = dc.desc
    n, H, P, D = d.num_pages, d.kv_heads, d.page_size, d.head_dim
    torch.cuda.synchronize()
    row = D if fmt == "int8" else (3 * D // 8 if fmt == "codec3" else D // 2)
    kc = dc.k_codes.cpu().numpy().reshape(n, H, P, row)
    vc = dc.v_codes.cpu().numpy().reshape(n, H, P, row)
    if fmt == "int8":
        kc, vc = kc.view(np.int8), vc.view(np.int8)
    if fmt == "int4h":
        ks = dc.k_scales.cpu().numpy().view(np.float16)[:n * H * P * (D // d.group_k)].reshape(n, H, P, -1)
        vs = dc.v_scales.cpu().numpy().view(np.float16)[:n * H * P * (D // d.group_v)].reshape(n, H, P, -1)
    else:
        ks = dc.k_scales.cpu().numpy().reshape(n, H, P, -1)
        vs = dc.v_scales.cpu().numpy().reshape(n, H, P, -1)
    return kc, ks, vc, vs


def _logical(dc, fmt, table, lens):
    """The pool gathered through the table into [B, H, N, .] (the oracle's gather)."""
    P = dc.desc.page_size
    return [paged.gather(x, table, lens, P) for x in _pool(dc, fmt)]


def _oracle_codes(fmt, x16, g):
    if fmt == "int4":
        q, s = quant.quantize_int4(x16, g)
        return quant.pack_nibbles(q), s
    if fmt == "int4h":
        q, s = quant.quantize_int4_fp16_scale(x16, g)
        return quant.pack_nibbles(q), s
    q, s = quant.quantize_int8(x16)
    return q, s[..., None]


def _hat_from_logical(fmt, lg, k16, v16, lens, gk, gv):
    """Dequantized rows for the oracle's attention: the oracle's own quantization for
    the integer formats (their codes are checked bit for bit first), the GPU's indices
    held to the codec rule for the codec."""
    kc, ks, vc, vs = lg
    if fmt in ("codec", "codec3"):
        bits = 3 if fmt == "codec3" else 4
        out = []
        for x16, c_, s_ in ((k16, kc, ks), (v16, vc, vs)):
            idx, sc, _ = codec.encode(x16, bits=bits)
            for b, ln in enumerate(lens):
                g_idx = codec_indices(c_[b, :, :ln], fmt)
                check_codec_rows(g_idx, s_[b, :, :ln, 0], x16[b, :, :ln], bits)
                idx[b, :, :ln] = g_idx
                sc[b, :, :ln] = s_[b, :, :ln, 0]
            out.append(codec.decode(idx, sc, bits=bits))
        return out
    for x16, c_, s_, g in ((k16, kc, ks, gk), (v16, vc, vs, gv)):
        oc, osc = _oracle_codes(fmt, x16, g)
        for b, ln in enumerate(lens):
            assert np.array_equal(c_[b, :, :ln], oc[b, :, :ln]), f"{fmt} codes of sequence {b}"
            assert np.array_equal(np.asarray(s_[b, :, :ln]).view(np.uint8),
                                  np.asarray(osc[b, :, :ln]).view(np.uint8)), f"{fmt} scales of sequence {b}"
    if fmt == "int8":
        qk, sk = quant.quantize_int8(k16)
        qv, sv = quant.quantize_int8(v16)
        return quant.dequantize_int8_exact(qk, sk), quant.dequantize_int8_exact(qv, sv)
    qf = quant.quantize_int4 if fmt == "int4" else quant.quantize_int4_fp16_scale
    qk, sk = qf(k16, gk)
    qv, sv = qf(v16, gv)
    return (quant.dequantize_int4_exact(qk, np.asarray(sk, np.float32), gk),
            quant.dequantize_int4_exact(qv, np.asarray(sv, np.float32), gv))


LAYOUT_CASES = [
    # fmt, D, P
    ("int4", 128, 16), ("int4", 128, 64), ("int8", 128, 32), ("int4h", 128, 16),
    ("codec", 256, 32), ("int4", 64, 256),
]


@pytest.mark.parametrize("fmt,D,P", LAYOUT_CASES, ids=[f"{c[0]}-{c[1]}-p{c[2]}" for c in LAYOUT_CASES])
def test_paged_rows_through_the_table(fmt, D, P):
    """Prefill in two calls, then three one-position appends: every written row, read
    back through the block table, is the oracle's quantization of that position."""
    B, H = 3, 2
    lens = [5 * P + 7, 3 * P, 2 * P + 1]
    L = max(lens)
    cap = ((L + 3 + P - 1) // P + 1) * P
    k = synth.kv_source((B, H, L + 3, D), 3100 + P, DEV, outlier_channels=2,
                        zero_groups=((0, 1, 3, 0, D),))
    v = synth.kv_source((B, H, L + 3, D), 3200 + P, DEV, outlier_channels=2)
    # every sequence gets pages for all L + 3 positions (each prefill call writes its
    # positions for every sequence); the appends then rewrite three positions of each
    desc, dc, table = _paged_cache(fmt, B, H, D, cap, P, [L + 3] * B, 3300 + P)
    half = L // 2
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :half].contiguous(), v[:, :, :half].contiguous(), 0, half)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, half:L].contiguous(), v[:, :, half:L].contiguous(), half, L - half)
    # each sequence appends its own next three positions
    for i in range(3):
        pos = [ln + i for ln in lens]
        idx = torch.tensor(pos, device=DEV)
        ar = torch.arange(B, device=DEV)
        kvq.kvq_append(desc, dc.c, k[ar, :, idx].contiguous(), v[ar, :, idx].contiguous(), pos)
    # written: [0, L) by the prefill and ln .. ln + 2 of sequence b by the appends (the
    # same source rows where they overlap the prefill)
    written = [max(L, ln + 3) for ln in lens]
    lg = _logical(dc, fmt, table, written)
    _hat_from_logical(fmt, lg, np16(k), np16(v), written, min(64, D), min(128, D))


@pytest.mark.parametrize("fmt,P", [("int4", 16), ("int8", 64), ("codec", 32)])
def test_paged_dequant(fmt, P):
    B, H, D = 2, 2, 128
    n = 4 * P + 9
    cap = 6 * P
    k = synth.kv_source((B, H, n, D), 3400 + P, DEV, outlier_channels=2)
    v = synth.kv_source((B, H, n, D), 3500 + P, DEV, outlier_channels=2)
    desc, dc, table = _paged_cache(fmt, B, H, D, cap, P, [n, n], 3600 + P)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, n)
    start, cnt = P - 3, 2 * P + 5       # across page boundaries
    out = torch.empty((B, H, cnt, D), dtype=torch.float32, device=DEV)
    kvq.kvq_dequant(desc, dc.c, 1, start, cnt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    vn = np16(v)[:, :, start:start + cnt]
    if fmt == "codec":   # the oracle decodes the indices the GPU stored (held to the rule)
        lg = _logical(dc, fmt, table, [n, n])
        idx = quant.unpack_nibbles(lg[2][:, :, start:start + cnt], signed=False)
        check_codec_rows(idx, lg[3][:, :, start:start + cnt, 0], vn, 4)
        ref = codec.decode(idx, lg[3][:, :, start:start + cnt, 0])
        assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    elif fmt == "int8":
        q, s = quant.quantize_int8(vn)
        assert np.array_equal(got, quant.dequantize_int8(q, s))
    else:
        q, s = quant.quantize_int4(vn, 128)
        assert np.array_equal(got, quant.dequantize_int4(q, s, 128))


DECODE_CASES = [
    # fmt, D, G, gk, P, lens, window, nsplit, fused
    ("int4", 128, 4, 64, 16, [8193, 3000], 0, 0, False),   # matrix-core, two pages per tile
    ("int4", 128, 4, 64, 32, [2000, 777], 0, 5, False),
    ("int4", 128, 8, 32, 64, [1500, 1500], 700, 3, False),   # window, 16 columns
    ("int4", 128, 2, 128, 256, [3333, 100], 0, 0, False),
    ("int4", 128, 4, 64, 16, [4097, 1025], 1000, 2, True),  # fused append, window
    ("int4", 128, 1, 64, 16, [1, 17], 0, 0, True),          # one-position sequence
    ("int8", 128, 4, 64, 16, [3000, 1234], 0, 0, False),    # INT8 tiles
    ("int8", 128, 2, 64, 64, [2500, 2500], 900, 4, False),
    ("codec", 256, 2, 64, 32, [2000, 600], 512, 0, True),   # codec split-K, fused
    ("int4h", 128, 4, 64, 16, [1800, 900], 0, 0, True),     # fp16 scales, matrix-core, fused
    ("int4h", 128, 2, 64, 32, [2000, 1300], 600, 3, False),  # fp16 scales, matrix-core, window
    ("int4h", 64, 4, 32, 16, [900, 400], 0, 0, True),       # fp16 scales, split-K, fused
    ("int4", 64, 4, 64, 16, [1200, 300], 0, 40, False),     # head_dim 64 split-K + merge kernel
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"paged{i}" for i in range(len(DECODE_CASES))])
def test_paged_decode(case):
    fmt, D, G, gk, P, lens, W, ns, fused = case
    B, H = len(lens), 2
    L = max(lens)
    cap = ((L + P - 1) // P + 1) * P
    k = synth.kv_source((B, H, L, D), 3700 + P + L, DEV, outlier_channels=3)
    v = synth.kv_source((B, H, L, D), 3800 + P + L, DEV, outlier_channels=3,
                        zero_groups=((0, 0, 0, 0, D),))
    q = synth.query((B, H * G, D), 3900 + P + L, DEV)
    # pages for L positions in every sequence (the prefill writes L rows of each); the
    # per-sequence lengths are what the decode attends
    desc, dc, table = _paged_cache(fmt, B, H, D, cap, P, [L] * B, 4000 + P + L, gk=gk)
    pre = L - 1 if fused else L
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :pre].contiguous(), v[:, :, :pre].contiguous(), 0, pre)
    if fused:
        idx = torch.tensor([ln - 1 for ln in lens], device=DEV)
        ar = torch.arange(B, device=DEV)
        out = append_decode(desc, dc, k[ar, :, idx].contiguous(), v[ar, :, idx].contiguous(), q,
                            H * G, lens, W, 0.0, ns)
    else:
        out = decode(desc, dc, q, H * G, lens, W, 0.0, ns)
    k16, v16 = np16(k), np16(v)
    lg = _logical(dc, fmt, table, lens)
    kh, vh = _hat_from_logical(fmt, lg, k16, v16, lens, min(gk, D), min(128, D))
    ref = attention.decode_attention(np16(q), kh, vh, lens, W)
    assert_attn_close(out.cpu().numpy(), ref, f"paged {case}")


def test_paged_step_equals_contiguous_step():
    """The Llama-3-8B-shaped layer (batch 8, 8 KV heads, 32 query heads, 8193 positions)
    in pages of 16 (the benchmark's paged workload) and in the contiguous layout: the
    fused step leaves the same codes in every logical row, and its output meets the
    attention bar against the oracle (over the oracle's own codes, which the logical
    rows equal bit for bit)."""
    w = synth.WORKLOADS[2]
    k, v, q, kn, vn = synth.layer_inputs(w, 3, DEV)
    B, H, D, S = w.batch, w.kv_heads, w.head_dim, w.context
    L = S + 1
    P = 16
    cap = (L + P - 1) // P * P
    lens = [L] * B
    desc_c = kvq.make_desc("int4", B, H, D, L)
    dcc = kvq.DeviceCache(desc_c, DEV)
    desc_p, dcp, table = _paged_cache("int4", B, H, D, cap, P, lens, 4100)
    for desc, dc in ((desc_c, dcc), (desc_p, dcp)):
        kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, S)
    oc = append_decode(desc_c, dcc, kn, vn, q, w.q_heads, lens)
    op = append_decode(desc_p, dcp, kn, vn, q, w.q_heads, lens)
    lg = _logical(dcp, "int4", table, lens)
    cont = [x.cpu().numpy().reshape(B, H, L, -1) for x in (dcc.k_codes, dcc.k_scales, dcc.v_codes, dcc.v_scales)]
    for a_, b_ in zip(lg, cont):
        assert np.array_equal(np.asarray(a_).view(np.uint8), np.asarray(b_).view(np.uint8))
    del cont
    kall = np.concatenate([np16(k), np16(kn)[:, :, None]], axis=2)
    vall = np.concatenate([np16(v), np16(vn)[:, :, None]], axis=2)
    del k, v
    kh, vh = _hat_from_logical("int4", lg, kall, vall, lens, 64, 128)
    ref = attention.decode_attention(np16(q), kh, vh, lens)
    assert_attn_close(op.cpu().numpy(), ref, "paged step at full size")
    assert_attn_close(oc.cpu().numpy(), ref, "contiguous step at full size")
