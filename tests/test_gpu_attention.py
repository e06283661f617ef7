"""GPU parity of split-K decode attention over the packed cache against the fp64 oracle.

Bar (over the same dequantized values): max abs error <= 2e-3 and relative L2 error
<= 1e-4 of the fp32 output.  Semantics: bxzpzcl.cn/news/2871434 §3.2 (window, GQA,
scale), lpnh.cn/news/2042373 §1.1 (append then attend over the whole cache).
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


def _fill(fmt, k, v, cap, gk=64, gv=128):
    B, H, S, D = k.shape
    gk, gv = min(gk, D), min(gv, D)
    desc = kvq.make_desc(fmt, B, H, D, cap, gk, gv)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, S)
    return desc, dc


def _oracle_hat(fmt, k16, v16, gk=64, gv=128):
    D = k16.shape[-1]
    gk, gv = min(gk, D), min(gv, D)
    if fmt == "int4":
        qk, sk = quant.quantize_int4(k16, gk)
        qv, sv = quant.quantize_int4(v16, gv)
        return quant.dequantize_int4_exact(qk, sk, gk), quant.dequantize_int4_exact(qv, sv, gv)
    qk, sk = quant.quantize_int8(k16)
    qv, sv = quant.quantize_int8(v16)
    return quant.dequantize_int8_exact(qk, sk), quant.dequantize_int8_exact(qv, sv)


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_tiny_workload(fmt):
    w = synth.WORKLOADS[1]
    k, v, q, _, _ = synth.layer_inputs(w, 0, DEV)
    desc, dc = _fill(fmt, k, v, w.context)
    out = decode(desc, dc, q, w.q_heads, [w.context])
    kh, vh = _oracle_hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, [w.context])
    assert_attn_close(out.cpu().numpy(), ref, f"tiny {fmt}")


CASES = [
    # B, Hkv, G, D, lens, window, nsplit
    (2, 2, 1, 128, [1, 2], 0, 0),
    (3, 2, 2, 64, [37, 300, 129], 0, 0),
    (2, 3, 4, 128, [513, 77], 0, 3),
    (2, 1, 8, 128, [600, 64], 0, 7),
    (2, 2, 4, 256, [257, 1000], 0, 0),
    (2, 2, 4, 128, [700, 700], 100, 0),
    (1, 2, 2, 128, [1000], 999, 5),
    (2, 2, 4, 128, [50, 1000], 0, 64),     # more splits than positions of sequence 0
    (1, 2, 4, 128, [4000], 0, 130),        # more splits than lanes in the in-kernel merge
    (4, 1, 1, 64, [5, 17, 33, 65], 16, 0),
]


@pytest.mark.parametrize("fmt", ["int4", "int8"])
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_shapes_lengths_windows_splits(fmt, case):
    B, Hkv, G, D, lens, window, nsplit = case
    S = max(lens)
    k = synth.kv_source((B, Hkv, S, D), 100 + S, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, S, D), 200 + S, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 300 + S, DEV)
    desc, dc = _fill(fmt, k, v, S)
    out = decode(desc, dc, q, Hkv * G, lens, window, 0.0, nsplit)
    kh, vh = _oracle_hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, lens, window)
    assert_attn_close(out.cpu().numpy(), ref, f"{fmt} {case}")


def test_split_count_invariance_and_scale():
    B, Hkv, G, D, S = 2, 2, 4, 128, 2000
    k = synth.kv_source((B, Hkv, S, D), 5, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, S, D), 6, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 7, DEV)
    desc, dc = _fill("int4", k, v, S)
    kh, vh = _oracle_hat("int4", np16(k), np16(v))
    for ns in (1, 2, 9, 31, 0):
        out = decode(desc, dc, q, Hkv * G, [S, 1500], 0, 0.0, ns)
        ref = attention.decode_attention(np16(q), kh, vh, [S, 1500])
        assert_attn_close(out.cpu().numpy(), ref, f"nsplit={ns}")
    out = decode(desc, dc, q, Hkv * G, [S, 1500], 0, 0.25)
    ref = attention.decode_attention(np16(q), kh, vh, [S, 1500], scale=0.25)
    assert_attn_close(out.cpu().numpy(), ref, "scale=0.25")


def test_ring_window_equals_unwrapped():
    """A window layer whose ring (capacity W) has wrapped attends exactly like the
    unwrapped cache restricted to the last W positions."""
    B, Hkv, G, D, W, L = 2, 2, 2, 128, 256, 1000
    k = synth.kv_source((B, Hkv, L, D), 8, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 9, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 10, DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, W)
    dc = kvq.DeviceCache(desc, DEV)
    for start in range(0, L, W):        # prefill in W-sized chunks through the ring
        n = min(W, L - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    out = decode(desc, dc, q, Hkv * G, [L, L], W)
    kh, vh = _oracle_hat("int4", np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, [L, L], W)
    assert_attn_close(out.cpu().numpy(), ref, "ring")


def test_llama8b_shape_full_layer_with_append():
    """One full layer of the Llama-3-8B-shaped decode step: prefill 8192 positions,
    append the new token (position 8192), attend over 8193 with GQA 4:1, batch 8.
    Both forms of the step are held to the oracle: kvq_append + kvq_decode_attn, and the
    one-launch kvq_append_decode_attn with the library's split plan, eager and replayed
    from a HIP graph (the call and launch configuration the benchmark times)."""
    w = synth.WORKLOADS[2]
    layer = 5
    k, v, q, kn, vn = synth.layer_inputs(w, layer, DEV)
    L = w.context + 1
    desc, dc = _fill("int4", k, v, L)
    dfused = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dfused.c, k, v, 0, w.context)
    kvq.kvq_append(desc, dc.c, kn, vn, [w.context] * w.batch)
    out = decode(desc, dc, q, w.q_heads, [L] * w.batch)
    assert kvq.kvq_plan_splits(desc, w.q_heads, L) == 4
    ws = kvq.decode_workspace(desc, w.q_heads, L, device=DEV)
    fused = append_decode(desc, dfused, kn, vn, q, w.q_heads, [L] * w.batch, ws=ws)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    replayed = torch.full_like(fused, float("nan"))
    with torch.cuda.graph(g, stream=s):
        kvq.kvq_append_decode_attn(desc, dfused.c, kn, vn, q, w.q_heads, [L] * w.batch, 0, 0.0, 0,
                                   replayed, ws)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(dc, name), getattr(dfused, name)), name
    kall = np.concatenate([np16(k), np16(kn)[:, :, None]], axis=2)
    vall = np.concatenate([np16(v), np16(vn)[:, :, None]], axis=2)
    del k, v
    kh, vh = _oracle_hat("int4", kall, vall)
    ref = attention.decode_attention(np16(q), kh, vh, [L] * w.batch)
    assert_attn_close(out.cpu().numpy(), ref, "llama8b layer, append + decode")
    assert_attn_close(fused.cpu().numpy(), ref, "llama8b layer, fused step")
    assert_attn_close(replayed.cpu().numpy(), ref, "llama8b layer, fused step from a graph")


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_128k_single_sequence(fmt):
    """The 128K-context, batch-1 split-K workload (one layer), INT4 and INT8."""
    w = synth.WORKLOADS[5]
    k, v, q, _, _ = synth.layer_inputs(w, 0, DEV)
    desc, dc = _fill(fmt, k, v, w.context)
    out = decode(desc, dc, q, w.q_heads, [w.context])
    kn, vn = np16(k), np16(v)
    del k, v
    kh, vh = _oracle_hat(fmt, kn, vn)
    ref = attention.decode_attention(np16(q), kh, vh, [w.context])
    assert_attn_close(out.cpu().numpy(), ref, f"128k {fmt}")


def test_mha7b_shape_sampled_heads():
    """The MHA-7B-shaped 20K x 8 workload (G = 1): full launch, oracle on sampled
    (batch, head) pairs."""
    w = synth.WORKLOADS[3]
    k, v, q, _, _ = synth.layer_inputs(w, 0, DEV)
    desc, dc = _fill("int4", k, v, w.context)
    out = decode(desc, dc, q, w.q_heads, [w.context] * w.batch).cpu().numpy()
    for (b, h) in [(0, 0), (3, 17), (7, 31)]:
        kn = k[b:b + 1, h:h + 1].cpu().numpy()
        vn = v[b:b + 1, h:h + 1].cpu().numpy()
        kh, vh = _oracle_hat("int4", kn, vn)
        ref = attention.decode_attention(np16(q[b:b + 1, h:h + 1]), kh, vh, [w.context])
        assert_attn_close(out[b:b + 1, h:h + 1], ref, f"mha7b b={b} h={h}")


MFMA_CASES = [
    # gk, G, lens, window, cap    (head_dim 128, V group 128: the matrix-core kernel)
    (32, 1, [33, 1000], 0, None),
    (64, 2, [511, 97], 0, None),
    (128, 4, [700, 1], 0, None),
    (32, 8, [1025, 640], 0, None),
    (64, 4, [1500, 1500], 300, 512),    # window ring, capacity 512 (wraps)
    (128, 8, [2049, 40], 0, None),
    (64, 8, [1300, 33], 0, None),       # 16 (head, group) columns: one position set
    (32, 4, [777, 1024], 0, None),      # 16 columns, K group 32
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=[f"mfma{i}" for i in range(len(MFMA_CASES))])
def test_int4_matrix_core_path(case):
    gk, G, lens, window, cap = case
    B, Hkv, D = len(lens), 2, 128
    S = max(lens)
    k = synth.kv_source((B, Hkv, S, D), 400 + gk + G, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, S, D), 500 + gk + G, DEV, outlier_channels=3,
                        zero_groups=((0, 1, 0, 0, D),))
    q = synth.query((B, Hkv * G, D), 600 + gk + G, DEV)
    C = cap or S
    desc = kvq.make_desc("int4", B, Hkv, D, C, gk, 128)
    dc = kvq.DeviceCache(desc, DEV)
    for start in range(0, S, C):
        n = min(C, S - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    for ns in (0, 1, 5):
        out = decode(desc, dc, q, Hkv * G, lens, window, 0.0, ns)
        kh, vh = _oracle_hat("int4", np16(k), np16(v), gk, 128)
        ref = attention.decode_attention(np16(q), kh, vh, lens, window)
        assert_attn_close(out.cpu().numpy(), ref, f"mfma {case} nsplit={ns}")


INT8_MFMA_CASES = [
    # G, lens, window, cap    (head_dim 128: the matrix-core kernel with 16-position tiles)
    (1, [33, 1000], 0, None),
    (2, [511, 17], 0, None),
    (4, [16, 15, 1], 0, None),          # contexts of one tile or less
    (8, [1025, 640], 0, None),
    (4, [1500, 1500], 300, 512),        # window ring, capacity 512 (wraps)
    (4, [700, 300], 0, None),
]


@pytest.mark.parametrize("case", INT8_MFMA_CASES, ids=[f"int8mfma{i}" for i in range(len(INT8_MFMA_CASES))])
def test_int8_matrix_core_path(case):
    G, lens, window, cap = case
    B, Hkv, D = len(lens), 2, 128
    S = max(lens)
    k = synth.kv_source((B, Hkv, S, D), 700 + G, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, S, D), 800 + G, DEV, outlier_channels=3,
                        zero_groups=((0, 1, 0, 0, D),))
    q = synth.query((B, Hkv * G, D), 900 + G, DEV)
    C = cap or S
    desc = kvq.make_desc("int8", B, Hkv, D, C)
    dc = kvq.DeviceCache(desc, DEV)
    for start in range(0, S, C):
        n = min(C, S - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    kh, vh = _oracle_hat("int8", np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, lens, window)
    for ns in (0, 1, 5):
        out = decode(desc, dc, q, Hkv * G, lens, window, 0.0, ns)
        assert_attn_close(out.cpu().numpy(), ref, f"int8 mfma {case} nsplit={ns}")


@pytest.mark.parametrize("gv,cap", [(64, None), (128, 16)])
def test_int4_generic_fallback(gv, cap):
    """INT4 shapes the matrix-core kernel does not take (V group < head_dim, capacity
    below one tile) run on the generic kernel."""
    B, Hkv, G, D, L = 2, 2, 4, 128, 300
    k = synth.kv_source((B, Hkv, L, D), 71, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 72, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 73, DEV)
    C = cap or L
    desc = kvq.make_desc("int4", B, Hkv, D, C, 64, gv)
    dc = kvq.DeviceCache(desc, DEV)
    for start in range(0, L, C):
        n = min(C, L - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    W = C if cap else 0
    out = decode(desc, dc, q, Hkv * G, [L, L], W)
    kh, vh = _oracle_hat("int4", np16(k), np16(v), 64, gv)
    ref = attention.decode_attention(np16(q), kh, vh, [L, L], W)
    assert_attn_close(out.cpu().numpy(), ref, f"generic gv={gv} cap={cap}")


FUSED_CASES = [
    # fmt, gk, gv, G, D, lens, window, cap, nsplit   (cases 0, 2, 3: matrix-core kernel)
    ("int4", 64, 128, 4, 128, [300, 45], 0, None, 0),
    ("int4", 32, 128, 8, 128, [1100, 1], 0, None, 5),     # a sequence of length 1
    ("int4", 128, 128, 1, 128, [97, 640], 0, None, 64),   # more splits than positions
    ("int4", 64, 128, 2, 128, [900, 900], 256, 256, 0),   # ring of 256 slots, wrapped
    ("int4", 64, 64, 4, 128, [300, 45], 0, None, 0),      # V group 64: append kernel first
    ("int8", 64, 128, 4, 128, [300, 45], 0, None, 3),
    ("codec", 64, 128, 4, 128, [300, 45], 0, None, 0),
    ("codec", 64, 128, 2, 256, [1500, 1], 300, 512, 0),    # codec, ring, a 1-token sequence
    ("codec", 64, 128, 2, 256, [4097, 1025], 1024, 1024, 3),  # window = capacity
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[f"fused{i}" for i in range(len(FUSED_CASES))])
def test_append_decode_step(case):
    """kvq_append_decode_attn: the new token lands in the cache exactly as kvq_append
    stores it, and the attention covers it (lpnh.cn/news/2042373 section 1.1)."""
    fmt, gk, gv, G, D, lens, window, cap, ns = case
    B, Hkv = len(lens), 2
    L = max(lens)
    C = cap or L
    k = synth.kv_source((B, Hkv, L, D), 700 + L, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 800 + L, DEV, outlier_channels=3,
                        zero_groups=((1, 0, 0, 0, D),))
    q = synth.query((B, Hkv * G, D), 900 + L, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, C, gk, gv)
    ref_cache = kvq.DeviceCache(desc, DEV)
    dc = kvq.DeviceCache(desc, DEV)
    # positions 0 .. len_b - 2 from the prefill (ring-chunked), position len_b - 1 new
    for start in range(0, L, C):
        n = min(C, L - start)
        for cache in (dc, ref_cache):
            kvq.kvq_quantize_prefill(desc, cache.c, k[:, :, start:start + n].contiguous(),
                                     v[:, :, start:start + n].contiguous(), start, n)
    # a ring shorter than the longest sequence now holds that sequence's last positions
    # in every row: a shorter sequence gets its own last C - 1 positions back
    one = kvq.make_desc(fmt, 1, Hkv, D, C, gk, gv)
    for b, ln in enumerate(lens):
        lo = max(0, ln - C)
        if ln < L and C < L and ln - 1 > lo:
            for cache in (dc, ref_cache):
                sub = kvq.kvq_cache(*[t.view(B, -1)[b].data_ptr() for t in
                                      (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales)])
                kvq.kvq_quantize_prefill(one, sub, k[b:b + 1, :, lo:ln - 1].contiguous(),
                                         v[b:b + 1, :, lo:ln - 1].contiguous(), lo, ln - 1 - lo)
    idx = torch.tensor([ln - 1 for ln in lens], device=DEV)
    ar = torch.arange(B, device=DEV)
    kn = k[ar, :, idx].contiguous()           # [B, Hkv, D]
    vn = v[ar, :, idx].contiguous()
    # clobber slot len_b - 1 of the fused cache so the call must write it
    for b, ln in enumerate(lens):
        s = (ln - 1) % C
        dc.k_codes.view(B, Hkv, C, -1)[b, :, s] = 0x5A
        dc.v_codes.view(B, Hkv, C, -1)[b, :, s] = 0xA5
        dc.k_scales.view(B, Hkv, C, -1)[b, :, s] = -1.0
        dc.v_scales.view(B, Hkv, C, -1)[b, :, s] = -1.0
    kvq.kvq_append(desc, ref_cache.c, kn, vn, [ln - 1 for ln in lens])
    out = append_decode(desc, dc, kn, vn, q, Hkv * G, lens, window, 0.0, ns)
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(dc, name), getattr(ref_cache, name)), name
    if fmt == "codec":   # over the rows the GPU coded (each held to the codec rule)
        kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), lens, window)
    else:
        kh, vh = _oracle_hat(fmt, np16(k), np16(v), gk, gv)
    ref = attention.decode_attention(np16(q), kh, vh, lens, window)
    assert_attn_close(out.cpu().numpy(), ref, f"fused {case}")


def test_append_decode_loop_reuses_workspace():
    """Eight consecutive decode steps through one workspace (split counters are reset by
    each call), the split count changing between calls; each step matches the oracle."""
    B, Hkv, G, D, P, steps = 2, 2, 4, 128, 500, 8
    L = P + steps
    k = synth.kv_source((B, Hkv, L, D), 31, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 32, DEV, outlier_channels=3)
    qs = synth.query((steps, B, Hkv * G, D), 33, DEV)
    desc = kvq.make_desc("int4", B, Hkv, D, L)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :P].contiguous(), v[:, :, :P].contiguous(), 0, P)
    ws = kvq.decode_workspace(desc, Hkv * G, L, 0, 64, DEV)
    kh, vh = _oracle_hat("int4", np16(k), np16(v))
    for t in range(steps):
        pos = P + t
        q = qs[t].contiguous()
        ns = (0, 1, 7, 64)[t % 4]
        out = append_decode(desc, dc, k[:, :, pos].contiguous(), v[:, :, pos].contiguous(), q,
                            Hkv * G, [pos + 1, pos + 1], 0, 0.0, ns, ws=ws)
        ref = attention.decode_attention(np16(q), kh, vh, [pos + 1, pos + 1])
        assert_attn_close(out.cpu().numpy(), ref, f"step {t} nsplit={ns}")
        counters = ws[: B * Hkv].view(torch.int32)
        assert int(counters.abs().sum()) == 0, "split counters not reset"
    # a smaller batch through the same workspace
    desc1 = kvq.make_desc("int4", 1, Hkv, D, L)
    dc1 = kvq.DeviceCache(desc1, DEV)
    kvq.kvq_quantize_prefill(desc1, dc1.c, k[:1].contiguous(), v[:1].contiguous(), 0, L)
    out = decode(desc1, dc1, qs[0, :1].contiguous(), Hkv * G, [L], 0, 0.0, 9, ws=ws)
    ref = attention.decode_attention(np16(qs[0, :1]), kh[:1], vh[:1], [L])
    assert_attn_close(out.cpu().numpy(), ref, "batch 1 after batch 2")


@pytest.mark.parametrize("fmt,D", [("int8", 128), ("int8", 64), ("codec", 128), ("int4", 256)])
def test_other_paths_loop_reuse_workspace(fmt, D):
    """Consecutive append + decode steps through one workspace on the INT8 matrix-core
    kernel (D = 128) and the split-K kernel (the rest; splits merged in-kernel up to 32,
    by the merge kernel beyond): the split counters are zero after every call and each
    step matches the oracle."""
    B, Hkv, G, P, steps = 2, 2, 2, 300, 7
    L = P + steps
    k = synth.kv_source((B, Hkv, L, D), 41, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, L, D), 42, DEV, outlier_channels=2)
    qs = synth.query((steps, B, Hkv * G, D), 43, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, L, min(64, D), min(128, D))
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :P].contiguous(), v[:, :, :P].contiguous(), 0, P)
    ws = kvq.decode_workspace(desc, Hkv * G, L, 0, 70, DEV)
    if fmt == "codec":
        kidx, ksc, _ = codec.encode(np16(k))
        vidx, vsc, _ = codec.encode(np16(v))
        kh, vh = codec.decode(kidx, ksc), codec.decode(vidx, vsc)
    else:
        kh, vh = _oracle_hat(fmt, np16(k), np16(v), min(64, D), min(128, D))
    for t in range(steps):
        pos = P + t
        q = qs[t].contiguous()
        ns = (0, 1, 7, 16, 17, 40, 70)[t]
        out = append_decode(desc, dc, k[:, :, pos].contiguous(), v[:, :, pos].contiguous(), q,
                            Hkv * G, [pos + 1, pos + 1], 0, 0.0, ns, ws=ws)
        if fmt == "codec":   # over the rows the GPU coded, this step's included
            kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), [pos + 1, pos + 1])
        ref = attention.decode_attention(np16(q), kh, vh, [pos + 1, pos + 1])
        assert_attn_close(out.cpu().numpy(), ref, f"{fmt} D={D} step {t} nsplit={ns}")
        counters = ws[: B * Hkv].view(torch.int32)
        assert int(counters.abs().sum()) == 0, "split counters not reset"


VSCALE_CASES = [
    # fmt, G, V magnitude per position block (multipliers of N(0, 1)), lens, nsplit
    ("int4", 4, "tiny", [3000, 1200], 0),      # V ~ 1e-3 N(0, 1) everywhere
    ("int8", 4, "tiny", [3000, 1200], 0),
    ("int4", 2, "mixed", [4000, 2500], 3),     # 1e-6 .. 1 blocks along the sequence
    ("int8", 8, "mixed", [4000, 2500], 1),
    ("int4", 1, "mixed", [2100, 700], 0),
]


@pytest.mark.parametrize("case", VSCALE_CASES, ids=[f"vscale{i}" for i in range(len(VSCALE_CASES))])
def test_matrix_core_small_and_mixed_value_scales(case):
    """Heads whose V values are small (~1e-3) or change scale by many decades along the
    sequence keep the attention bar on the matrix-core kernels: P' = p * sV enters P.V in
    fp16 hi + lo parts, which must stay in fp16's normal range whatever the V scale."""
    fmt, G, kind, lens, ns = case
    B, Hkv, D = len(lens), 2, 128
    S = max(lens)
    k = synth.kv_source((B, Hkv, S, D), 1300 + G, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, S, D), 1400 + G, DEV, outlier_channels=3).float()
    if kind == "tiny":
        v *= 1e-3
    else:   # blocks of 700 positions from 1e-6 to 1 (fp16 keeps ~1e-6 as subnormals); the
        # largest block is 1 so that the outputs, and the absolute bar, stay at unit scale
        mult = torch.tensor([1e-3, 1e-6, 1.0, 1e-3, 3e-2, 1e-6], device=DEV)
        v *= mult[(torch.arange(S, device=DEV) // 700) % 6].view(1, 1, S, 1)
    v = v.to(torch.float16)
    q = synth.query((B, Hkv * G, D), 1500 + G, DEV)
    desc, dc = _fill(fmt, k, v, S)
    out = decode(desc, dc, q, Hkv * G, lens, 0, 0.0, ns)
    kh, vh = _oracle_hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, lens)
    assert_attn_close(out.cpu().numpy(), ref, f"{fmt} {kind} G={G}")


MANY_SPLIT_CASES = [
    # fmt, gk, G, lens, nsplit, window, cap, sinks, recent, fused
    ("int4", 64, 4, [6000, 4100], 3, 0, None, 0, 0, False),   # ragged units
    ("int4", 32, 8, [5000], 2, 0, None, 0, 0, False),         # 16 columns (one position set)
    ("int4", 64, 4, [20000], 8, 0, None, 0, 0, False),        # many splits
    ("int4", 64, 2, [50000], 2, 0, None, 0, 0, False),        # long splits
    ("int8", 64, 4, [9000, 3000], 4, 0, None, 0, 0, False),   # 16-position tiles
    ("int8", 64, 1, [60000], 32, 0, None, 0, 0, False),       # INT8, many splits
    ("int4", 64, 4, [9000, 9000], 2, 4000, 4096, 0, 0, False),   # window ring
    ("int4", 64, 4, [9000, 5000], 2, 4000, 4100, 4, 0, False),   # sinks + window ring
    ("int4", 64, 4, [7000, 7000], 3, 0, None, 0, 64, False),     # recent fp16 rows
    ("int4", 64, 4, [6001, 6001], 3, 0, None, 0, 0, True),       # fused append
    ("int4", 128, 2, [8193, 8193, 8193, 8193], 0, 0, None, 0, 0, True),   # planned splits
]


@pytest.mark.parametrize("case", MANY_SPLIT_CASES, ids=[f"splits{i}" for i in range(len(MANY_SPLIT_CASES))])
def test_matrix_core_long_contexts_many_splits(case):
    """Long contexts cut into 2 .. 32 splits per (sequence, KV head), ragged units,
    16-position (INT8) and 32-position tiles, window rings, sinks, recent fp16 rows and
    the fused append: every position attended exactly once across the splits."""
    fmt, gk, G, lens, ns, W, cap, S, R, fused = case
    B, Hkv, D = len(lens), 2, 128
    L = max(lens)
    C = cap or L
    k = synth.kv_source((B, Hkv, L, D), 1700 + L + ns, DEV, outlier_channels=3)
    v = synth.kv_source((B, Hkv, L, D), 1800 + L + ns, DEV, outlier_channels=3)
    q = synth.query((B, Hkv * G, D), 1900 + L + ns, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, C, gk, 128, sinks=S, recent=R)
    dc = kvq.DeviceCache(desc, DEV)
    P = L - 1 if fused else L        # positions written before the call
    if S:
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :S].contiguous(), v[:, :, :S].contiguous(), 0, S)
    first = max(S, P - (C - S))      # the rows the ring still holds
    for start in range(first, P, C - S):
        n = min(C - S, P - start)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, start:start + n].contiguous(),
                                 v[:, :, start:start + n].contiguous(), start, n)
    # a shorter sequence's own window: its last rows back into its ring (see fused tests)
    one = kvq.make_desc(fmt, 1, Hkv, D, C, gk, 128, sinks=S, recent=R)
    for b, ln in enumerate(lens):
        end = ln - 1 if fused else ln
        lo = max(S, end - (C - S))
        if ln < L and C < L and end > lo:
            sub = kvq.kvq_cache(*[t.view(B, -1)[b].data_ptr() for t in
                                  (dc.k_codes, dc.k_scales, dc.v_codes, dc.v_scales)],
                                *([t.view(B, -1)[b].data_ptr() for t in (dc.k_recent, dc.v_recent)]
                                  if R else []))
            kvq.kvq_quantize_prefill(one, sub, k[b:b + 1, :, lo:end].contiguous(),
                                     v[b:b + 1, :, lo:end].contiguous(), lo, end - lo)
    if fused:
        idx = torch.tensor([ln - 1 for ln in lens], device=DEV)
        ar = torch.arange(B, device=DEV)
        out = append_decode(desc, dc, k[ar, :, idx].contiguous(), v[ar, :, idx].contiguous(), q,
                            Hkv * G, lens, W, 0.0, ns)
    else:
        out = decode(desc, dc, q, Hkv * G, lens, W, 0.0, ns)
    kh, vh = _oracle_hat(fmt, np16(k), np16(v), gk, 128)
    if R:
        kh = attention.recent_fp16_rows(kh, np16(k), lens, R)
        vh = attention.recent_fp16_rows(vh, np16(v), lens, R)
    ref = attention.decode_attention(np16(q), kh, vh, lens, W, sinks=S)
    assert_attn_close(out.cpu().numpy(), ref, f"splits {case}")


@pytest.mark.parametrize("fmt", ["int4", "codec"])
def test_maximum_units_fused_step(fmt):
    """The largest call the library takes: 256 sequences (KVQ_MAX_BATCH) x 64 KV heads =
    16384 (sequence, KV head) units, one split counter each in the workspace, with ragged
    lengths 1 .. 48 (lengths 1 and 2 included), GQA 2, the fused append + decode step;
    every unit against the oracle."""
    B, Hkv, G, D, C = 256, 64, 2, 128, 48
    lens = [1 + (b * 7) % C for b in range(B)]
    lens[0], lens[1] = 1, 2
    k = synth.kv_source((B, Hkv, C, D), 5100, DEV, outlier_channels=2)
    v = synth.kv_source((B, Hkv, C, D), 5101, DEV)
    q = synth.query((B, Hkv * G, D), 5102, DEV)
    desc = kvq.make_desc(fmt, B, Hkv, D, C)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, C)   # every slot; each sequence attends its own lens
    idx = torch.tensor([ln - 1 for ln in lens], device=DEV)
    ar = torch.arange(B, device=DEV)
    kn, vn = k[ar, :, idx].contiguous(), v[ar, :, idx].contiguous()
    out = append_decode(desc, dc, kn, vn, q, Hkv * G, lens)
    if fmt == "codec":
        kh, vh, _ = codec_hat_from_device(dc, fmt, np16(k), np16(v), lens)
    else:
        kh, vh = _oracle_hat(fmt, np16(k), np16(v))
    ref = attention.decode_attention(np16(q), kh, vh, lens)
    assert_attn_close(out.cpu().numpy(), ref, f"{fmt} at 16384 units")
