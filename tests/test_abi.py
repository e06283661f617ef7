"""Host-side tests of the C ABI (no GPU work): exports, size queries, validation errors,
the library's codebook against the oracle's, and an exhaustive check of the quantizers'
scalar arithmetic compiled for the host."""
import os
import re
import subprocess

import numpy as np
import pytest

import int4_quantized_kv_amd as kvq
from oracle import codec, memory

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 17
    assert sorted(kvq.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    for n in names:
        assert n in exported, n
    assert kvq.kvq_version() == 8


def test_status_strings():
    assert kvq.status_str(0) == "ok"
    assert kvq.status_str(-4) == "workspace too small"
    assert kvq.status_str(12345) == "unknown status"


def test_size_queries_match_closed_forms():
    for fmt in ("int4", "int8", "codec", "codec3", "int4h"):
        for (B, H, D, C, gk, gv) in [(8, 8, 128, 8193, 64, 128), (1, 4, 256, 1024, 64, 128),
                                     (3, 2, 64, 17, 32, 64)]:
            d = kvq.make_desc(fmt, B, H, D, C, gk, gv)
            assert kvq.kvq_check_desc(d) == 0
            if fmt in ("int4", "int4h"):
                sb = 4 if fmt == "int4" else 2
                assert kvq.kvq_codes_bytes(d, 0) + kvq.kvq_scales_bytes(d, 0) == \
                    memory.int4_cache_bytes(B, H, C, D, gk, scale_bytes=sb)
                assert kvq.kvq_codes_bytes(d, 1) + kvq.kvq_scales_bytes(d, 1) == \
                    memory.int4_cache_bytes(B, H, C, D, gv, scale_bytes=sb)
            elif fmt == "int8":
                assert kvq.kvq_codes_bytes(d, 0) == B * H * C * D
                assert kvq.kvq_scales_bytes(d, 1) == B * H * C * 4
            elif fmt == "codec":
                assert kvq.kvq_codes_bytes(d, 1) == B * H * C * D // 2
                assert kvq.kvq_scales_bytes(d, 0) == B * H * C * 4
            else:                                   # 3-bit indices packed: 3D/8 bytes
                assert kvq.kvq_codes_bytes(d, 1) == B * H * C * 3 * D // 8
                assert kvq.kvq_scales_bytes(d, 0) == B * H * C * 4
            assert kvq.kvq_codes_bytes(d, 2) == 0
    # effective bits with fp32 scales: K (g=64) 4.5 bits, V (g=128) 4.25 bits per element
    d = kvq.make_desc("int4", 1, 1, 128, 1000)
    kb = (kvq.kvq_codes_bytes(d, 0) + kvq.kvq_scales_bytes(d, 0)) * 8 / (1000 * 128)
    vb = (kvq.kvq_codes_bytes(d, 1) + kvq.kvq_scales_bytes(d, 1)) * 8 / (1000 * 128)
    assert kb == memory.effective_bits(64, scale_bits=32) == 4.5
    assert vb == memory.effective_bits(128, scale_bits=32) == 4.25


@pytest.mark.parametrize("fields,status", [
    (dict(format=7), kvq.KVQ_ERR_ARG),
    (dict(batch=0), kvq.KVQ_ERR_ARG),
    (dict(batch=257), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(head_dim=96), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(group_k=48), kvq.KVQ_ERR_UNSUPPORTED),     # not a power of two / D % g != 0
    (dict(group_k=16), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(group_v=256), kvq.KVQ_ERR_UNSUPPORTED),    # g > D
    (dict(capacity=0), kvq.KVQ_ERR_ARG),
    (dict(kv_heads=-1), kvq.KVQ_ERR_ARG),
    (dict(sinks=-1), kvq.KVQ_ERR_ARG),
    (dict(sinks=64), kvq.KVQ_ERR_ARG),                # no ring slot left
])
def test_descriptor_validation(fields, status):
    base = dict(format=0, batch=2, kv_heads=4, head_dim=128, capacity=64, group_k=64,
                group_v=128, sinks=0)
    base.update(fields)
    d = kvq.kvq_cache_desc(*[base[k] for k in ("format", "batch", "kv_heads", "head_dim",
                                               "capacity", "group_k", "group_v", "sinks")])
    assert kvq.kvq_check_desc(d) == status
    assert kvq.kvq_codes_bytes(d, 0) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation before any launch


def _cache():
    return kvq.kvq_cache(FAKE, FAKE, FAKE, FAKE)


def _expect(status, fn, *args):
    with pytest.raises(kvq.KvqError) as e:
        fn(*args)
    assert e.value.status == status


def test_error_paths_enqueue_nothing():
    d = kvq.make_desc("int4", 2, 4, 128, 64)
    c = _cache()
    # prefill: n > capacity, n < 1, negative start, null source
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_quantize_prefill, d, c, FAKE, FAKE, 0, 65, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, d, c, FAKE, FAKE, 0, 0, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, d, c, FAKE, FAKE, -1, 4, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, d, c, 0, FAKE, 0, 4, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, d, kvq.kvq_cache(FAKE, 0, FAKE, FAKE),
            FAKE, FAKE, 0, 4, 0)
    # append: negative position
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_append, d, c, FAKE, FAKE, [3, -1], 0)
    # decode: Hq % Hkv, unsupported group, len 0, len > capacity without window,
    # window > capacity with len > capacity, too-small / missing workspace
    ws = kvq.kvq_decode_workspace_bytes(d, 8, 64)
    assert ws == kvq.KVQ_WS_COUNTER_BYTES + 2 * 8 * kvq.kvq_plan_splits(d, 8, 64) * 130 * 4
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, d, c, FAKE, 6, [10, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_decode_attn, d, c, FAKE, 64, [10, 10], 0, 0.0, 0, FAKE, FAKE, 1 << 30, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, d, c, FAKE, 8, [10, 0], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_decode_attn, d, c, FAKE, 8, [65, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_decode_attn, d, c, FAKE, 8, [100, 10], 65, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_WORKSPACE, kvq.kvq_decode_attn, d, c, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, FAKE, ws - 1, 0)
    _expect(kvq.KVQ_ERR_WORKSPACE, kvq.kvq_decode_attn, d, c, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, 0, ws, 0)
    # more (sequence, KV head) units than the workspace's 16384 split counters
    big = kvq.make_desc("int4", 256, 65, 128, 64)
    _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_decode_attn, big, c, FAKE, 65, [10] * 256, 0, 0.0, 0, FAKE, FAKE,
            1 << 30, 0)
    _expect(kvq.KVQ_ERR_WORKSPACE, kvq.kvq_decode_attn, d, c, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, FAKE + 8, ws, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, d, c, FAKE, 8, [64, 10], -1, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, d, c, FAKE, 8, [64, 10], 0, float("nan"), 0, FAKE, FAKE, ws, 0)
    # fused append + decode: null new rows, then the decode checks
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_append_decode_attn, d, c, 0, FAKE, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_append_decode_attn, d, c, FAKE, 0, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_append_decode_attn, d, c, FAKE, FAKE, FAKE, 8, [65, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_WORKSPACE, kvq.kvq_append_decode_attn, d, c, FAKE, FAKE, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, FAKE, ws - 1, 0)
    # the no-allocation step: the same checks, and calls whose counters and partials
    # exceed the library's scratch array are rejected before anything is enqueued
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_append_decode_attn_noalloc, d, c, 0, FAKE, FAKE, 8, [64, 10], 0, 0.0, 0, FAKE, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_append_decode_attn_noalloc, d, c, FAKE, FAKE, FAKE, 8, [65, 10], 0, 0.0, 0, FAKE, 0)
    wide = kvq.make_desc("int4", 64, 8, 128, 64)
    need = kvq.kvq_decode_workspace_bytes(wide, 64, 64, 0, 8)
    assert need > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    _expect(kvq.KVQ_ERR_WORKSPACE, kvq.kvq_append_decode_attn_noalloc, wide, c, FAKE, FAKE, FAKE, 64, [64] * 64, 0, 0.0, 8, FAKE, 0)
    # the split counters bound batch * kv_heads
    big = kvq.make_desc("int4", 256, 128, 128, 64)
    _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_decode_attn, big, c, FAKE, 128, [10] * 256, 0, 0.0, 1, FAKE, FAKE, 1 << 40, 0)
    # dequant: bad kv selector, n > capacity
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_dequant, d, c, 2, 0, 4, FAKE, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_dequant, d, c, 0, 0, 65, FAKE, 0)
    # an invalid descriptor is reported by every call
    bad = kvq.make_desc("codec", 2, 4, 96, 64)
    _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_quantize_prefill, bad, c, FAKE, FAKE, 0, 4, 0)
    _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_dequant, bad, c, 0, 0, 4, FAKE, 0)


def test_sinks_validation_and_workspace():
    """A cache of 20 slots with 4 sink slots: a ring of 16.  Writes of more ring positions
    than ring slots, and windows longer than the ring over a wrapped cache, are
    rejected; the workspace covers the window plus the sinks."""
    d = kvq.make_desc("int4", 2, 4, 128, 20, sinks=4)
    assert kvq.kvq_check_desc(d) == 0
    assert kvq.kvq_check_desc(kvq.make_desc("int4", 2, 4, 128, 20, sinks=19)) == 0
    c = _cache()
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_quantize_prefill, d, c, FAKE, FAKE, 0, 21, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_quantize_prefill, d, c, FAKE, FAKE, 10, 17, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_dequant, d, c, 0, 2, 19, FAKE, 0)   # ring part 17
    ws = kvq.kvq_decode_workspace_bytes(d, 8, 100, 10)
    span = 10 + 4
    assert ws == kvq.KVQ_WS_COUNTER_BYTES + 2 * 8 * kvq.kvq_plan_splits(d, 8, span) * 130 * 4
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_decode_attn, d, c, FAKE, 8, [30, 10], 17, 0.0, 0, FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_decode_attn, d, c, FAKE, 8, [30, 10], 0, 0.0, 0, FAKE, FAKE, ws, 0)


def test_recent_validation_and_workspace():
    """Recent fp16 rows: INT4 only, not with sinks, at most KVQ_MAX_RECENT; the rings are
    required when R > 0; decode needs the matrix-core INT4 kernel; the workspace is the
    splits' alone."""
    ok = kvq.make_desc("int4", 2, 4, 128, 64, recent=128)
    assert kvq.kvq_check_desc(ok) == 0
    assert kvq.kvq_recent_bytes(ok) == 2 * 4 * 128 * 128 * 2
    assert kvq.kvq_recent_bytes(kvq.make_desc("int4", 2, 4, 128, 64)) == 0
    assert kvq.kvq_check_desc(kvq.make_desc("int4", 2, 4, 128, 64, recent=-1)) == kvq.KVQ_ERR_ARG
    for bad in (kvq.make_desc("int4", 2, 4, 128, 64, recent=kvq.KVQ_MAX_RECENT + 1),
                kvq.make_desc("int8", 2, 4, 128, 64, recent=16),
                kvq.make_desc("codec", 2, 4, 128, 64, recent=16),
                kvq.make_desc("int4", 2, 4, 128, 64, sinks=4, recent=16)):
        assert kvq.kvq_check_desc(bad) == kvq.KVQ_ERR_UNSUPPORTED
        assert kvq.kvq_recent_bytes(bad) == 0
    assert kvq.kvq_check_desc(kvq.make_desc("int4", 2, 4, 128, 64, recent=kvq.KVQ_MAX_RECENT)) == 0
    for R in (1, 128, 1024):
        d = kvq.make_desc("int4", 2, 4, 128, 64, recent=R)
        ns = kvq.kvq_plan_splits(d, 8, 60)
        assert kvq.kvq_decode_workspace_bytes(d, 8, 60, 0) == kvq.KVQ_WS_COUNTER_BYTES + 2 * 8 * ns * 130 * 4
        assert kvq.kvq_decode_workspace_bytes(d, 8, 60, 0, 7) == kvq.KVQ_WS_COUNTER_BYTES + 2 * 8 * 7 * 130 * 4
    no_rings = _cache()
    rings = kvq.kvq_cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, ok, no_rings, FAKE, FAKE, 0, 10, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_append, ok, no_rings, FAKE, FAKE, [3, 4], 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, ok, no_rings, FAKE, 8, [30, 10], 0, 0.0, 0, FAKE, FAKE, 1 << 30, 0)
    # shapes the matrix-core kernel does not take
    for d, hq in ((kvq.make_desc("int4", 2, 4, 64, 64, 32, 64, recent=16), 8),
                  (kvq.make_desc("int4", 2, 4, 128, 64, 64, 64, recent=16), 8),
                  (kvq.make_desc("int4", 2, 4, 128, 64, 32, 128, recent=16), 32)):
        _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_decode_attn, d, rings, FAKE, hq, [30, 10], 0, 0.0, 0, FAKE,
                FAKE, 1 << 30, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_decode_attn, ok, rings, FAKE, 8, [30, 10], 0, 0.0, 1025, FAKE, FAKE,
            1 << 30, 0)


def test_split_plan():
    d2 = kvq.make_desc("int4", 8, 8, 128, 8193)
    n2 = kvq.kvq_plan_splits(d2, 32, 8193)
    assert 1 <= n2 <= 64
    d5 = kvq.make_desc("int4", 1, 8, 128, 131072)
    # only 8 natural (batch, kv head) units: the splits must give every one of the 256
    # CUs a workgroup
    assert 8 * kvq.kvq_plan_splits(d5, 32, 131072) >= 256
    assert kvq.kvq_plan_splits(d5, 32, 1) == 1
    assert kvq.kvq_plan_splits(d5, 31, 100) == 0


def test_library_codebook_matches_oracle():
    lv, th = kvq.kvq_codec_codebook()
    c, t, _ = codec.codebook(4)
    assert np.allclose(lv, c, atol=1e-6) and np.allclose(th, t, atol=1e-6)
    assert th[7] == 0.0 and lv[7] == -lv[8]
    assert kvq.kvq_codec_codebook_bits(4) == (lv, th)
    lv3, th3 = kvq.kvq_codec_codebook_bits(3)
    c3, t3, _ = codec.codebook(3)
    assert len(lv3) == 8 and len(th3) == 7
    assert np.allclose(lv3, c3, atol=1e-6) and np.allclose(th3, t3, atol=1e-6)
    assert th3[3] == 0.0 and lv3[3] == -lv3[4] and np.all(np.diff(th3) > 0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_codec_codebook_bits(2)
    # the kernels code a value by binary search over the thresholds: they must ascend
    assert np.all(np.diff(th) > 0)


@pytest.mark.parametrize("rule", ["int4", "int8"])
def test_quantizer_arithmetic_exhaustive_on_host(tmp_path, rule):
    exe = tmp_path / "arith_exhaustive"
    src = os.path.join(ROOT, "tests", "host", "arith_exhaustive.c")
    inc = os.path.join(ROOT, "int4_quantized_kv_amd", "csrc")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-I", inc, src, "-o", str(exe),
                    "-lm"], check=True)
    r = subprocess.run([str(exe), rule], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "quotient_mismatches=0" in r.stdout and "scale_mismatches=0" in r.stdout
    assert "code_mismatches=0" in r.stdout


def test_paged_validation_and_sizes():
    """Paged layout (bxzpzcl.cn/news/2871434 section 3.1 pages; section 4 sizes): page
    sizes 16 .. 256 (powers of two), capacity a multiple of the page, no sinks or recent
    rows; buffers sized by the pool; positions beyond the capacity rejected."""
    ok = kvq.make_desc("int4", 2, 8, 128, 1024, page_size=16, num_pages=100)
    assert kvq.kvq_check_desc(ok) == kvq.KVQ_OK
    assert kvq.kvq_codes_bytes(ok, 0) == 100 * 8 * 16 * 64
    assert kvq.kvq_scales_bytes(ok, 0) == 100 * 8 * 16 * 2 * 4
    assert kvq.kvq_scales_bytes(ok, 1) == 100 * 8 * 16 * 1 * 4
    i8 = kvq.make_desc("int8", 2, 8, 128, 1024, page_size=64, num_pages=7)
    assert kvq.kvq_codes_bytes(i8, 1) == 7 * 8 * 64 * 128
    for fields, status in [
        (dict(page_size=8, num_pages=10), kvq.KVQ_ERR_UNSUPPORTED),      # below 16
        (dict(page_size=48, num_pages=10), kvq.KVQ_ERR_UNSUPPORTED),     # not a power of two
        (dict(page_size=512, num_pages=10), kvq.KVQ_ERR_UNSUPPORTED),    # above 256
        (dict(page_size=16, num_pages=0), kvq.KVQ_ERR_ARG),              # empty pool
        (dict(page_size=-16, num_pages=10), kvq.KVQ_ERR_ARG),
        (dict(page_size=16, num_pages=10, sinks=4), kvq.KVQ_ERR_UNSUPPORTED),
        (dict(page_size=16, num_pages=10, recent=16), kvq.KVQ_ERR_UNSUPPORTED),
    ]:
        d = kvq.make_desc("int4", 2, 8, 128, 1024, **fields)
        assert kvq.kvq_check_desc(d) == status, fields
    odd = kvq.make_desc("int4", 2, 8, 128, 1000, page_size=16, num_pages=10)   # C % P != 0
    assert kvq.kvq_check_desc(odd) == kvq.KVQ_ERR_UNSUPPORTED
    c = kvq.kvq_cache(FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE)
    no_table = kvq.kvq_cache(FAKE, FAKE, FAKE, FAKE)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_quantize_prefill, ok, no_table, FAKE, FAKE, 0, 4, 0)
    # no ring: positions at or past the capacity are rejected, windowed or not
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_quantize_prefill, ok, c, FAKE, FAKE, 1000, 25, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_append, ok, c, FAKE, FAKE, [1024, 3], 0)
    ws = kvq.kvq_decode_workspace_bytes(ok, 32, 1024)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_decode_attn, ok, c, FAKE, 32, [1025, 10], 512, 0.0, 0,
            FAKE, FAKE, ws, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_dequant, ok, c, 0, 1020, 5, FAKE, 0)


def test_prefill_attn_validation():
    """kvq_prefill_attn: INT4 (fp32 or fp16 scales) with head_dim 128, V group 128 and K
    group 64 or 128 only; chunk within each sequence; a ring must hold the chunk's window."""
    d = kvq.make_desc("int4", 2, 8, 128, 4096)
    c = _cache()
    out = FAKE
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_prefill_attn, d, c, FAKE, 32, 0, [100, 100], 0, 0.0, out, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_prefill_attn, d, c, FAKE, 32, 200, [100, 300], 0, 0.0, out, 0)
    _expect(kvq.KVQ_ERR_ARG, kvq.kvq_prefill_attn, d, c, FAKE, 30, 16, [100, 300], 0, 0.0, out, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_prefill_attn, d, c, FAKE, 32, 16, [5000, 300], 0, 0.0, out, 0)
    _expect(kvq.KVQ_ERR_CAPACITY, kvq.kvq_prefill_attn, d, c, FAKE, 32, 16, [5000, 300], 4090, 0.0, out, 0)
    for bad in (kvq.make_desc("int8", 2, 8, 128, 4096), kvq.make_desc("int4", 2, 8, 64, 4096),
                kvq.make_desc("int4", 2, 8, 128, 4096, 32, 128), kvq.make_desc("int4", 2, 8, 128, 4096, 64, 64),
                kvq.make_desc("codec", 2, 8, 128, 4096), kvq.make_desc("int4h", 2, 8, 128, 4096, 32, 128),
                kvq.make_desc("codec3", 2, 8, 128, 4096)):
        _expect(kvq.KVQ_ERR_UNSUPPORTED, kvq.kvq_prefill_attn, bad, c, FAKE, 32, 16, [100, 100], 0, 0.0, out, 0)
