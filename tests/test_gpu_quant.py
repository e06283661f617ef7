"""GPU parity of quantize-append, bulk prefill quantize and dequantize against the oracle.

Bar: INT4 / INT8 codes and fp32 scales bit-exact (round-half-to-even), dequantized
values bit-exact (fl32(q * s)).  INT4 rule: lpnh.cn/news/2042373 §2.1; INT8 rule:
bxzpzcl.cn/news/2871434 §3.1.
"""
import numpy as np
import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from oracle import quant
from tests.kvq_testutil import cache_arrays, np16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _expect_int4(k16, v16, gk, gv):
    qk, sk = quant.quantize_int4(k16, gk)
    qv, sv = quant.quantize_int4(v16, gv)
    return quant.pack_nibbles(qk), sk, quant.pack_nibbles(qv), sv


def _expect_int8(k16, v16):
    qk, sk = quant.quantize_int8(k16)
    qv, sv = quant.quantize_int8(v16)
    return qk, sk[..., None], qv, sv[..., None]


def _prefill(fmt, k, v, cap=None, gk=64, gv=128, start=0):
    B, H, S, D = k.shape
    desc = kvq.make_desc(fmt, B, H, D, cap or S, gk, gv)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, start, S)
    return desc, dc


def _assert_cache(got, exp, rows=None):
    names = ("k_codes", "k_scales", "v_codes", "v_scales")
    for name, g, e in zip(names, got, exp):
        if rows is not None:
            g = g[:, :, rows]
        assert g.shape == e.shape, (name, g.shape, e.shape)
        if not np.array_equal(g, e):
            bad = np.argwhere(g != e)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[0].tolist()}")


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_tiny_workload_prefill_bit_exact(fmt):
    w = synth.WORKLOADS[1]
    k, v, _, _, _ = synth.layer_inputs(w, 0, DEV)
    desc, dc = _prefill(fmt, k, v)
    got = cache_arrays(dc, fmt)
    exp = _expect_int4(np16(k), np16(v), 64, 128) if fmt == "int4" else _expect_int8(np16(k), np16(v))
    _assert_cache(got, exp)
    if fmt == "int4":   # the zeroed V row (one g=128 group) has scale 1 and zero codes
        assert got[3][0, 1, 37, 0] == 1.0 and not got[2][0, 1, 37].any()


@pytest.mark.parametrize("gk,gv,D", [(64, 128, 128), (32, 64, 64), (128, 256, 256), (32, 32, 128)])
def test_group_sizes_and_head_dims(gk, gv, D):
    k = synth.kv_source((2, 3, 77, D), 11, DEV, outlier_channels=3)
    v = synth.kv_source((2, 3, 77, D), 12, DEV, outlier_channels=2, zero_groups=((1, 2, 5, 0, D),))
    desc, dc = _prefill("int4", k, v, gk=gk, gv=gv)
    _assert_cache(cache_arrays(dc, "int4"), _expect_int4(np16(k), np16(v), gk, gv))


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_exhaustive_fp16_sweep(fmt):
    """Every finite fp16 value x in groups whose amax is a spread of fp16 values: codes
    and scales bit-exact against the oracle."""
    allh = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    fin = allh[np.isfinite(allh)]
    pos = fin[fin > 0]
    rng = np.random.default_rng(11)
    amaxes = np.concatenate([pos[[0, 1, 100, 1023, 1024, 5000, 15000, 15360, 20000, 30000, -1]],
                             rng.choice(pos, 21, replace=False)])
    rows = []
    for a in amaxes:
        xs = fin[np.abs(fin.astype(np.float64)) <= float(a)]
        n = -(-len(xs) // 63) * 63
        pad = np.zeros(n, np.float16)
        pad[:len(xs)] = xs
        r = np.empty((n // 63, 64), np.float16)
        r[:, 0] = a
        r[:, 1:] = pad.reshape(-1, 63)
        rows.append(r)
    rows = np.concatenate(rows)
    rows = rows[: len(rows) // 2 * 2].reshape(1, 1, -1, 128)   # two 64-groups per row
    k = torch.from_numpy(rows.copy()).to(DEV)
    v = torch.from_numpy(rows[:, :, ::-1].copy()).to(DEV)
    desc, dc = _prefill(fmt, k, v)
    exp = _expect_int4(np16(k), np16(v), 64, 128) if fmt == "int4" else _expect_int8(np16(k), np16(v))
    _assert_cache(cache_arrays(dc, fmt), exp)


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_append_one_by_one_equals_prefill_and_ring(fmt):
    B, H, S, D = 3, 2, 40, 128
    k = synth.kv_source((B, H, S, D), 21, DEV, outlier_channels=3)
    v = synth.kv_source((B, H, S, D), 22, DEV, outlier_channels=3)
    desc, dc_pre = _prefill(fmt, k, v)
    dc_app = kvq.DeviceCache(desc, DEV)
    for t in range(S):
        kvq.kvq_append(desc, dc_app.c, k[:, :, t].contiguous(), v[:, :, t].contiguous(), [t] * B)
    a, p = cache_arrays(dc_app, fmt), cache_arrays(dc_pre, fmt)
    for x, y in zip(a, p):
        assert np.array_equal(x, y)
    # ring: capacity 16, per-sequence positions differ; slot = pos % 16 holds the last write
    ring = kvq.make_desc(fmt, B, H, D, 16)
    dr = kvq.DeviceCache(ring, DEV)
    ends = [40, 33, 17]
    for t in range(S):
        pos = [min(t, e - 1) for e in ends]
        kk = torch.stack([k[b, :, pos[b]] for b in range(B)]).contiguous()
        vv = torch.stack([v[b, :, pos[b]] for b in range(B)]).contiguous()
        kvq.kvq_append(ring, dr.c, kk, vv, pos)
    got = cache_arrays(dr, fmt)
    full = _expect_int4(np16(k), np16(v), 64, 128) if fmt == "int4" else _expect_int8(np16(k), np16(v))
    for b, e in enumerate(ends):
        for p in range(e - 16, e):
            for gi, fi in zip(got, full):
                assert np.array_equal(gi[b, :, p % 16], fi[b, :, p])


def test_prefill_into_ring_offset():
    """Prefill of positions [start, start + n) into a smaller ring lands at pos % C."""
    B, H, D = 2, 2, 128
    k = synth.kv_source((B, H, 24, D), 31, DEV)
    v = synth.kv_source((B, H, 24, D), 32, DEV)
    desc = kvq.make_desc("int4", B, H, D, 32)
    dc = kvq.DeviceCache(desc, DEV)
    kvq.kvq_quantize_prefill(desc, dc.c, k, v, 20, 24)     # positions 20..43 -> slots 20..31, 0..11
    got = cache_arrays(dc, "int4")
    exp = _expect_int4(np16(k), np16(v), 64, 128)
    slots = [(20 + t) % 32 for t in range(24)]
    for gi, ei in zip(got, exp):
        assert np.array_equal(gi[:, :, slots], ei)


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_dequant_bit_exact(fmt):
    B, H, S, D = 2, 3, 50, 128
    k = synth.kv_source((B, H, S, D), 41, DEV, outlier_channels=3)
    v = synth.kv_source((B, H, S, D), 42, DEV, outlier_channels=3)
    desc, dc = _prefill(fmt, k, v)
    for kv, src, g in ((0, k, 64), (1, v, 128)):
        out = torch.empty((B, H, 13, D), dtype=torch.float32, device=DEV)
        kvq.kvq_dequant(desc, dc.c, kv, 7, 13, out)
        torch.cuda.synchronize()
        x = np16(src)[:, :, 7:20]
        if fmt == "int4":
            q, s = quant.quantize_int4(x, g)
            exp = quant.dequantize_int4(q, s, g)
        else:
            q, s = quant.quantize_int8(x)
            exp = quant.dequantize_int8(q, s)
        assert np.array_equal(out.cpu().numpy(), exp)


def test_deterministic_repeat():
    w = synth.WORKLOADS[1]
    k, v, _, _, _ = synth.layer_inputs(w, 0, DEV)
    _, a = _prefill("int4", k, v)
    _, b = _prefill("int4", k, v)
    for x, y in zip(cache_arrays(a, "int4"), cache_arrays(b, "int4")):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("wid", [2, 3])
def test_full_size_layer_prefill(wid):
    """One layer of the Llama-3-8B-shaped (8K x 8) and the MHA-7B-shaped (20K x 8)
    workloads at full size, quantized in one launch.  Quantization is row-local, so the
    oracle checks every position of sampled (batch, kv head) pairs: all of them for the
    8K workload, the four corner pairs for the 20K one."""
    w = synth.WORKLOADS[wid]
    layer = w.layers - 1
    k, v, _, _, _ = synth.layer_inputs(w, layer, DEV)
    desc, dc = _prefill("int4", k, v, cap=w.context + 1)
    got = cache_arrays(dc, "int4")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)] if wid == 2 else \
        [(0, 0), (0, w.kv_heads - 1), (w.batch - 1, 0), (w.batch - 1, w.kv_heads - 1)]
    bs = sorted({b for b, _ in pairs})
    hs = sorted({h for _, h in pairs})
    kn = k[bs][:, hs].cpu().numpy()
    vn = v[bs][:, hs].cpu().numpy()
    del k, v
    exp = _expect_int4(kn, vn, 64, 128)
    sub = [g[bs][:, hs] for g in got]
    _assert_cache(sub, exp, rows=slice(0, w.context))
