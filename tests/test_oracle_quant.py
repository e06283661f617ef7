"""Pins of oracle/quant.py against what the pages and the arithmetic fix (CPU only).

The INT4 rule ([KV-4bit] lpnh.cn/news/2042373 §2.1): per group of g head_dim
elements, s = amax/7 (1 for an all-zero group), q = clamp(round(x/s), -7, 7), with
round-half-to-even and fp32 scales.  The INT8 rule ([KV-opt] bxzpzcl.cn/news/2871434
§3.1): per (token, head), s = max(amax/127, 1e-8), q = clamp(round(x/s), -128, 127).
"""
import numpy as np
import pytest

from oracle import memory, quant
import torch

F16_ALL = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
F16_FINITE = F16_ALL[np.isfinite(F16_ALL)]


def _fp64_route_int4(x16, g):
    """Same definition in fp64 then one rounding to fp32.  Division is one of the
    operations for which rounding through a format with >= 2p+2 bits first is
    innocuous (53 >= 2*24 + 2), so fl32(fl64(a/b)) == fl32(a/b) exactly."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    D = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (D // g, g))
    a = np.abs(xg).max(-1)
    s = np.float32(a / 7.0) if np.ndim(a) == 0 else (a / 7.0).astype(np.float32)
    s = np.where(s == 0, np.float32(1), s).astype(np.float32)
    y = (xg / s.astype(np.float64)[..., None]).astype(np.float32)
    q = np.clip(np.rint(y.astype(np.float64)), -7, 7).astype(np.int8)
    return q.reshape(x.shape), s


def test_hand_example_groups_along_head_dim():
    # One row, D = 128, g = 64: the first 64 elements hold 7 and 3.5, the next 64 hold 14.
    x = np.zeros((1, 128), np.float16)
    x[0, 0] = 7.0
    x[0, 1] = 3.5        # 3.5 / 1 -> tie -> 4 (even)
    x[0, 2] = -0.5       # tie -> 0
    x[0, 64] = 14.0
    x[0, 65] = 3.0       # 3 / 2 = 1.5 -> tie -> 2
    x[0, 66] = -5.0      # -2.5 -> -2
    q, s = quant.quantize_int4(x, 64)
    assert s.dtype == np.float32 and s.shape == (1, 2)
    assert s[0, 0] == np.float32(1.0) and s[0, 1] == np.float32(2.0)
    assert list(q[0, :3]) == [7, 4, 0]
    assert list(q[0, 64:67]) == [7, 2, -2]
    assert not q[0, 3:64].any() and not q[0, 67:].any()
    # With g = 128 the whole row is one group: s = 14/7 = 2.
    q2, s2 = quant.quantize_int4(x, 128)
    assert s2.shape == (1, 1) and s2[0, 0] == np.float32(2.0)
    assert list(q2[0, :3]) == [4, 2, 0]   # 7/2=3.5->4, 3.5/2=1.75->2, -0.25->0


@pytest.mark.parametrize("v,expect", [(0.5, 0), (1.5, 2), (2.5, 2), (3.5, 4), (4.5, 4),
                                      (5.5, 6), (6.5, 6), (0.49951171875, 0), (1.4990234375, 1)])
def test_ties_round_half_to_even(v, expect):
    # amax 7 -> s = 1 exactly, so x / s = x and only the integer rounding acts.
    x = np.zeros((64,), np.float16)
    x[0] = 7.0
    x[1] = v
    x[2] = -v
    q, s = quant.quantize_int4(x, 64)
    assert s[0] == 1.0
    assert q[1] == expect and q[2] == -expect


def test_zero_group_gets_scale_one():
    x = np.zeros((3, 128), np.float16)
    x[1, 70] = 2.0
    q, s = quant.quantize_int4(x, 64)
    assert np.all(s[0] == 1.0) and np.all(s[2] == 1.0) and s[1, 0] == 1.0
    assert s[1, 1] == np.float32(2.0) / np.float32(7.0)
    assert not q[0].any() and not q[2].any()


def _rand_rows(rng, n, D, outliers=True):
    x = rng.standard_normal((n, D)).astype(np.float32)
    if outliers:
        x[:, rng.choice(D, 3, replace=False)] *= 20
    return x.astype(np.float16)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_invariants_random(g):
    rng = np.random.default_rng(7)
    x = _rand_rows(rng, 2000, 128)
    q, s = quant.quantize_int4(x, g)
    xg = x.astype(np.float64).reshape(2000, 128 // g, g)
    qg = q.astype(np.float64).reshape(2000, 128 // g, g)
    sg = s.astype(np.float64)[..., None]
    # |x - q s| <= s (1/2 + 2^-21): rounding to an integer plus one fp32 rounding of x/s
    assert np.all(np.abs(xg - qg * sg) <= sg * (0.5 + 2.0 ** -21))
    # the amax element of every non-zero group maps to +-7, and codes stay in [-7, 7]
    am = np.abs(xg).argmax(-1)
    top = np.take_along_axis(qg, am[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 7)
    assert q.min() >= -7 and q.max() <= 7
    # odd symmetry
    qn, sn = quant.quantize_int4(-x, g)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # same as the fp64 route (double rounding through fp64 is innocuous for division)
    q64, s64 = _fp64_route_int4(x, g)
    assert np.array_equal(q, q64) and np.array_equal(s, s64)


def test_exhaustive_fp16_sweep():
    """Every finite fp16 value x, inside groups whose amax is a spread of fp16 values."""
    pos = F16_FINITE[(F16_FINITE > 0)]
    rng = np.random.default_rng(11)
    amaxes = np.concatenate([pos[[0, 1, 100, 1023, 1024, 5000, 15000, 15360, 20000, 30000, -1]],
                             rng.choice(pos, 40, replace=False)]).astype(np.float16)
    for a in amaxes:
        xs = F16_FINITE[np.abs(F16_FINITE.astype(np.float64)) <= float(a)]
        n = -(-len(xs) // 63) * 63
        pad = np.zeros(n, np.float16)
        pad[:len(xs)] = xs
        rows = np.empty((n // 63, 64), np.float16)
        rows[:, 0] = a
        rows[:, 1:] = pad.reshape(-1, 63)
        q, s = quant.quantize_int4(rows, 64)
        assert np.all(s == (np.float32(a) / np.float32(7.0)))
        q64, s64 = _fp64_route_int4(rows, 64)
        assert np.array_equal(q, q64)
        xr = rows.astype(np.float64)
        assert np.all(np.abs(xr - q * s.astype(np.float64)) <= s.astype(np.float64) * (0.5 + 2.0 ** -21))


def test_pack_layout():
    codes = np.array([1, -1, -7, 7, 0, -8, 3, 4], np.int8)
    p = quant.pack_nibbles(codes)
    assert list(p) == [0xF1, 0x79, 0x80, 0x43]
    assert np.array_equal(quant.unpack_nibbles(p), codes)
    u = np.array([0, 15, 7, 8], np.uint8)
    assert list(quant.pack_nibbles(u)) == [0xF0, 0x87]
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(u), signed=False), u)
    rng = np.random.default_rng(3)
    c = rng.integers(-7, 8, size=(5, 6, 128)).astype(np.int8)
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(c)), c)


def test_dequant_is_fl32_of_exact_product():
    rng = np.random.default_rng(5)
    x = _rand_rows(rng, 300, 128)
    q, s = quant.quantize_int4(x, 64)
    d = quant.dequantize_int4(q, s, 64)
    exact = quant.dequantize_int4_exact(q, s, 64)
    # q (3 bits) * s (24 bits) is exact in fp64; fl32 of it is one rounding
    assert np.array_equal(d, exact.astype(np.float32))
    # and exact product is q*s by hand for a few entries
    assert exact[0, 0] == float(q[0, 0]) * float(s[0, 0])


@pytest.mark.parametrize("g", [32, 64, 128])
def test_dequant_error_bound_every_group(g):
    """|x - dequant(quant(x))| <= s/2 element by element, with the bound taken per group
    from the dequantized output itself ([KV-4bit] §2.1: round to the nearest multiple of
    the group's scale).  Adjacent groups get scales four decades apart, so a dequantizer
    that applied one group's scale to another group would break the bound by orders of
    magnitude."""
    rng = np.random.default_rng(11)
    D = 128
    ng = D // g
    x = rng.standard_normal((400, D))
    mag = 10.0 ** (4 * (np.arange(ng) % 2) - 2)            # 1e-2, 1e2, 1e-2, ...
    x = (x.reshape(400, ng, g) * mag[None, :, None]).reshape(400, D).astype(np.float16)
    q, s = quant.quantize_int4(x, g)
    xd = x.astype(np.float64).reshape(400, ng, g)
    bound = s.astype(np.float64)[..., None] * (0.5 + 2.0 ** -21)
    for deq in (quant.dequantize_int4(q, s, g).astype(np.float64),
                quant.dequantize_int4_exact(q, s, g)):
        err = np.abs(xd - deq.reshape(400, ng, g))
        # fl32 of the product adds at most half an ulp of |q s| <= 7 s
        assert np.all(err <= bound + 7 * s.astype(np.float64)[..., None] * 2.0 ** -24)
        # the groups' outputs really live at their own scale
        assert np.all(np.abs(deq.reshape(400, ng, g)).max(-1) <= 7 * s.astype(np.float64) * (1 + 2.0 ** -23))


def test_dequant_hand_case_two_groups():
    """By hand, D = 128, g = 64.  Group 0 holds 7, 3.5, 0: amax 7, s = 1, codes 7, 4
    (half to even), 0 -> 7, 4, 0.  Group 1 holds -1400, 700, 350: amax 1400, s = 200,
    codes -7, 4 (3.5 to even), 2 (1.75) -> -1400, 800, 400."""
    x = np.zeros((1, 128), np.float16)
    x[0, :3] = [7.0, 3.5, 0.0]
    x[0, 64:67] = [-1400.0, 700.0, 350.0]
    q, s = quant.quantize_int4(x, 64)
    assert list(s[0]) == [1.0, 200.0]
    for deq in (quant.dequantize_int4(q, s, 64), quant.dequantize_int4_exact(q, s, 64)):
        assert list(deq[0, :3]) == [7.0, 4.0, 0.0]
        assert list(deq[0, 64:67]) == [-1400.0, 800.0, 400.0]
        assert not deq[0, 3:64].any() and not deq[0, 67:].any()


def test_int8_dequant_bound_and_hand_case():
    """Per-token INT8 ([KV-opt] §3.1): |x - dequant(quant(x))| <= s/2 per row, with rows
    of very different magnitude; by hand, row 0 = (127, 63.5): s = 1, codes 127, 64 (to
    even) -> 127, 64; row 1 = (-254, 1): s = 2, codes -127, 0 (0.5 to even) -> -254, 0."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((300, 128)) * 10.0 ** rng.integers(-3, 4, (300, 1))).astype(np.float16)
    q, s = quant.quantize_int8(x)
    sd = s.astype(np.float64)[:, None]
    for deq in (quant.dequantize_int8(q, s).astype(np.float64), quant.dequantize_int8_exact(q, s)):
        err = np.abs(x.astype(np.float64) - deq)
        assert np.all(err <= sd * (0.5 + 2.0 ** -17) + 127 * sd * 2.0 ** -24)
    h = np.zeros((2, 128), np.float16)
    h[0, :2] = [127.0, 63.5]
    h[1, :2] = [-254.0, 1.0]
    qh, sh = quant.quantize_int8(h)
    assert list(sh) == [1.0, 2.0]
    for deq in (quant.dequantize_int8(qh, sh), quant.dequantize_int8_exact(qh, sh)):
        assert list(deq[0, :2]) == [127.0, 64.0] and list(deq[1, :2]) == [-254.0, 0.0]
        assert not deq[:, 2:].any()


# ---------------------------------------------------------------- INT8 per-token


def test_int8_rules():
    rng = np.random.default_rng(9)
    x = _rand_rows(rng, 500, 128)
    x[17] = 0
    q, s = quant.quantize_int8(x)
    assert s.shape == (500,) and s.dtype == np.float32
    assert s[17] == np.float32(1e-8) and not q[17].any()
    xd = x.astype(np.float64)
    am = np.abs(xd).argmax(-1)
    nz = np.abs(xd).max(-1) > 0
    assert np.all(np.abs(q[np.arange(500), am][nz]) == 127)
    assert np.all(np.abs(xd - q * s.astype(np.float64)[:, None]) <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -17))
    # fp64 route
    a = np.abs(xd).max(-1)
    s64 = np.maximum((a / 127.0).astype(np.float32), np.float32(1e-8))
    y = (xd / s64.astype(np.float64)[:, None]).astype(np.float32)
    q64 = np.clip(np.rint(y.astype(np.float64)), -128, 127).astype(np.int8)
    assert np.array_equal(s, s64) and np.array_equal(q, q64)
    # tiny rows hit the 1e-8 floor: amax below 127e-8
    t = np.zeros((1, 128), np.float16)
    t[0, 0] = np.float16(6e-8)   # smallest fp16 subnormal ~5.96e-8
    qt, st = quant.quantize_int8(t)
    assert st[0] == np.float32(1e-8) and qt[0, 0] == 6
    dq = quant.dequantize_int8(q, s)
    assert np.array_equal(dq, quant.dequantize_int8_exact(q, s).astype(np.float32))



# ---- INT4 with fp16 scales (lpnh.cn/news/2042373 §2.1 computed in fp16; §2.2's 16-bit
# scale accounting)

def _page_fp16(x16, group):
    """The page's quantize_4bit_group as torch fp16 operations on the CPU."""
    x = torch.from_numpy(np.ascontiguousarray(x16)).reshape(-1, group)
    scale = x.abs().amax(dim=-1, keepdim=True) / 7
    scale = torch.where(scale == 0, torch.ones_like(scale), scale)
    q = torch.round(x / scale).clamp(-7, 7)
    return q.to(torch.int8).reshape(x16.shape).numpy(), scale.reshape(x16.shape[:-1] + (-1,)).numpy()


@pytest.mark.parametrize("group", [32, 64, 128])
def test_fp16_scale_quantizer_equals_the_pages_fp16_code(group):
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-12, 6, (64, 1)))).astype(np.float16)
    x[3] = 0                                               # all-zero groups
    x[5, :group] = np.float16(6e-8)                        # amax / 7 underflows to 0 in fp16
    x[7, 0] = np.float16(65504.0)                          # the largest fp16
    q, s = quant.quantize_int4_fp16_scale(x, group)
    qp, sp = _page_fp16(x, group)
    assert s.dtype == np.float16
    assert np.array_equal(s.view(np.uint16), sp.view(np.uint16))
    assert np.array_equal(q, qp)
    assert np.all(s[3] == 1.0) and np.all(q[3] == 0) and s[5, 0] == 1.0


def test_fp16_scale_quotient_rounds_in_fp16():
    """amax 4.176 (fp16 0x442D) gives s = fl16(amax / 7) = 0.5967; x = 3.281 (0x4290)
    then has x / s = 5.49918..., which is 5.5 in fp16 and rounds half to even to 6,
    where rounding the fp32 quotient would give 5: the codes follow the fp16 quotient."""
    x = np.zeros(32, dtype=np.float16)
    x[0] = np.array(0x442D, dtype=np.uint16).view(np.float16)
    x[1] = np.array(0x4290, dtype=np.uint16).view(np.float16)
    q, sc = quant.quantize_int4_fp16_scale(x, 32)
    assert np.float32(x[1]) / np.float32(sc[0]) < 5.5
    assert q[1] == 6 and q[0] == 7
    qp, _ = _page_fp16(x, 32)
    assert np.array_equal(q, qp)


def test_fp16_scale_storage_matches_the_pages_bits():
    """fp16 scales give the page's 4 + 16/g bits: 4.25 (K, g 64) and 4.125 (V, g 128)."""
    assert memory.int4_cache_bytes(1, 1, 1, 128, 64, scale_bytes=2) * 8 / 128 == memory.effective_bits(64)
    assert memory.effective_bits(64) == 4.25 and memory.effective_bits(128) == 4.125
