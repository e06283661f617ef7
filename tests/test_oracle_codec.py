"""Pins of oracle/codec.py (CPU only).

[LARQL] pwwt.cn/news/5725003, engine three: per-head Walsh-Hadamard rotation then
Lloyd-Max quantization at 3/4 bits; head_dim a power of two; 4-bit row cosine ~0.9954.
"""
import math

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

from oracle import codec
from tests.golden.parse import lloyd_max_table, page_figures


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_wht_matches_sylvester_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, d))
    H = scipy.linalg.hadamard(d).astype(np.float64)   # Sylvester construction
    assert np.allclose(codec.hadamard_transform(x), x @ H.T, atol=1e-12)
    # H_ij = (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pc = np.vectorize(lambda n: bin(n).count("1"))(i & j)
    assert np.array_equal(H, (-1.0) ** pc)


def test_rotation_identities():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((10, 256))
    y = codec.rotate(x)
    assert np.allclose(codec.rotate(y), x, atol=1e-12)                      # involution
    assert np.allclose((y * y).sum(-1), (x * x).sum(-1), rtol=1e-12)        # Parseval
    e0 = np.zeros(256)
    e0[0] = 1
    assert np.allclose(codec.rotate(e0), np.full(256, 1 / 16), atol=1e-15)  # H e0 / sqrt(d)
    with pytest.raises(ValueError):
        codec.hadamard_transform(np.ones(48))


def test_lloyd_max_one_bit_closed_form():
    c, t, mse = codec.lloyd_max_gaussian(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-12)
    assert np.allclose(t, [0.0], atol=1e-15)
    assert abs(mse - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960_table(bits):
    tab = lloyd_max_table()[1 << bits]
    c, t, mse = codec.lloyd_max_gaussian(bits)
    n = 1 << bits
    assert np.allclose(c[n // 2:], tab["outputs"], atol=1.5e-3)
    if n > 2:
        assert np.allclose(t[n // 2:], tab["thresholds"], atol=1.5e-3)
    assert abs(mse - tab["mse"]) <= 1e-3 * tab["mse"] + 1e-6


def test_lloyd_max_optimality_by_quadrature():
    """Levels are conditional means of their cells (numerical quadrature, independent of
    the closed-form pdf/cdf expression); thresholds are midpoints; symmetric."""
    c, t, mse = codec.lloyd_max_gaussian(4)
    assert np.allclose(c, -c[::-1], atol=1e-12)
    assert np.allclose(t, 0.5 * (c[1:] + c[:-1]), atol=1e-15)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    pdf = scipy.stats.norm.pdf
    tot = 0.0
    for j in range(16):
        m0 = scipy.integrate.quad(pdf, edges[j], edges[j + 1])[0]
        m1 = scipy.integrate.quad(lambda s: s * pdf(s), edges[j], edges[j + 1])[0]
        assert abs(m1 / m0 - c[j]) < 1e-9
        tot += scipy.integrate.quad(lambda s: (s - c[j]) ** 2 * pdf(s), edges[j], edges[j + 1])[0]
    assert abs(tot - mse) < 1e-9


def test_encode_decode_rules():
    levels, thr, _ = codec.codebook(4)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 256)).astype(np.float16)
    idx, s, u = codec.encode(x)
    # idx counts the thresholds strictly below u
    assert np.array_equal(idx, (u[..., None] > thr).sum(-1))
    # s is the row RMS, fp32
    xd = x.astype(np.float64)
    assert np.allclose(s, np.sqrt((xd * xd).mean(-1)), rtol=1e-7)
    # scaling the row by a power of two leaves the codes unchanged
    idx2, s2, _ = codec.encode((x.astype(np.float32) * 4).astype(np.float16))
    assert np.array_equal(idx, idx2) and np.allclose(s2, 4 * s, rtol=1e-7)
    # zero row -> s = 0, decodes to zero
    z = np.zeros((1, 256), np.float16)
    iz, sz, _ = codec.encode(z)
    assert sz[0] == 0 and np.all(iz == 7) and np.all(codec.decode(iz, sz) == 0)
    # midpoint thresholds make the code the nearest level to y/s (ties to the lower one)
    dist = np.abs(u[..., None] - levels)
    assert np.all(dist[np.arange(50)[:, None], np.arange(256)[None, :], idx] <= dist.min(-1) + 1e-15)


def test_codec_row_cosine_matches_page():
    """Gaussian rows at head_dim 256: the mean row cosine after the 4-bit codec sits at
    the page's ~0.9954, and the rotated-domain MSE sits at the Lloyd-Max distortion."""
    fig = [f for f in page_figures() if f[0] == "codec_row_cosine"][0][1]
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4000, 256)).astype(np.float16)
    idx, s, u = codec.encode(x)
    xh = codec.decode(idx, s)
    cos = codec.row_cosine(x.astype(np.float64), xh)
    assert abs(cos.mean() - fig["expect"]) <= fig["abs_tol"]
    levels, _, mse = codec.codebook(4)
    err = (u - levels[idx]) ** 2
    assert abs(err.mean() - mse) < 4e-4


def test_codec_3bit_distortion_and_cosine():
    """At 3 bits (the page's other width) the rotated-domain MSE of Gaussian rows sits at
    the 8-level Lloyd-Max distortion (0.03454 in Max's 1960 table), and the row cosine
    follows from it: with centroid levels the coded row is the projection of the row,
    so cos^2 = 1 - mse (to first order in the scale's spread)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4000, 256)).astype(np.float16)
    idx, s, u = codec.encode(x, bits=3)
    assert idx.max() == 7 and idx.min() == 0
    levels, _, mse = codec.codebook(3)
    assert abs(mse - 0.03454) < 2e-5
    err = (u - levels[idx]) ** 2
    assert abs(err.mean() - mse) < 6e-4
    cos = codec.row_cosine(x.astype(np.float64), codec.decode(idx, s, bits=3)).mean()
    assert abs(cos - np.sqrt(1.0 - mse)) < 2e-3, cos
