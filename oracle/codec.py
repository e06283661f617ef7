"""Walsh-Hadamard rotation + Lloyd-Max 4-bit KV codec (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page cited
  [LARQL]  "长上下文内存大瘦身：LARQL 四大 KV 缓存引擎原理与横向对比"
           (pwwt.cn/news/5725003), "engine three: codec (turbo-quant)": each K/V row
           is coded per head with a Walsh-Hadamard (WHT) rotation followed by
           Lloyd-Max quantization at 3 or 4 bits; head_dim must be a power of two;
           the codec is approximate, with a per-row cosine of about 0.9954 at 4 bits.

The page names the two steps and nothing else.  The plainest algorithm that its
statement supports, used here:
  1. rotate:   y = H_d x / sqrt(d), H_d the Sylvester-ordered +-1 Hadamard matrix
               (H_ij = (-1)^popcount(i & j)); orthonormal, no random sign flips;
  2. scale:    s = ||x||_2 / sqrt(d) (the RMS of the row; the codebook is for a
               unit-variance Gaussian, which the rotated coordinates approach);
  3. quantize: idx_i = #{ j : tau_j < y_i / s } over the 15 decision thresholds of
               the 16-level Lloyd-Max quantizer of N(0, 1) (ties go to the lower
               cell; a zero row has s = 0 and is coded as y / 1 = 0);
  4. decode:   x_hat = s * H_d c[idx] / sqrt(d).
The codebook is the fixed point of Lloyd's two conditions for N(0, 1): thresholds
are midpoints of adjacent levels, and each level is the conditional mean of its
cell, c_j = (phi(t_{j-1}) - phi(t_j)) / (Phi(t_j) - Phi(t_{j-1})).
"""

import math

import numpy as np


def hadamard_transform(x):
    """Unnormalized Sylvester Walsh-Hadamard transform of the last axis (fp64).

    Butterflies of the recursive definition H_2n = [[H_n, H_n], [H_n, -H_n]].
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("head_dim must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def rotate(x):
    """Orthonormal rotation y = H_d x / sqrt(d) (its own inverse)."""
    d = np.shape(x)[-1]
    return hadamard_transform(x) / math.sqrt(d)


def _phi(t):
    return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _Phi(t):
    return 0.5 * (1.0 + np.vectorize(math.erf)(t / math.sqrt(2.0)))


def lloyd_max_gaussian(bits, tol=1e-14, max_iter=200000):
    """Lloyd-Max quantizer of N(0, 1) with 2**bits levels (fp64 fixed-point iteration).

    Returns (levels [2**bits] ascending, thresholds [2**bits - 1] ascending, mse).
    """
    n = 1 << bits
    c = np.linspace(-2.5, 2.5, n)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], t))
        hi = np.concatenate((t, [np.inf]))
        pl = np.where(np.isinf(lo), 0.0, _phi(np.where(np.isinf(lo), 0.0, lo)))
        ph = np.where(np.isinf(hi), 0.0, _phi(np.where(np.isinf(hi), 0.0, hi)))
        Pl = np.where(np.isinf(lo), 0.0, _Phi(np.where(np.isinf(lo), 0.0, lo)))
        Ph = np.where(np.isinf(hi), 1.0, _Phi(np.where(np.isinf(hi), 0.0, hi)))
        c_new = (pl - ph) / (Ph - Pl)
        done = np.max(np.abs(c_new - c)) < tol
        c = c_new
        if done:
            break
    c = 0.5 * (c - c[::-1])  # the N(0,1) quantizer is odd-symmetric; remove rounding asymmetry
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    P = np.where(np.isinf(hi), 1.0, _Phi(np.where(np.isinf(hi), 0.0, hi))) - \
        np.where(np.isinf(lo), 0.0, _Phi(np.where(np.isinf(lo), 0.0, lo)))
    mse = 1.0 - float(np.sum(c * c * P))  # E[X^2] - E[c(X)^2] at the fixed point
    return c, t, mse


_CODEBOOK = {}


def codebook(bits=4):
    if bits not in _CODEBOOK:
        _CODEBOOK[bits] = lloyd_max_gaussian(bits)
    return _CODEBOOK[bits]


def encode(x16, bits=4):
    """Codec encode of rows (last axis = head_dim) per the four steps above.

    Returns (idx uint8 [..., D] in 0..2**bits-1, scale float32 [...], normalized
    rotated values u = y / s as fp64 [..., D] for boundary checks).
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    d = x.shape[-1]
    levels, thr, _ = codebook(bits)
    y = rotate(x)
    s = np.sqrt(np.sum(x * x, axis=-1)) / math.sqrt(d)
    div = np.where(s == 0.0, 1.0, s)
    u = y / div[..., None]
    idx = np.searchsorted(thr, u, side="left")  # number of thresholds strictly below u
    return idx.astype(np.uint8), s.astype(np.float32), u


def decode(idx, scale, bits=4):
    """x_hat = s * H_d c[idx] / sqrt(d), fp64."""
    levels, _, _ = codebook(bits)
    c = levels[np.asarray(idx, dtype=np.int64)]
    return np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None] * rotate(c)


def row_cosine(x, x_hat):
    x = np.asarray(x, dtype=np.float64)
    x_hat = np.asarray(x_hat, dtype=np.float64)
    num = np.sum(x * x_hat, axis=-1)
    den = np.sqrt(np.sum(x * x, axis=-1) * np.sum(x_hat * x_hat, axis=-1))
    return num / den
