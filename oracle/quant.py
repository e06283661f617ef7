"""Group-wise symmetric INT4 and per-token INT8 KV quantization (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited
  [KV-4bit]  lpnh.cn/news/2042373, the practitioner article on compressing the KV
             cache from FP16 to 4 bits: section 2.1 (``quantize_4bit_group`` /
             ``dequantize_4bit_group``) and section 2.2 (group size table; K group 64,
             V group 128).
  [KV-opt]   "AI 推理性能调优：KV Cache 优化与显存管理的工程实践"
             (bxzpzcl.cn/news/2871434), section 3.1 (``KVCacheQuantizer.quantize_int8``).

Readings taken where the text is silent or garbled:
  * Groups are ``g`` contiguous elements of the last axis (head_dim): the page
    reshapes "the last dim" into groups of ``group_size``.
  * The page's zero-group rule lost its comparison operator in the text: read as a
    scale that is exactly zero (a group of zeros) being replaced by 1.
  * Scales are fp32 and every step is fp32: ``s = fl32(amax / 7)``, then the
    quotient ``fl32(x / s)`` is rounded to fp32 *before* rounding to an integer.
  * Rounding is half-to-even (``torch.round`` semantics).
  * Codes are stored as 4-bit two's complement, element ``2i`` in the low nibble of
    byte ``i`` and element ``2i+1`` in the high nibble.
  * INT8: the scale is per (token, head) over head_dim (the code reduces ``dim=-1``
    although its comment says per-channel); the ``1e-8`` floor is applied in fp32
    (on an fp16 tensor it would underflow to zero).
"""

import numpy as np

F32 = np.float32


def quantize_int4(x16, group):
    """INT4 group quantization of the last axis ([KV-4bit] §2.1, ``quantize_4bit_group``).

    For each group of ``group`` contiguous elements of the last axis:
      a = max |x|;  s = fl32(a / 7), replaced by 1 when it is 0;
      q = clamp(round_half_even(fl32(x / s)), -7, 7).

    x16: array of fp16 values, last axis divisible by ``group``.
    Returns (codes int8 [..., D], scales float32 [..., D // group]).
    """
    x = np.asarray(x16, dtype=np.float16).astype(F32)  # exact widening
    D = x.shape[-1]
    if D % group != 0:
        raise ValueError("head_dim must be a multiple of the group size")
    xg = x.reshape(x.shape[:-1] + (D // group, group))
    a = np.max(np.abs(xg), axis=-1)                      # per-group amax, fp32 (exact)
    s = (a / F32(7.0)).astype(F32)                       # IEEE fp32 division
    s = np.where(s == F32(0.0), F32(1.0), s).astype(F32)  # all-zero group -> scale 1
    y = (xg / s[..., None]).astype(F32)                  # fl32(x / s)
    q = np.clip(np.rint(y), -7, 7)                       # half-to-even, clamp [-7, 7]
    return q.astype(np.int8).reshape(x.shape), s


def quantize_int4_fp16_scale(x16, group):
    """INT4 group quantization with fp16 scales: the page's ``quantize_4bit_group`` run
    in the tensor's own fp16 ([KV-4bit] §2.1; the fp16 storage is the 16-bit scale its
    §2.2 accounting assumes, 4 + 16/g bits per element).

      s = fl16(a / 7), replaced by 1 when it is 0;  q = clamp(rne(fl16(x / s)), -7, 7).

    Each quotient is formed in fp64 and rounded once to fp16: the correctly rounded fp16
    quotient.  Returns (codes int8 [..., D], scales float16 [..., D // group]).
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)   # exact widening
    D = x.shape[-1]
    if D % group != 0:
        raise ValueError("head_dim must be a multiple of the group size")
    xg = x.reshape(x.shape[:-1] + (D // group, group))
    a = np.max(np.abs(xg), axis=-1)
    s = (a / 7.0).astype(np.float16)                            # fl16(a / 7)
    s = np.where(s == 0, np.float16(1.0), s).astype(np.float16)
    y = (xg / s.astype(np.float64)[..., None]).astype(np.float16)   # fl16(x / s)
    q = np.clip(np.rint(y.astype(np.float64)), -7, 7)
    return q.astype(np.int8).reshape(x.shape), s


def dequantize_int4(codes, scales, group):
    """``x_hat = fl32(q * s)`` per group ([KV-4bit] §2.1, ``dequantize_4bit_group``)."""
    q = np.asarray(codes).astype(F32)
    D = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (D // group, group))
    out = (qg * np.asarray(scales, dtype=F32)[..., None]).astype(F32)
    return out.reshape(q.shape)


def dequantize_int4_exact(codes, scales, group):
    """``q * s`` evaluated exactly in fp64 (the values attention is defined over)."""
    q = np.asarray(codes).astype(np.float64)
    D = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (D // group, group))
    out = qg * np.asarray(scales, dtype=F32).astype(np.float64)[..., None]
    return out.reshape(q.shape)


def pack_nibbles(codes):
    """Pack 4-bit values (signed -8..7 or unsigned 0..15) two per byte.

    Element 2i goes to the low nibble of byte i, element 2i+1 to the high nibble;
    signed values are stored as 4-bit two's complement.
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, signed=True):
    """Inverse of ``pack_nibbles``: uint8 [..., D/2] -> int8 [..., D]."""
    b = np.asarray(packed).astype(np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def quantize_int8(x16):
    """Per-token symmetric INT8 over head_dim ([KV-opt] §3.1, ``quantize_int8``).

    s = max(fl32(amax / 127), 1e-8);  q = clamp(round_half_even(fl32(x / s)), -128, 127).
    Returns (codes int8 [..., D], scales float32 [...]).
    """
    x = np.asarray(x16, dtype=np.float16).astype(F32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / F32(127.0)).astype(F32)
    s = np.maximum(s, F32(1e-8)).astype(F32)
    y = (x / s[..., None]).astype(F32)
    q = np.clip(np.rint(y), -128, 127)
    return q.astype(np.int8), s


def dequantize_int8(codes, scales):
    """``x_hat = fl32(q * s)`` ([KV-opt] §3.1, ``dequantize_int8``)."""
    q = np.asarray(codes).astype(F32)
    return (q * np.asarray(scales, dtype=F32)[..., None]).astype(F32)


def dequantize_int8_exact(codes, scales):
    q = np.asarray(codes).astype(np.float64)
    return q * np.asarray(scales, dtype=F32).astype(np.float64)[..., None]
