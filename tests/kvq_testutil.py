"""Helpers for the GPU parity tests: device buffers <-> numpy, error metrics.

No arithmetic of the method lives here; expected values come from ``oracle/`` only.
"""
import os

import numpy as np
import torch

import int4_quantized_kv_amd as kvq
from oracle import attention, codec, quant

# Attention tolerance against the fp64 oracle over the same dequantized values.
ATTN_MAX_ABS = 2e-3
ATTN_REL_L2 = 1e-4


def np16(t):
    return t.detach().to("cpu").numpy().astype(np.float16)


def cache_arrays(dc, fmt):
    """(k_codes, k_scales, v_codes, v_scales) of a DeviceCache as numpy, shaped
    [B, Hkv, C, bytes per row] / [B, Hkv, C, scales per row]."""
    d = dc.desc
    B, H, C, D = d.batch, d.kv_heads, d.capacity, d.head_dim
    torch.cuda.synchronize()
    row = D if fmt == "int8" else (3 * D // 8 if fmt == "codec3" else D // 2)
    kc = dc.k_codes.cpu().numpy().reshape(B, H, C, row)
    vc = dc.v_codes.cpu().numpy().reshape(B, H, C, row)
    if fmt == "int8":
        kc = kc.view(np.int8)
        vc = vc.view(np.int8)
    if fmt == "int4h":   # fp16 scales, D / g per row
        ks = dc.k_scales.cpu().numpy().view(np.float16)[:B * H * C * (D // d.group_k)].reshape(B, H, C, -1)
        vs = dc.v_scales.cpu().numpy().view(np.float16)[:B * H * C * (D // d.group_v)].reshape(B, H, C, -1)
    else:
        ks = dc.k_scales.cpu().numpy().reshape(B, H, C, -1)
        vs = dc.v_scales.cpu().numpy().reshape(B, H, C, -1)
    return kc, ks, vc, vs


def attn_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return max_abs, rel


def assert_attn_close(got, ref, what=""):
    max_abs, rel = attn_errors(got, ref)
    log = os.environ.get("KVQ_TEST_METRICS")   # optional: one line per check, for margins
    if log:
        with open(log, "a") as f:
            f.write(f"{max_abs:.3e} {rel:.3e} {what}\n")
    assert max_abs <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, \
        f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def decode(desc, dc, q, q_heads, lens, window=0, scale=0.0, num_splits=0, ws=None):
    """Run kvq_decode_attn (with a fresh zeroed workspace unless one is given); returns
    the fp32 output tensor."""
    if ws is None:
        ws = kvq.decode_workspace(desc, q_heads, max(lens), window, num_splits, q.device)
    out = torch.empty((desc.batch, q_heads, desc.head_dim), dtype=torch.float32, device=q.device)
    kvq.kvq_decode_attn(desc, dc.c, q, q_heads, lens, window, scale, num_splits, out, ws)
    torch.cuda.synchronize()
    return out


def append_decode(desc, dc, k_new, v_new, q, q_heads, lens, window=0, scale=0.0,
                  num_splits=0, ws=None):
    """Run kvq_append_decode_attn (fresh zeroed workspace unless one is given)."""
    if ws is None:
        ws = kvq.decode_workspace(desc, q_heads, max(lens), window, num_splits, q.device)
    out = torch.empty((desc.batch, q_heads, desc.head_dim), dtype=torch.float32, device=q.device)
    kvq.kvq_append_decode_attn(desc, dc.c, k_new, v_new, q, q_heads, lens, window, scale,
                               num_splits, out, ws)
    torch.cuda.synchronize()
    return out


# ----------------------------------------------------------------------------- codec rows

def pack3(idx):
    """3-bit indices [..., D] (0..7) -> the library's rows [..., 3 * D / 8] uint8: index i in
    bits 3i .. 3i + 2 of the row read as a little-endian bit string."""
    idx = np.asarray(idx, dtype=np.uint8)
    bits = ((idx[..., None] >> np.arange(3, dtype=np.uint8)) & 1).reshape(*idx.shape[:-1], -1)
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack3(rows):
    rows = np.asarray(rows, dtype=np.uint8)
    bits = np.unpackbits(rows, axis=-1, bitorder="little").reshape(*rows.shape[:-1], -1, 3)
    return (bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)).astype(np.uint8)


def codec_indices(codes, fmt):
    """Stored codec rows -> indices [..., D]."""
    if fmt == "codec3":
        return unpack3(codes)
    return quant.unpack_nibbles(codes, signed=False)


def check_codec_rows(got_idx, got_scale, x16, bits):
    """The codec's GPU rule: scales within 1e-5 relative of the oracle's, and an index
    may differ from the oracle's only where the oracle's normalized rotated value lies
    within 1e-5 of a decision threshold.  Returns the number of differing indices."""
    idx, s, u = codec.encode(x16, bits=bits)
    assert np.allclose(got_scale, s, rtol=1e-5, atol=0), "codec row scales differ"
    mism = got_idx != idx
    if mism.any():
        _, thr, _ = codec.codebook(bits)
        d = np.min(np.abs(u[mism][:, None] - thr[None, :]), axis=1)
        assert np.all(d <= 1e-5), f"{int((d > 1e-5).sum())} codes differ away from a threshold"
    return int(mism.sum())


def slot_of(p, cap, sinks=0):
    """Slot of position p: p below the sinks, else the ring of cap - sinks slots."""
    return p if p < sinks else sinks + (p - sinks) % (cap - sinks)


def codec_hat_from_device(dc, fmt, k16, v16, lens, window=0):
    """Rows attention is checked over, for a codec cache coded on the GPU.

    k16, v16: fp16 [B, Hkv, N, D] source rows indexed by position (N >= max(lens)).
    Every position a decode at ``lens`` attends is read back from its slot in the
    device cache and held to the codec rule of ``check_codec_rows`` against the
    oracle's own encoding of the same fp16 row; the oracle then decodes those indices
    (where the rule leaves two indices correct, the one the GPU stored is used, so both
    sides attend over identical values).  Positions not attended keep the oracle's
    codes.  Returns (k_hat, v_hat) fp64 [B, Hkv, N, D] and the number of indices that
    differ from the oracle's.
    """
    d = dc.desc
    bits = 3 if fmt == "codec3" else 4
    kc, ks, vc, vs = cache_arrays(dc, fmt)
    out = []
    nmis = 0
    for x16, codes, scales in ((k16, kc, ks), (v16, vc, vs)):
        idx, sc, _ = codec.encode(x16, bits=bits)
        idx, sc = idx.copy(), sc.copy()
        for b, ln in enumerate(lens):
            pos = attention.attended_positions(int(ln), window, d.sinks)
            slots = np.array([slot_of(int(p), d.capacity, d.sinks) for p in pos])
            g_idx = codec_indices(codes[b][:, slots], fmt)
            g_sc = scales[b][:, slots, 0]
            nmis += check_codec_rows(g_idx, g_sc, x16[b][:, pos], bits)
            idx[b][:, pos] = g_idx
            sc[b][:, pos] = g_sc
        out.append(codec.decode(idx, sc, bits=bits))
    return out[0], out[1], nmis
