"""Helpers for the GPU parity tests: device buffers <-> numpy, error metrics.

No arithmetic of the method lives here; expected values come from ``oracle/`` only.
"""
import numpy as np
import torch

import int4_quantized_kv_amd as kvq

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
