"""Seeded synthetic K/V/query generators shared by the tests, the benchmark and smoke.

This module holds no quantization, attention or codec arithmetic: it only draws
fp16 tensors with the shapes, value distributions and structure (outlier channels,
per-head scales, zeroed groups) of the workloads the pages describe, so that the
oracle and the HIP library can be fed identical inputs.

Seeds follow ``1000 * workload + 10 * layer + stream`` with stream 0 = K source,
1 = V source, 2 = query, 3 = appended K row, 4 = appended V row.
The bulk normal draws use a ``torch.Generator`` on the requested device (the GPU
stream differs from the CPU stream for the same seed, so parity tests draw on the
device and copy to the host); outlier channels and per-head scales are always
drawn on the CPU so they do not depend on the device.
"""

import math
from dataclasses import dataclass, field

import torch

K_SRC, V_SRC, Q_SRC, K_NEW, V_NEW = 0, 1, 2, 3, 4


def seed_of(workload, layer, stream):
    return 1000 * workload + 10 * layer + stream


def _normal(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def kv_source(shape, seed, device="cpu", outlier_channels=0, outlier_mult=20.0,
              head_scale_range=None, zero_groups=(), struct_seed=None):
    """fp16 [B, H, S, D] ~ N(0, 1) with optional structure.

    outlier_channels: number of head_dim channels per head (drawn without
        replacement, shared across batch and positions) multiplied by ``outlier_mult``.
    head_scale_range: (lo, hi) -> each head is multiplied by exp(U(ln lo, ln hi)).
    zero_groups: iterable of (b, h, t, start, length) spans set to exactly zero.
    struct_seed: seed of the outlier channels and head scales (default ``seed``), so
        that appended rows share the structure of the cache they are appended to.
    """
    B, H, S, D = shape
    x = _normal(shape, seed, device)
    gc = torch.Generator(device="cpu")
    gc.manual_seed((seed if struct_seed is None else struct_seed) + 7_000_000)
    if head_scale_range is not None:
        lo, hi = head_scale_range
        u = torch.rand((H,), generator=gc, dtype=torch.float64)
        sc = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.float32)
        x *= sc.to(device).view(1, H, 1, 1)
    if outlier_channels > 0:
        mult = torch.ones((H, D), dtype=torch.float32)
        for h in range(H):
            idx = torch.randperm(D, generator=gc)[:outlier_channels]
            mult[h, idx] = outlier_mult
        x *= mult.to(device).view(1, H, 1, D)
    for (b, h, t, start, length) in zero_groups:
        x[b, h, t, start:start + length] = 0.0
    return x.to(torch.float16)


def query(shape, seed, device="cpu"):
    """fp16 [B, Hq, D] ~ N(0, 1)."""
    return _normal(shape, seed, device).to(torch.float16)


@dataclass
class Workload:
    """Shape and input recipe of one synthetic workload."""
    wid: int
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    context: int            # cached positions before the decode step
    append: bool            # whether the decode step first appends one token
    outlier_channels: int = 0
    outlier_mult: float = 20.0
    head_scale_range: tuple = None
    fmt: str = "int4"        # "int4", "int4h" (fp16 scales), "int8", "codec", "codec3"
    group_k: int = 64
    group_v: int = 128
    window_layers: int = 0  # number of sliding-window layers (the first ones)
    window: int = 0
    sinks: int = 0          # attention-sink positions kept besides a window layer's ring
    recent: int = 0         # last positions also kept (and read) in fp16
    zero_groups: tuple = field(default=())
    page_size: int = 0      # paged layout: positions per page (0 = contiguous buffers)

    def layer_window(self, layer):
        return self.window if layer < self.window_layers else 0


WORKLOADS = {
    1: Workload(1, "tiny-mha-d128-s256", layers=1, batch=1, q_heads=4, kv_heads=4,
                head_dim=128, context=256, append=False, outlier_channels=2,
                zero_groups=((0, 1, 37, 0, 128),)),
    2: Workload(2, "llama3-8b-gqa4-ctx8k-b8", layers=32, batch=8, q_heads=32, kv_heads=8,
                head_dim=128, context=8192, append=True,
                outlier_channels=round(0.02 * 128)),
    3: Workload(3, "mha7b-ctx20k-b8", layers=32, batch=8, q_heads=32, kv_heads=32,
                head_dim=128, context=20480, append=False,
                outlier_channels=round(0.01 * 128), outlier_mult=30.0,
                head_scale_range=(0.05, 5.0)),
    4: Workload(4, "gemma3-4b-window-codec-b4", layers=34, batch=4, q_heads=8, kv_heads=4,
                head_dim=256, context=4096, append=True, fmt="codec",
                window_layers=29, window=1024),
    5: Workload(5, "ctx128k-b1-gqa4", layers=32, batch=1, q_heads=32, kv_heads=8,
                head_dim=128, context=131072, append=False,
                outlier_channels=round(0.02 * 128)),
    6: Workload(6, "llama3-8b-window4k-sinks4-b8", layers=32, batch=8, q_heads=32, kv_heads=8,
                head_dim=128, context=8192, append=True,
                outlier_channels=round(0.02 * 128), window_layers=32, window=4096, sinks=4),
    7: Workload(7, "llama3-8b-gqa4-ctx8k-b8-recent128", layers=32, batch=8, q_heads=32,
                kv_heads=8, head_dim=128, context=8192, append=True,
                outlier_channels=round(0.02 * 128), recent=128),
    8: Workload(8, "gemma3-4b-window-codec3-b4", layers=34, batch=4, q_heads=8, kv_heads=4,
                head_dim=256, context=4096, append=True, fmt="codec3",
                window_layers=29, window=1024),
    9: Workload(9, "llama3-8b-gqa4-ctx8k-b8-int4h", layers=32, batch=8, q_heads=32, kv_heads=8,
                head_dim=128, context=8192, append=True, fmt="int4h",
                outlier_channels=round(0.02 * 128)),
    10: Workload(10, "llama3-8b-gqa4-ctx8k-b8-paged16", layers=32, batch=8, q_heads=32, kv_heads=8,
                 head_dim=128, context=8192, append=True, outlier_channels=round(0.02 * 128),
                 page_size=16),
}


def block_table(batch, positions, page_size, seed, spare=0):
    """A seeded block table [batch, ceil(positions / page_size)] (int32, CPU) over a
    pool of exactly the pages the sequences need plus `spare`: page ids in a shuffled
    order, so that consecutive pages of a sequence lie anywhere in the pool.  Returns
    (table, pages in the pool)."""
    pps = (positions + page_size - 1) // page_size
    pages = batch * pps + spare
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 9_000_000)
    perm = torch.randperm(pages, generator=g)[:batch * pps]
    return perm.view(batch, pps).to(torch.int32).contiguous(), pages


def layer_inputs(w, layer, device, context=None, batch=None):
    """Source K/V [B, Hkv, S, D], query [B, Hq, D] and (if the workload appends) the new
    token's K/V rows [B, Hkv, D] for one layer of workload ``w``."""
    S = w.context if context is None else context
    B = w.batch if batch is None else batch
    shp = (B, w.kv_heads, S, w.head_dim)
    zg = tuple(z for z in w.zero_groups if z[0] < B and z[2] < S)
    k = kv_source(shp, seed_of(w.wid, layer, K_SRC), device, w.outlier_channels,
                  w.outlier_mult, w.head_scale_range)
    v = kv_source(shp, seed_of(w.wid, layer, V_SRC), device, w.outlier_channels,
                  w.outlier_mult, w.head_scale_range, zero_groups=zg)
    q = query((B, w.q_heads, w.head_dim), seed_of(w.wid, layer, Q_SRC), device)
    kn = vn = None
    if w.append:
        one = (B, w.kv_heads, 1, w.head_dim)
        kn = kv_source(one, seed_of(w.wid, layer, K_NEW), device, w.outlier_channels,
                       w.outlier_mult, w.head_scale_range,
                       struct_seed=seed_of(w.wid, layer, K_SRC))[:, :, 0]
        vn = kv_source(one, seed_of(w.wid, layer, V_NEW), device, w.outlier_channels,
                       w.outlier_mult, w.head_scale_range,
                       struct_seed=seed_of(w.wid, layer, V_SRC))[:, :, 0]
    return k, v, q, kn, vn
