"""Pins of oracle/memory.py against the figures the pages print (tests/golden)."""
import pytest

from oracle import memory
from tests.golden.parse import page_figures

# the codec's row-cosine figure is checked against the codec oracle in test_oracle_codec.py
FIGS = [f for f in page_figures() if f[0] != "codec_row_cosine"]


@pytest.mark.parametrize("name,d,cite", FIGS, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(FIGS)])
def test_page_figure(name, d, cite):
    if name == "kv_bytes":
        got = memory.kv_bytes(int(d["layers"]), int(d["kv_heads"]), int(d["head_dim"]),
                              int(d["seq"]), int(d["batch"]), d["bits"])
    elif name == "effective_bits":
        got = memory.effective_bits(int(d["group"]))
    elif name == "compression":
        got = memory.compression_vs_fp16(int(d["group"]))
    elif name == "resident_rows":
        got = memory.resident_rows(int(d["layers_window"]), int(d["window"]),
                                   int(d["layers_global"]), int(d["positions"]))
    elif name == "resident_gib":
        rows = memory.resident_rows(int(d["layers_window"]), int(d["window"]),
                                    int(d["layers_global"]), int(d["positions"]))
        got = rows * 2 * d["kv_dim"] * d["bytes"] / 2 ** 30
    elif name == "residency_saving":
        full = memory.resident_rows(0, 1024, 34, 4096)
        win = memory.resident_rows(29, 1024, 5, 4096)
        got = 1 - win / full
    else:
        raise AssertionError(name)
    exp = d["expect"]
    tol = d.get("rel_tol", 0.0)
    assert abs(got - exp) <= tol * abs(exp) + 1e-12, (name, got, exp, cite)


def test_packed_int4_bytes_per_row():
    # codes D/2 bytes plus one fp32 scale per group: K (g=64) and V (g=128) at D=128
    assert memory.int4_cache_bytes(1, 1, 1, 128, 64) == 64 + 8
    assert memory.int4_cache_bytes(1, 1, 1, 128, 128) == 64 + 4
    # 140 B per (position, kv head) for K+V -> 8x8x8193 positions = 73.4 MB per layer
    tot = memory.int4_cache_bytes(8, 8, 8193, 128, 64) + memory.int4_cache_bytes(8, 8, 8193, 128, 128)
    assert tot == 8 * 8 * 8193 * 140
