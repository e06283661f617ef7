"""KV-cache size and effective-bit closed forms (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited
  [INT4-SM] "LLM长上下文推理优化：用INT4状态机管理KV Cache" (pwwt.cn/news/4219524),
            section 2 (bytes per token, 2 * layers * heads * head_dim * dtype) and
            section 6.2 (``cache_memory``).
  [KV-4bit] lpnh.cn/news/2042373, section 1.2 (M = 2 * L * H_kv * d_head * S * B *
            dtype_size; its FP16 table) and section 2.2 (effective bits 4 + 16/g).
  [KV-opt]  bxzpzcl.cn/news/2871434, section 2 (the same formula).
  [LARQL]   pwwt.cn/news/5725003, the Gemma 3 4B residency table.

Reading: "KB" / "GB" on the pages are binary units (KiB / GiB).
"""


def kv_bytes(layers, kv_heads, head_dim, seq, batch, bits_per_elem):
    """M = 2 (K and V) * L * H_kv * d * S * B * bits / 8, in bytes."""
    return 2 * layers * kv_heads * head_dim * seq * batch * bits_per_elem / 8


def effective_bits(group, code_bits=4, scale_bits=16):
    """Bits per element when every ``group`` codes share one scale: 4 + 16/g at fp16."""
    return code_bits + scale_bits / group


def compression_vs_fp16(group, code_bits=4, scale_bits=16):
    return 16.0 / effective_bits(group, code_bits, scale_bits)


def int4_cache_bytes(batch, kv_heads, capacity, head_dim, group, scale_bytes=4):
    """Bytes of one packed INT4 tensor (K or V): codes D/2 per row plus one scale per group."""
    return batch * kv_heads * capacity * (head_dim // 2 + scale_bytes * (head_dim // group))


def resident_rows(layers_window, window, layers_global, positions):
    """Rows kept when window layers hold only their last ``window`` positions."""
    return layers_window * min(window, positions) + layers_global * positions
