"""Plain single-token decode attention over a (dequantized) KV cache (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited
  [KV-opt]  "AI 推理性能调优：KV Cache 优化与显存管理的工程实践"
            (bxzpzcl.cn/news/2871434), section 3.2 ``SlidingWindowAttention``:
            window ``[max(0, i - W + 1), i]``, GQA by repeating each KV head
            ``n_rep = Hq // Hkv`` times (query head h reads KV head ``h // n_rep``),
            ``scale = head_dim ** -0.5``, masked softmax, then weights times V.
  [KV-4bit] lpnh.cn/news/2042373, section 1.1: at decode each new token's query
            attends over every cached key/value, the new token's own K/V included.
  [INT4-SM] "LLM长上下文推理优化：用INT4状态机管理KV Cache" (pwwt.cn/news/4219524),
            section 5 step 5: the operator reads INT4 data and dequantizes inside.

Readings: the window is inclusive of the current token and holds W positions, so the
attended positions are ``[max(0, len - W), len)`` (``W = 0`` means global).  With
attention sinks ([KV-opt] §3.2: every position also sees the first
``num_sink_tokens`` positions, default 4) a windowed query attends
``[0, min(n_sink, len)) U [max(0, len - W), len)``; the page's mask also marks the
first n_sink columns for rows i < n_sink, positions after i that a decode step does
not have yet, so at decode the sinks stop at ``len``.  Everything is fp64; the
dequantized values passed in are exact (``q * s`` in fp64).

Recent tokens in FP16 ([INT4-SM] section 8.3, first way of cutting memory: INT4 for
the older tokens' K/V, FP16 kept for the recent ones).  The page fixes neither the
size of the recent span nor when a token changes form.  Reading: the span is the last
R positions of the sequence, ``[max(0, len - R), len)``, read at their fp16 values;
every older position is read at its INT4 dequantized value.  A token is quantized when
it arrives and also kept in fp16 while it is among the last R, so nothing is
re-quantized when it leaves the span.
"""

import numpy as np


def attended_positions(length, window, sinks=0):
    """Positions a decode query at sequence length ``length`` attends ([KV-opt] §3.2):
    the last ``window`` positions (all of them for window 0) and, with a window, the
    first ``sinks`` positions."""
    if length <= 0:
        raise ValueError("length must be positive")
    if window < 0 or sinks < 0:
        raise ValueError("window and sinks must be non-negative")
    lo = max(0, length - window) if window > 0 else 0
    if window > 0 and sinks > 0:
        return np.concatenate([np.arange(0, min(sinks, lo)), np.arange(lo, length)])
    return np.arange(lo, length)


def recent_fp16_rows(x_hat, x16, lens, recent):
    """Rows a decode step reads when the last ``recent`` positions stay in fp16
    ([INT4-SM] section 8.3): for sequence b, positions ``[max(0, len_b - recent),
    len_b)`` take their fp16 values from ``x16``, older positions their dequantized
    values from ``x_hat``.  x_hat, x16: [B, Hkv, N, D] indexed by position.  Returns
    fp64 [B, Hkv, N, D] (rows at or past len_b copied from x_hat; never attended)."""
    if recent < 0:
        raise ValueError("recent must be non-negative")
    out = np.array(x_hat, dtype=np.float64, copy=True)
    for b, length in enumerate(lens):
        lo = max(0, int(length) - recent)
        out[b, :, lo:int(length)] = np.asarray(x16[b, :, lo:int(length)], dtype=np.float64)
    return out


def decode_attention(q, k_hat, v_hat, lens, window=0, scale=None, sinks=0):
    """out[b, h] = sum_t softmax_t(scale * q[b,h] . k_hat[b,kv,t]) * v_hat[b,kv,t].

    q:      [B, Hq, D] (any float; taken as exact values)
    k_hat:  [B, Hkv, N, D] dequantized keys indexed by *position* (fp64)
    v_hat:  [B, Hkv, N, D] dequantized values indexed by position (fp64)
    lens:   [B] valid lengths (positions 0..len-1, the just-appended one included)
    window: 0 for global attention, else the horizon W
    scale:  softmax scale; None -> 1/sqrt(D)
    sinks:  with a window, the number of leading positions also attended
    Returns fp64 [B, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_hat.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("q heads must be a multiple of kv heads")
    n_rep = Hq // Hkv
    if scale is None:
        scale = D ** -0.5
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        T = attended_positions(int(lens[b]), window, sinks)
        for h in range(Hq):
            kv = h // n_rep
            K = np.asarray(k_hat[b, kv, T], dtype=np.float64)
            V = np.asarray(v_hat[b, kv, T], dtype=np.float64)
            z = scale * (K @ q[b, h])
            e = np.exp(z - z.max())
            p = e / e.sum()
            out[b, h] = p @ V
    return out


def prefill_attention(q, k_hat, v_hat, lens, window=0, scale=None):
    """Chunked-prefill attention: the chunk's nq queries of each sequence, at positions
    [len_b - nq, len_b), each attend causally ([KV-4bit] §1.1: the prefill processes every
    position of the prompt, each seeing the positions up to its own): query i is a decode
    query at length len_b - nq + i + 1 (the same horizon, window and GQA rule).

    q:     [B, Hq, nq, D];  k_hat, v_hat: [B, Hkv, N, D] by position;  lens: [B].
    Returns fp64 [B, Hq, nq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, nq, D = q.shape
    out = np.zeros((B, Hq, nq, D), dtype=np.float64)
    for i in range(nq):
        lens_i = [int(ln) - nq + i + 1 for ln in lens]
        out[:, :, i] = decode_attention(q[:, :, i], k_hat, v_hat, lens_i, window, scale)
    return out
