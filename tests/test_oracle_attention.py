"""Pins of oracle/attention.py (CPU only): closed forms, invariants, a library routine.

Semantics ([KV-opt] bxzpzcl.cn/news/2871434 §3.2): window [max(0, i-W+1), i],
query head h reads KV head h // (Hq // Hkv), scale head_dim ** -0.5, softmax, P V.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, quant
from oracle.attention import attended_positions, decode_attention, recent_fp16_rows


def _rand(rng, B=2, Hq=4, Hkv=2, N=37, D=16):
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, N, D)) * 2
    v = rng.standard_normal((B, Hkv, N, D))
    return q, k, v


def test_two_position_closed_form():
    # q = (1, 0), scale 1: z = (0, ln 3) -> p = (1/4, 3/4)
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[0.0, 0.0], [math.log(3.0), 5.0]]]])
    v = np.array([[[[4.0, -8.0], [8.0, 4.0]]]])
    o = decode_attention(q, k, v, [2], scale=1.0)
    assert np.allclose(o[0, 0], [0.25 * 4 + 0.75 * 8, 0.25 * -8 + 0.75 * 4], atol=1e-15)


def test_single_position_returns_value_row():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng)
    o = decode_attention(q, k, v, [1, 1])
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h], v[b, h // 2, 0])


def test_zero_query_is_mean_of_window():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng)
    q[:] = 0
    o = decode_attention(q, k, v, [37, 20], window=8)
    assert np.allclose(o[0, 3], v[0, 1, 29:37].mean(0), atol=1e-14)
    assert np.allclose(o[1, 0], v[1, 0, 12:20].mean(0), atol=1e-14)


def test_window_bounds():
    assert list(attended_positions(10, 0)) == list(range(10))
    assert list(attended_positions(10, 4)) == [6, 7, 8, 9]
    assert list(attended_positions(3, 4)) == [0, 1, 2]
    with pytest.raises(ValueError):
        attended_positions(0, 0)
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng)
    # W >= len is global attention; W < len equals global attention over the last W rows
    assert np.allclose(decode_attention(q, k, v, [37, 30], window=37),
                       decode_attention(q, k, v, [37, 30], window=0), atol=1e-14)
    o = decode_attention(q, k, v, [37, 30], window=5)
    o2 = decode_attention(q, k[:, :, 32:37], v[:, :, 32:37], [5, 5])
    assert np.allclose(o[0], o2[0], atol=1e-14)


def test_permutation_invariance_and_gqa_equals_repeated_mha():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng)
    perm = rng.permutation(37)
    o = decode_attention(q, k, v, [37, 37])
    op = decode_attention(q, k[:, :, perm], v[:, :, perm], [37, 37])
    assert np.allclose(o, op, atol=1e-13)
    k_rep = np.repeat(k, 2, axis=1)
    v_rep = np.repeat(v, 2, axis=1)
    assert np.allclose(o, decode_attention(q, k_rep, v_rep, [37, 37]), atol=1e-14)


@pytest.mark.parametrize("lens,window", [([37, 11], 0), ([37, 30], 7), ([5, 37], 40)])
def test_matches_torch_sdpa_fp64(lens, window):
    """torch's scaled_dot_product_attention in float64 on the CPU, fed the window's rows
    with the KV heads expanded by repeat_interleave."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng)
    o = decode_attention(q, k, v, lens, window=window)
    for b, L in enumerate(lens):
        lo = max(0, L - window) if window else 0
        kt = torch.from_numpy(k[b, :, lo:L]).repeat_interleave(2, dim=0)
        vt = torch.from_numpy(v[b, :, lo:L]).repeat_interleave(2, dim=0)
        qt = torch.from_numpy(q[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0]
        assert np.allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_sink_positions():
    """Window plus attention sinks ([KV-opt] section 3.2): the first n_sink positions and
    the last W; contiguous once the window reaches the sinks; window 0 ignores them."""
    assert list(attended_positions(10, 4, sinks=2)) == [0, 1, 6, 7, 8, 9]
    assert list(attended_positions(10, 4, sinks=0)) == [6, 7, 8, 9]
    assert list(attended_positions(7, 4, sinks=4)) == [0, 1, 2, 3, 4, 5, 6]   # lo = 3 < 4
    assert list(attended_positions(3, 4, sinks=2)) == [0, 1, 2]
    assert list(attended_positions(2, 1, sinks=4)) == [0, 1]                  # sinks stop at len
    assert list(attended_positions(10, 0, sinks=3)) == list(range(10))
    with pytest.raises(ValueError):
        attended_positions(5, 2, sinks=-1)


@pytest.mark.parametrize("lens,window,sinks", [([37, 30], 7, 4), ([37, 6], 5, 4), ([9, 37], 3, 12)])
def test_sinks_match_torch_sdpa_with_the_pages_mask(lens, window, sinks):
    """The decode row of the page's mask (window rows [max(0, i - W + 1), i] plus the
    first n_sink columns, i = len - 1, columns limited to the len positions that exist),
    applied by torch's scaled_dot_product_attention in float64 over all positions."""
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng)
    o = decode_attention(q, k, v, lens, window=window, sinks=sinks)
    for b, L in enumerate(lens):
        i = L - 1
        mask = torch.zeros(L, dtype=torch.bool)
        mask[max(0, i - window + 1): i + 1] = True
        mask[:sinks] = True
        kt = torch.from_numpy(k[b, :, :L]).repeat_interleave(2, dim=0)
        vt = torch.from_numpy(v[b, :, :L]).repeat_interleave(2, dim=0)
        qt = torch.from_numpy(q[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None, :])[:, 0]
        assert np.allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-13)


# ---- recent tokens in fp16 ("LLM长上下文推理优化：用INT4状态机管理KV Cache",
# pwwt.cn/news/4219524, section 8.3: older tokens' K/V in INT4, recent ones in FP16)

def _fp16_and_int4(rng, B=2, H=2, N=40, D=64):
    x16 = (rng.standard_normal((B, H, N, D)) * 1.5).astype(np.float16)
    c, s = quant.quantize_int4(x16, 32)
    return x16, quant.dequantize_int4_exact(c, s, 32)


def _sdpa(q, K, V):
    """torch's scaled_dot_product_attention in float64, one query over rows K, V."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


@pytest.mark.parametrize("lens,recent,window", [([40, 17], 8, 0), ([40, 5], 8, 0), ([33, 40], 1, 0),
                                                ([40, 29], 12, 20), ([40, 40], 30, 10)])
def test_recent_rows_match_sdpa_over_the_two_forms(lens, recent, window):
    """The attended rows split at len - R: INT4 dequantized values before, fp16 values
    from there on; torch's attention over exactly those rows, built by slicing."""
    rng = np.random.default_rng(21)
    k16, kh = _fp16_and_int4(rng)
    v16, vh = _fp16_and_int4(rng)
    q = rng.standard_normal((2, 4, 64))
    o = decode_attention(q, recent_fp16_rows(kh, k16, lens, recent),
                         recent_fp16_rows(vh, v16, lens, recent), lens, window=window)
    for b, L in enumerate(lens):
        lo = max(0, L - window) if window else 0
        cut = max(lo, L - recent)
        K = np.concatenate([kh[b, :, lo:cut], k16[b, :, cut:L].astype(np.float64)], axis=1)
        V = np.concatenate([vh[b, :, lo:cut], v16[b, :, cut:L].astype(np.float64)], axis=1)
        for h in range(4):
            assert np.allclose(o[b, h], _sdpa(q[b, h], K[h // 2], V[h // 2]), rtol=1e-12, atol=1e-13)


def test_recent_span_covering_the_sequence_is_plain_fp16_attention():
    rng = np.random.default_rng(22)
    k16, kh = _fp16_and_int4(rng)
    v16, vh = _fp16_and_int4(rng)
    q = rng.standard_normal((2, 4, 64))
    lens = [40, 9]
    o = decode_attention(q, recent_fp16_rows(kh, k16, lens, 64), recent_fp16_rows(vh, v16, lens, 64), lens)
    ref = decode_attention(q, k16.astype(np.float64), v16.astype(np.float64), lens)
    assert np.array_equal(o, ref)
    # and the INT4 form alone differs (the two forms are not the same values)
    assert not np.allclose(o, decode_attention(q, kh, vh, lens))


def test_recent_reads_each_position_from_one_form_only():
    """Planting garbage in the form a position is not read from changes nothing; planting
    it in the form it is read from changes the output."""
    rng = np.random.default_rng(23)
    k16, kh = _fp16_and_int4(rng)
    v16, vh = _fp16_and_int4(rng)
    q = rng.standard_normal((2, 4, 64))
    lens, R = [40, 23], 10
    base = decode_attention(q, recent_fp16_rows(kh, k16, lens, R), recent_fp16_rows(vh, v16, lens, R), lens)
    kh2, k162 = kh.copy(), k16.copy()
    for b, L in enumerate(lens):
        kh2[b, :, L - R:L] = 50.0                      # INT4 form of the recent rows
        k162[b, :, :L - R] = 50.0                      # fp16 form of the older rows
    same = decode_attention(q, recent_fp16_rows(kh2, k162, lens, R), recent_fp16_rows(vh, v16, lens, R), lens)
    assert np.array_equal(base, same)
    k163 = k16.copy()
    k163[1, :, 23 - R] = 50.0                          # the first recent position of sequence 1
    moved = decode_attention(q, recent_fp16_rows(kh, k163, lens, R), recent_fp16_rows(vh, v16, lens, R), lens)
    assert not np.allclose(base[1], moved[1]) and np.array_equal(base[0], moved[0])


def test_prefill_attention_matches_torch_causal_sdpa():
    """The chunk's queries against torch's scaled_dot_product_attention with a causal
    mask aligned to the end of the key range (query i sees keys 0 .. len - nq + i), in
    fp64 on the CPU, for GQA 4:1 (the KV heads repeated per query head) and a window
    (the mask also drops keys before len - nq + i - W + 1)."""
    import torch
    rng = np.random.default_rng(21)
    B, Hkv, G, D, nq = 2, 2, 4, 16, 7
    lens = [40, 29]
    N = max(lens)
    q = rng.standard_normal((B, Hkv * G, nq, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    for W in (0, 9):
        got = attention.prefill_attention(q, k, v, lens, W)
        for b, ln in enumerate(lens):
            kk = torch.from_numpy(k[b:b + 1, :, :ln]).repeat_interleave(G, dim=1)
            vv = torch.from_numpy(v[b:b + 1, :, :ln]).repeat_interleave(G, dim=1)
            pos_q = torch.arange(ln - nq, ln)[:, None]
            pos_k = torch.arange(ln)[None, :]
            mask = pos_k <= pos_q
            if W:
                mask &= pos_k > pos_q - W
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b:b + 1]), kk, vv, attn_mask=mask).numpy()
            assert np.allclose(got[b:b + 1], ref, rtol=1e-12, atol=1e-12), (W, b)


def test_prefill_last_query_is_the_decode_query():
    """The chunk's last query attends exactly like a decode step at the full length; a
    one-token chunk is a decode step."""
    rng = np.random.default_rng(22)
    B, H, D, nq = 2, 3, 8, 5
    lens = [12, 30]
    q = rng.standard_normal((B, H, nq, D))
    k = rng.standard_normal((B, H, 30, D))
    v = rng.standard_normal((B, H, 30, D))
    out = attention.prefill_attention(q, k, v, lens, 6)
    assert np.array_equal(out[:, :, -1], attention.decode_attention(q[:, :, -1], k, v, lens, 6))
    one = attention.prefill_attention(q[:, :, :1], k, v, lens)
    assert np.array_equal(one[:, :, 0], attention.decode_attention(q[:, :, 0], k, v, lens))
    # the first query of a chunk that starts the sequence sees only position 0
    first = attention.prefill_attention(q, k, v, [nq, nq])
    assert np.allclose(first[:, :, 0], v[:, :, 0])
