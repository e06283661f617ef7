"""kvq_append_decode_attn_noalloc: the decode step for callers that cannot allocate.

The call keeps its split counters and partials in the library's per-GPU scratch array
instead of a caller workspace.  Checked through the C ABI against kvq_append_decode_attn
(the same step with a workspace) on identically prefilled caches: the output within the
attention bar (max abs 2e-3, relative L2 1e-4), the cache bytes equal, on consecutive
calls that reuse the array, each later one smaller than the one before (the array keeps
the previous call's partials, and its counters must be back at zero).  Paths: the INT4
matrix-core kernel (splits merged in-kernel) and the codec's split-K kernel (in-kernel
merge, then the merge kernel).
"""
import ctypes

import pytest
import torch

import int4_quantized_kv_amd as kvq
import synth
from tests.kvq_testutil import assert_attn_close

pytestmark = pytest.mark.gpu
DEV = "cuda"

STEPS = [
    # fmt, D, G, batch, Hkv, lens, window, num_splits
    ("int4", 128, 4, 8, 8, [8193] * 8, 0, 0),      # the Llama-3-8B-shaped layer, 4 splits
    ("int4", 128, 4, 2, 2, [700, 513], 0, 7),      # smaller, more splits per unit
    ("int4", 128, 2, 1, 2, [300], 128, 0),         # smaller still, a window
    ("codec", 256, 2, 2, 2, [1500, 900], 0, 40),   # split-K + merge kernel
    ("codec", 256, 2, 1, 2, [600], 0, 0),          # smaller, in-kernel merge
]


def _caches(fmt, B, Hkv, D, L, k, v):
    desc = kvq.make_desc(fmt, B, Hkv, D, L, min(64, D), min(128, D))
    out = []
    for _ in range(2):
        dc = kvq.DeviceCache(desc, DEV)
        kvq.kvq_quantize_prefill(desc, dc.c, k[:, :, :L - 1].contiguous(), v[:, :, :L - 1].contiguous(),
                                 0, L - 1)
        out.append(dc)
    return desc, out


def test_noalloc_step_equals_workspace_step():
    for i, (fmt, D, G, B, Hkv, lens, W, ns) in enumerate(STEPS):
        print(f"[noalloc] step {i}: {fmt} D={D} G={G} B={B} Hkv={Hkv} lens={lens} W={W} ns={ns}",
              flush=True)
        L = max(lens)
        k = synth.kv_source((B, Hkv, L, D), 2100 + i, DEV, outlier_channels=2)
        v = synth.kv_source((B, Hkv, L, D), 2200 + i, DEV, outlier_channels=2)
        q = synth.query((B, Hkv * G, D), 2300 + i, DEV)
        desc, (dws, dna) = _caches(fmt, B, Hkv, D, L, k, v)
        idx = torch.tensor([ln - 1 for ln in lens], device=DEV)
        ar = torch.arange(B, device=DEV)
        kn, vn = k[ar, :, idx].contiguous(), v[ar, :, idx].contiguous()
        Hq = Hkv * G
        ws = kvq.decode_workspace(desc, Hq, L, W, ns, DEV)
        ref = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        kvq.kvq_append_decode_attn(desc, dws.c, kn, vn, q, Hq, lens, W, 0.0, ns, ref, ws)
        # through the C ABI directly (plain pointers, the current stream)
        lens_c = (ctypes.c_int32 * B)(*lens)
        st = kvq.LIB.kvq_append_decode_attn_noalloc(
            ctypes.byref(desc), ctypes.byref(dna.c), kn.data_ptr(), vn.data_ptr(), q.data_ptr(), Hq,
            lens_c, W, 0.0, ns, got.data_ptr(),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == kvq.KVQ_OK, kvq.status_str(st)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all(), f"step {i}: an output was not written"
        assert_attn_close(got.cpu().numpy(), ref.cpu().numpy().astype("float64"), f"noalloc step {i}")
        for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
            assert torch.equal(getattr(dws, name), getattr(dna, name)), (i, name)


def test_noalloc_rejects_calls_beyond_the_scratch():
    desc = kvq.make_desc("int4", 64, 8, 128, 64)
    need = kvq.kvq_decode_workspace_bytes(desc, 64, 64, 0, 8)
    assert need > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append_decode_attn_noalloc(desc, kvq.kvq_cache(1, 1, 1, 1), 16, 16, 16, 64, [64] * 64,
                                           0, 0.0, 8, 16)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
