"""ctypes binding of ``libkvq.so`` (the C ABI in ``include/kvq.h``).

Argument marshalling only: every computation runs in the library's HIP kernels.
Functions carry the C names.  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed; dtype, contiguity and device are checked here) or raw
integer addresses.  ``stream=None`` means torch's current HIP stream on the current
device.  A negative status raises ``KvqError``.

The library is loaded from this package directory; if it has not been built the
import fails loudly: there is no fallback implementation.

torch is imported before the library is opened.  The PyTorch ROCm wheel carries its own
HIP runtime (soname libamdhip64.so.7) that its own libraries request under the name
libamdhip64.so; opening libkvq.so first would load the system runtime under the soname
and torch would then load a second runtime, so the library's launches would go to a
runtime that does not know torch's streams or memory.  With torch loaded first,
libkvq.so's dependency resolves to the runtime torch already uses.
"""
import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL below: one HIP runtime per process)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_INT4_G, KVQ_INT8_TOKEN, KVQ_WHT_LM4, KVQ_WHT_LM3, KVQ_INT4_G16 = 0, 1, 2, 3, 4
FORMATS = {"int4": KVQ_INT4_G, "int8": KVQ_INT8_TOKEN, "codec": KVQ_WHT_LM4, "codec3": KVQ_WHT_LM3,
           "int4h": KVQ_INT4_G16}
KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH = \
    0, -1, -2, -3, -4, -5
KVQ_MAX_BATCH = 256
KVQ_WS_COUNTER_BYTES = 65536
KVQ_MAX_RECENT = 1024
KVQ_NOALLOC_SCRATCH_BYTES = 8 << 20

# Every symbol include/kvq.h declares.
EXPORTS = (
    "kvq_version", "kvq_status_str", "kvq_check_desc", "kvq_codes_bytes", "kvq_scales_bytes",
    "kvq_recent_bytes",
    "kvq_plan_splits", "kvq_decode_workspace_bytes", "kvq_codec_codebook", "kvq_codec_codebook_bits",
    "kvq_quantize_prefill", "kvq_append", "kvq_decode_attn", "kvq_append_decode_attn",
    "kvq_append_decode_attn_noalloc", "kvq_prefill_attn", "kvq_dequant",
)


class kvq_cache_desc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("group_k", ctypes.c_int32),
                ("group_v", ctypes.c_int32), ("sinks", ctypes.c_int32),
                ("recent", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class kvq_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("k_recent", ctypes.c_void_p), ("v_recent", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def _load(path=LIB_PATH):
    """Open the library at `path` (the timeline probe build has the same C ABI)."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m int4_quantized_kv_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    i32, sz, vp, f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    D, C = P(kvq_cache_desc), P(kvq_cache)
    sig = {
        "kvq_version": (i32, []),
        "kvq_status_str": (ctypes.c_char_p, [i32]),
        "kvq_check_desc": (i32, [D]),
        "kvq_codes_bytes": (sz, [D, i32]),
        "kvq_scales_bytes": (sz, [D, i32]),
        "kvq_recent_bytes": (sz, [D]),
        "kvq_plan_splits": (i32, [D, i32, i32]),
        "kvq_decode_workspace_bytes": (sz, [D, i32, i32, i32, i32]),
        "kvq_codec_codebook": (i32, [P(f32), P(f32)]),
        "kvq_codec_codebook_bits": (i32, [i32, P(f32), P(f32)]),
        "kvq_quantize_prefill": (i32, [D, C, vp, vp, i32, i32, vp]),
        "kvq_append": (i32, [D, C, vp, vp, P(i32), vp]),
        "kvq_decode_attn": (i32, [D, C, vp, i32, P(i32), i32, f32, i32, vp, vp, sz, vp]),
        "kvq_append_decode_attn": (i32, [D, C, vp, vp, vp, i32, P(i32), i32, f32, i32, vp, vp,
                                         sz, vp]),
        "kvq_append_decode_attn_noalloc": (i32, [D, C, vp, vp, vp, i32, P(i32), i32, f32, i32, vp,
                                                 vp]),
        "kvq_prefill_attn": (i32, [D, C, vp, i32, i32, P(i32), i32, f32, vp, vp]),
        "kvq_dequant": (i32, [D, C, i32, i32, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


# ----------------------------------------------------------------------------- helpers

def status_str(status):
    return LIB.kvq_status_str(int(status)).decode()


def _check(status, where):
    if status != KVQ_OK:
        raise KvqError(status, where)
    return status


def make_desc(fmt, batch, kv_heads, head_dim, capacity, group_k=64, group_v=128, sinks=0,
              recent=0, page_size=0, num_pages=0):
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return kvq_cache_desc(f, batch, kv_heads, head_dim, capacity, group_k, group_v, sinks, recent,
                          page_size, num_pages)


def _ptr(t, dtype=None, name="tensor"):
    """Device address of a torch tensor (checked) or an int address."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _i32_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return arr


# --------------------------------------------------------------------------- C entry points

def kvq_version():
    return LIB.kvq_version()


def kvq_check_desc(desc):
    return LIB.kvq_check_desc(ctypes.byref(desc))


def kvq_codes_bytes(desc, kv):
    return LIB.kvq_codes_bytes(ctypes.byref(desc), kv)


def kvq_scales_bytes(desc, kv):
    return LIB.kvq_scales_bytes(ctypes.byref(desc), kv)


def kvq_recent_bytes(desc):
    return LIB.kvq_recent_bytes(ctypes.byref(desc))


def kvq_plan_splits(desc, q_heads, span):
    return LIB.kvq_plan_splits(ctypes.byref(desc), q_heads, span)


def kvq_decode_workspace_bytes(desc, q_heads, max_len, window=0, num_splits=0):
    return LIB.kvq_decode_workspace_bytes(ctypes.byref(desc), q_heads, max_len, window, num_splits)


def kvq_codec_codebook():
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(LIB.kvq_codec_codebook(lv, th), "kvq_codec_codebook")
    return list(lv), list(th)


def kvq_codec_codebook_bits(bits):
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(LIB.kvq_codec_codebook_bits(int(bits), lv, th), "kvq_codec_codebook_bits")
    return list(lv)[: 1 << bits], list(th)[: (1 << bits) - 1]


def kvq_quantize_prefill(desc, cache, k, v, start_pos, n, stream=None):
    import torch
    st = LIB.kvq_quantize_prefill(ctypes.byref(desc), ctypes.byref(cache),
                                  _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
                                  int(start_pos), int(n), _stream(stream))
    return _check(st, "kvq_quantize_prefill")


def kvq_append(desc, cache, k, v, pos, stream=None):
    import torch
    st = LIB.kvq_append(ctypes.byref(desc), ctypes.byref(cache), _ptr(k, torch.float16, "k"),
                        _ptr(v, torch.float16, "v"), _i32_array(pos), _stream(stream))
    return _check(st, "kvq_append")


def kvq_decode_attn(desc, cache, q, q_heads, lens, window, softmax_scale, num_splits, out,
                    workspace, ws_bytes=None, stream=None):
    import torch
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.kvq_decode_attn(ctypes.byref(desc), ctypes.byref(cache), _ptr(q, torch.float16, "q"),
                             int(q_heads), _i32_array(lens), int(window), float(softmax_scale),
                             int(num_splits), _ptr(out, torch.float32, "out"),
                             _ptr(workspace, None, "workspace"), int(ws_bytes), _stream(stream))
    return _check(st, "kvq_decode_attn")


def kvq_append_decode_attn(desc, cache, k, v, q, q_heads, lens, window, softmax_scale,
                           num_splits, out, workspace, ws_bytes=None, stream=None):
    import torch
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.kvq_append_decode_attn(
        ctypes.byref(desc), ctypes.byref(cache), _ptr(k, torch.float16, "k"),
        _ptr(v, torch.float16, "v"), _ptr(q, torch.float16, "q"), int(q_heads),
        _i32_array(lens), int(window), float(softmax_scale), int(num_splits),
        _ptr(out, torch.float32, "out"), _ptr(workspace, None, "workspace"), int(ws_bytes),
        _stream(stream))
    return _check(st, "kvq_append_decode_attn")


def kvq_append_decode_attn_noalloc(desc, cache, k, v, q, q_heads, lens, window, softmax_scale,
                                   num_splits, out, stream=None):
    import torch
    st = LIB.kvq_append_decode_attn_noalloc(
        ctypes.byref(desc), ctypes.byref(cache), _ptr(k, torch.float16, "k"),
        _ptr(v, torch.float16, "v"), _ptr(q, torch.float16, "q"), int(q_heads),
        _i32_array(lens), int(window), float(softmax_scale), int(num_splits),
        _ptr(out, torch.float32, "out"), _stream(stream))
    return _check(st, "kvq_append_decode_attn_noalloc")


def kvq_prefill_attn(desc, cache, q, q_heads, n_query, lens, window, softmax_scale, out,
                     stream=None):
    import torch
    st = LIB.kvq_prefill_attn(ctypes.byref(desc), ctypes.byref(cache), _ptr(q, torch.float16, "q"),
                              int(q_heads), int(n_query), _i32_array(lens), int(window),
                              float(softmax_scale), _ptr(out, torch.float32, "out"), _stream(stream))
    return _check(st, "kvq_prefill_attn")


def decode_workspace(desc, q_heads, max_len, window=0, num_splits=0, device="cuda"):
    """A zero-filled decode workspace (the split counters at its start must read zero
    before the first call; the library keeps them zero afterwards)."""
    import torch
    nbytes = kvq_decode_workspace_bytes(desc, q_heads, max_len, window, num_splits)
    if nbytes == 0:
        raise KvqError(KVQ_ERR_ARG, "kvq_decode_workspace_bytes")
    return torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device=device)


def kvq_dequant(desc, cache, kv, start_pos, n, out, stream=None):
    import torch
    st = LIB.kvq_dequant(ctypes.byref(desc), ctypes.byref(cache), int(kv), int(start_pos), int(n),
                         _ptr(out, torch.float32, "out"), _stream(stream))
    return _check(st, "kvq_dequant")


# ------------------------------------------------------------------- device buffers (plumbing)

class DeviceCache:
    """torch-owned device buffers of one layer's cache, sized by the library's own size
    queries, plus the ``kvq_cache`` struct pointing at them.  A paged descriptor
    (page_size > 0) takes its block table, a device int32 tensor [batch, capacity /
    page_size], as ``block_table``."""

    def __init__(self, desc, device="cuda", block_table=None):
        import torch
        self.desc = desc
        nb = [kvq_codes_bytes(desc, 0), kvq_scales_bytes(desc, 0),
              kvq_codes_bytes(desc, 1), kvq_scales_bytes(desc, 1)]
        if min(nb) == 0:
            raise KvqError(kvq_check_desc(desc), "DeviceCache")
        self.k_codes = torch.zeros(nb[0], dtype=torch.uint8, device=device)
        # (fp32 elements covering the byte size: fp16 scales may be an odd count)
        self.k_scales = torch.zeros((nb[1] + 3) // 4, dtype=torch.float32, device=device)
        self.v_codes = torch.zeros(nb[2], dtype=torch.uint8, device=device)
        self.v_scales = torch.zeros((nb[3] + 3) // 4, dtype=torch.float32, device=device)
        # recent fp16 rings (INT4 caches with desc.recent > 0), else absent
        nr = kvq_recent_bytes(desc) // 2
        self.k_recent = torch.zeros(nr, dtype=torch.float16, device=device) if nr else None
        self.v_recent = torch.zeros(nr, dtype=torch.float16, device=device) if nr else None
        if desc.page_size > 0:
            import torch
            if block_table is None or block_table.dtype != torch.int32 or not block_table.is_contiguous():
                raise ValueError("a paged cache needs a contiguous int32 block table")
            if tuple(block_table.shape) != (desc.batch, desc.capacity // desc.page_size):
                raise ValueError("block table must be [batch, capacity / page_size]")
        self.block_table = block_table
        self.c = kvq_cache(self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                           self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                           self.k_recent.data_ptr() if nr else None,
                           self.v_recent.data_ptr() if nr else None,
                           block_table.data_ptr() if block_table is not None else None)

    @property
    def nbytes(self):
        return sum(t.numel() * t.element_size()
                   for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales,
                             self.k_recent, self.v_recent) if t is not None)
