"""INT4 KV-cache quantization and INT4 decode attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libkvq.so`` (C ABI: ``include/kvq.h``); this
package is its Python binding.  Importing it fails if the library has not been built
(``python -m int4_quantized_kv_amd.build``): there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    EXPORTS, FORMATS, KVQ_ERR_ARG, KVQ_ERR_CAPACITY, KVQ_ERR_LAUNCH, KVQ_ERR_UNSUPPORTED,
    KVQ_ERR_WORKSPACE, KVQ_INT4_G, KVQ_INT4_G16, KVQ_INT8_TOKEN, KVQ_MAX_BATCH, KVQ_OK, KVQ_WHT_LM3, KVQ_WHT_LM4,
    KVQ_MAX_RECENT, KVQ_NOALLOC_SCRATCH_BYTES, KVQ_WS_COUNTER_BYTES, LIB, LIB_PATH, DeviceCache, KvqError, decode_workspace, kvq_append,
    kvq_append_decode_attn, kvq_append_decode_attn_noalloc, kvq_cache, kvq_cache_desc, kvq_check_desc,
    kvq_codec_codebook, kvq_codec_codebook_bits, kvq_codes_bytes, kvq_decode_attn, kvq_decode_workspace_bytes,
    kvq_dequant, kvq_plan_splits, kvq_prefill_attn, kvq_quantize_prefill, kvq_scales_bytes, kvq_recent_bytes, kvq_version,
    make_desc, status_str,
)
