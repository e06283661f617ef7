/*
 * kvq.h -- C ABI of the MI355X (gfx950) INT4 KV-cache library.
 *
 * The library stores an attention layer's key/value cache in packed low-precision
 * form and runs single-token decode attention directly on the packed data.  All
 * entry points take plain pointers and sizes; no C++ or PyTorch types cross this
 * boundary.
 *
 * Pages the operations follow (cited by title/address and section):
 *   [KV-4bit]  lpnh.cn/news/2042373, article on compressing the KV cache from FP16 to
 *              4 bits.  Section 1.1: the decode loop appends each new token's K/V to a
 *              per-layer cache and attends over all of it.  Section 2.1: group-wise
 *              symmetric INT4, scale = amax/7, an all-zero group gets scale 1,
 *              round then clamp to [-7, 7].  Section 2.2: K groups of 64, V of 128.
 *   [KV-opt]   "AI 推理性能调优：KV Cache 优化与显存管理的工程实践"
 *              (bxzpzcl.cn/news/2871434).  Section 3.1: per-token INT8 variant and the
 *              [batch, heads, seq, head_dim] layout.  Section 3.2: sliding window,
 *              GQA head mapping, softmax scale head_dim^-1/2.
 *   [INT4-SM]  "LLM长上下文推理优化：用INT4状态机管理KV Cache" (pwwt.cn/news/4219524),
 *              section 5 step 5: attention reads the INT4 data and dequantizes it
 *              inside the operator.
 *              Section 8.3, first way to cut memory: INT4 for older tokens' K/V,
 *              FP16 kept for the recent ones.
 *   [LARQL]    "长上下文内存大瘦身：LARQL 四大 KV 缓存引擎原理与横向对比"
 *              (pwwt.cn/news/5725003): window engine (keep only rows inside the
 *              attention horizon) and codec engine (per-head Walsh-Hadamard rotation
 *              plus Lloyd-Max 4-bit codes; head_dim must be a power of two).
 *
 * Conventions shared by every call
 *   - Device pointers point to HIP device memory of the GPU that is current on the
 *     calling thread; host pointers are ordinary CPU memory read before the call
 *     returns.  The caller owns every buffer.  The library allocates nothing,
 *     keeps no pointer after returning and has no mutable global state (it is
 *     re-entrant; calls on different streams touching different buffers may overlap),
 *     with one exception: kvq_append_decode_attn_noalloc uses a scratch array the
 *     library holds on each GPU (see there).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  Nothing synchronizes the host.
 *   - Every argument is validated before any work is enqueued.  On error a negative
 *     kvq_status is returned and nothing has been launched or written.
 *     KVQ_ERR_LAUNCH reports a launch failure seen right after enqueueing.
 *   - fp16 tensors are IEEE binary16 (`_Float16` / torch.float16), row-major,
 *     contiguous, 16-byte aligned.  fp32 outputs are IEEE binary32.
 *
 * Cache layout ([KV-opt] §3.1: [batch, kv_heads, seq, head_dim]) for capacity C:
 *   KVQ_INT4_G    codes  [B, Hkv, C, D/2] uint8: element 2i in the low nibble of byte
 *                        i, element 2i+1 in the high nibble, 4-bit two's complement
 *                        (values -7..7);
 *                 scales [B, Hkv, C, D/g] fp32, g = group_k for K and group_v for V.
 *   KVQ_INT4_G16  as KVQ_INT4_G with fp16 scales [B, Hkv, C, D/g] (4 + 16/g bits per
 *                 element, the 16-bit scale of [KV-4bit] §2.2's accounting).
 *   KVQ_INT8_TOKEN codes [B, Hkv, C, D] int8; scales [B, Hkv, C] fp32.
 *   KVQ_WHT_LM4   codes  [B, Hkv, C, D/2] uint8, unsigned 4-bit Lloyd-Max indices
 *                        (0..15) of the rotated row, same nibble order as INT4;
 *                 scales [B, Hkv, C] fp32 (the row's RMS).
 *   KVQ_WHT_LM3   codes  [B, Hkv, C, 3*D/8] uint8: the 3-bit indices (0..7) packed
 *                        back to back, index i in bits 3i .. 3i+2 of the row read as a
 *                        little-endian bit string;
 *                 scales [B, Hkv, C] fp32, as for KVQ_WHT_LM4.
 *   Position p of a sequence lives in slot p when p < S (S = sinks, the first
 *   positions kept for attention sinks, [KV-opt] §3.2), else in slot
 *   S + (p - S) mod (C - S): a ring of C - S slots (S = 0: slot p mod C).
 * Paged layout ([KV-opt] §3.1 KVCacheManager: the cache handed out in fixed pages of
 * page_size tokens from a pool of max_pages; §4: 16-64 token pages in practice), when
 * page_size = P > 0: every buffer above is a pool of num_pages pages, page n holding P
 * positions of one sequence for every kv head,
 *   codes  [num_pages, Hkv, P, row bytes], scales [num_pages, Hkv, P, D/g (or 1)],
 * and kvq_cache.block_table, device int32 [B, C / P], maps page j of sequence b (its
 * positions jP .. jP + P - 1) to its pool page: position p of sequence b, kv head h is
 * row ((table[b][p / P] * Hkv + h) * P + p mod P).  Capacity C is then the positions a
 * sequence may hold (a multiple of P); there is no ring (every position below C has
 * its own row), and sinks and recent rows are not combined with pages.  Table entries
 * must lie in [0, num_pages): the kernels clamp any other entry into that range, so a
 * wrong entry reads or writes the wrong page rather than outside the pool.
 * Recent fp16 rows ([INT4-SM] §8.3; INT4 caches with recent = R > 0):
 *   k_recent, v_recent  [B, Hkv, R, D] fp16, position p in row p mod R.  Every position
 *   is still quantized into the INT4 buffers when it arrives; the fp16 ring keeps the
 *   last R positions written, and decode reads positions [len - R, len) from it (and
 *   older ones from the INT4 codes).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_VERSION 8
/* Largest batch the decode/append calls accept (per-sequence lengths and positions
 * travel in the kernel argument block). */
#define KVQ_MAX_BATCH 256
/* Bytes at the start of a decode workspace that hold split-arrival counters: one
 * uint32 per (sequence, kv head), so the decode calls take batch * kv_heads <= 16384
 * (KVQ_ERR_UNSUPPORTED otherwise).  They must read zero when a decode call starts;
 * every decode call leaves them zero again. */
#define KVQ_WS_COUNTER_BYTES 65536
/* Largest recent fp16 span (kvq_cache_desc.recent). */
#define KVQ_MAX_RECENT 1024
/* Bytes of the per-GPU scratch array behind kvq_append_decode_attn_noalloc (its split
 * counters and partials; the same layout as a decode workspace). */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)

typedef enum {
  KVQ_INT4_G = 0,      /* group-wise symmetric INT4 ([KV-4bit] §2.1) */
  KVQ_INT8_TOKEN = 1,  /* per-token symmetric INT8 ([KV-opt] §3.1) */
  KVQ_WHT_LM4 = 2,     /* Walsh-Hadamard rotation + 4-bit Lloyd-Max codec ([LARQL]) */
  KVQ_WHT_LM3 = 3,     /* the same codec at 3 bits ([LARQL]: 3 or 4 bits) */
  KVQ_INT4_G16 = 4     /* group-wise INT4 with fp16 scales ([KV-4bit] §2.1 in fp16) */
} kvq_format;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,          /* null pointer, non-positive size, bad kv selector, len 0 */
  KVQ_ERR_UNSUPPORTED = -2,  /* shape the kernels do not implement (see kvq_check_desc) */
  KVQ_ERR_CAPACITY = -3,     /* positions that do not fit the cache / window */
  KVQ_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required */
  KVQ_ERR_LAUNCH = -5        /* the HIP runtime reported an error when enqueueing */
} kvq_status;

/* Shape and format of one layer's cache. */
typedef struct {
  int32_t format;    /* kvq_format */
  int32_t batch;     /* B, 1..KVQ_MAX_BATCH */
  int32_t kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;  /* D: 64, 128 or 256 */
  int32_t capacity;  /* C: slots per (b, kv head) >= 1 */
  int32_t group_k;   /* INT4 formats: K group size (default 64); power of two, 32 <= g <= D */
  int32_t group_v;   /* INT4 only: V group size (default 128); same rule */
  int32_t sinks;     /* S: leading positions kept outside the ring, 0 <= S < C (0: none) */
  int32_t recent;    /* R: last positions also kept in fp16 and read from there at
                        decode, 0 <= R <= KVQ_MAX_RECENT (0: none).  INT4 format and
                        S = 0 only (KVQ_ERR_UNSUPPORTED otherwise). */
  int32_t page_size; /* P: 0 = contiguous [B, Hkv, C, .] buffers; else the paged layout
                        (a power of two, 16 <= P <= 256, C % P == 0, S = R = 0;
                        KVQ_ERR_UNSUPPORTED otherwise) */
  int32_t num_pages; /* paged layout: pages in the pool (>= 1); ignored when P = 0 */
} kvq_cache_desc;

/* Device pointers of one layer's cache (layout above). */
typedef struct {
  void* k_codes;
  void* k_scales;
  void* v_codes;
  void* v_scales;
  void* k_recent;    /* R > 0: [B, Hkv, R, D] fp16 rings (kvq_recent_bytes each); */
  void* v_recent;    /*        R = 0: ignored */
  const int32_t* block_table;   /* P > 0: device int32 [B, C / P] (paged layout above);
                                   P = 0: ignored */
} kvq_cache;

/* A hipStream_t, passed as an opaque pointer; NULL is the null stream. */
typedef void* kvq_stream;

/* KVQ_VERSION of the built library. */
int32_t kvq_version(void);

/* Static, human-readable name of a kvq_status value ("unknown status" otherwise). */
const char* kvq_status_str(int32_t status);

/* Validate a descriptor without touching the GPU.  Returns KVQ_OK, KVQ_ERR_ARG (null,
 * non-positive sizes, unknown format) or KVQ_ERR_UNSUPPORTED (D not in {64,128,256};
 * INT4 group not a power of two in [32, D]; batch > KVQ_MAX_BATCH). */
int32_t kvq_check_desc(const kvq_cache_desc* desc);

/* Bytes of the codes (or scales) buffer of K (kv = 0) or V (kv = 1) for `desc`;
 * 0 if the descriptor is invalid or kv is not 0/1.  INT4: B*Hkv*C*D/2 and
 * B*Hkv*C*(D/g)*4 (fp16 scales: *2); INT8: B*Hkv*C*D and B*Hkv*C*4; codec: B*Hkv*C*D/2 (3-bit:
 * B*Hkv*C*3D/8) and B*Hkv*C*4.  Paged layout: num_pages*P in place of B*C. */
size_t kvq_codes_bytes(const kvq_cache_desc* desc, int32_t kv);
size_t kvq_scales_bytes(const kvq_cache_desc* desc, int32_t kv);
/* Bytes of each recent fp16 ring (K and V alike): B*Hkv*R*D*2; 0 if the descriptor is
 * invalid or R = 0. */
size_t kvq_recent_bytes(const kvq_cache_desc* desc);

/* Number of sequence splits kvq_decode_attn uses when called with num_splits = 0 for
 * a longest attended span of `span` positions and `q_heads` query heads; 0 if invalid. */
int32_t kvq_plan_splits(const kvq_cache_desc* desc, int32_t q_heads, int32_t span);

/* Workspace bytes kvq_decode_attn / kvq_append_decode_attn need for these arguments
 * (num_splits = 0: the library's own plan for the longest attended span at max_len:
 * max_len, or window + min(S, max_len - window) when 0 < window < max_len); 0 if
 * invalid.  Equal to KVQ_WS_COUNTER_BYTES + B * q_heads * nsplit *
 * (D + 2) * 4. */
size_t kvq_decode_workspace_bytes(const kvq_cache_desc* desc, int32_t q_heads,
                                  int32_t max_len, int32_t window, int32_t num_splits);

/* The library's own 4-bit Lloyd-Max quantizer of a unit Gaussian ([LARQL] codec):
 * 16 ascending output levels and the 15 midpoint decision thresholds, rounded to
 * fp32 from a double-precision fixed-point iteration.  Host pointers.  KVQ_ERR_ARG on
 * null. */
int32_t kvq_codec_codebook(float* levels16, float* thresholds15);

/* The same at `bits` = 3 or 4: 2^bits levels and 2^bits - 1 thresholds into the host
 * arrays.  KVQ_ERR_ARG on null or another bit count. */
int32_t kvq_codec_codebook_bits(int32_t bits, float* levels, float* thresholds);

/* Bulk quantize `n` consecutive positions [start_pos, start_pos + n) of every
 * (b, kv head) into the cache ([KV-4bit] §2.1 applied to the prefill rows).
 *   k_f16, v_f16: device, [B, Hkv, n, D] fp16 contiguous (the prompt's K and V).
 *   Position p goes to its slot (layout above).  Requires 0 <= start_pos, n >= 1 and
 *   at most C - S of the positions at or after S (KVQ_ERR_CAPACITY otherwise: more
 *   rows than ring slots would overwrite each other within one call).
 * INT4: per group, s = fl32(amax/7) (1 if 0), code = clamp(rne(fl32(x/s)), -7, 7).
 * INT4 with fp16 scales: s = fl16(amax/7) (1 if 0), code = clamp(rne(fl16(x/s)), -7, 7).
 * INT8: s = max(fl32(amax/127), 1e-8), code = clamp(rne(fl32(x/s)), -128, 127).
 * Codec: y = H x / sqrt(D), s = ||x||_2 / sqrt(D), index = #{thresholds < y/s}.
 * With recent fp16 rows (R > 0) the positions among the call's last R,
 * [start_pos + n - R, start_pos + n), are also copied unchanged into the fp16 rings. */
int32_t kvq_quantize_prefill(const kvq_cache_desc* desc, const kvq_cache* cache,
                             const void* k_f16, const void* v_f16,
                             int32_t start_pos, int32_t n, kvq_stream stream);

/* Quantize one new token's K/V row per (b, kv head) into the slot of position pos[b]
 * ([KV-4bit] §1.1 decode step: append the new token's K/V to the cache).
 *   k_f16, v_f16: device, [B, Hkv, D] fp16 contiguous.
 *   pos: host, [B] positions, each >= 0.
 * Same arithmetic as kvq_quantize_prefill; with R > 0 the fp16 rows also go to ring row
 * pos[b] mod R. */
int32_t kvq_append(const kvq_cache_desc* desc, const kvq_cache* cache,
                   const void* k_f16, const void* v_f16, const int32_t* pos,
                   kvq_stream stream);

/* Single-token decode attention reading the packed cache, dequantizing in registers
 * ([INT4-SM] §5 step 5; semantics of [KV-opt] §3.2):
 *   out[b, h] = sum_t softmax_t(scale * q[b,h] . x_K[b,kv,t]) * x_V[b,kv,t]
 * with kv = h / (q_heads / Hkv) (GQA), t over [max(0, len_b - window), len_b) and,
 * with a window, the attention sinks [0, min(S, len_b - window)) as well (window = 0:
 * [0, len_b)), x = the dequantized cache values; with R > 0, x = the fp16 ring rows for
 * t >= len_b - R (so they must hold the last R positions written).
 *   q_f16: device, [B, q_heads, D] fp16.  q_heads must be a multiple of Hkv with
 *          q_heads / Hkv in {1, 2, 4, 8}.
 *   lens: host, [B], 1 <= len_b; positions 0..len_b-1 must be in the cache
 *         (len_b <= C, or window in 1..C - S when len_b > C; KVQ_ERR_CAPACITY
 *         otherwise).
 *   softmax_scale: > 0, or 0 to select 1/sqrt(D); negative values are rejected.
 *   num_splits: sequence splits per (b, kv head), at most 1024; 0 = kvq_plan_splits.
 *   out: device, [B, q_heads, D] fp32.
 *   workspace: device scratch of at least kvq_decode_workspace_bytes bytes, 16-byte
 *              aligned (KVQ_ERR_WORKSPACE otherwise).  Zero-fill it once before its first use
 *              (hipMemset of the whole buffer, or of its first KVQ_WS_COUNTER_BYTES):
 *              the counters there must read zero when a call starts, and each call
 *              leaves them zero; the rest is clobbered.  Calls that may run at the same
 *              time need separate workspaces.
 * Split-K: each split writes an unnormalized partial (running max, sum, weighted V) to
 * the workspace; the partials are merged with the log-sum-exp rule by the last split to
 * finish (no second launch) on the matrix-core kernels (INT4, with fp32 or fp16 scales,
 * at head_dim 128 and V group 128, fp16 scales without sinks; INT8 with head_dim 128)
 * and, up to 32 splits, on the split-K kernel (every other case); above that by a second
 * kernel.  R > 0 runs on the INT4 matrix-core kernel
 * only (KVQ_ERR_UNSUPPORTED for other shapes), whose splits each attend a share of the
 * fp16 rows besides their share of the codes. */
int32_t kvq_decode_attn(const kvq_cache_desc* desc, const kvq_cache* cache,
                        const void* q_f16, int32_t q_heads, const int32_t* lens,
                        int32_t window, float softmax_scale, int32_t num_splits,
                        float* out, void* workspace, size_t ws_bytes, kvq_stream stream);

/* One whole decode step of a layer ([KV-4bit] §1.1: append the new token's K/V, then
 * attend over the cache including it): the same result as kvq_append with
 * pos[b] = lens[b] - 1 followed by kvq_decode_attn with the same arguments.
 *   k_f16, v_f16: device, [B, Hkv, D] fp16, the new token's rows (position lens[b] - 1).
 * Every other argument, the workspace rule and the errors are those of kvq_decode_attn
 * (KVQ_ERR_ARG also for null k_f16 / v_f16).  On the INT4 matrix-core kernel (head_dim
 * 128, V group 128, either scale type), for the codecs and for INT4 with fp16 scales at
 * other shapes, the new row is quantized inside the attention kernel, which writes it
 * to the cache (and, with R > 0, its fp16 row to the ring) and adds it to the softmax
 * without reading it back (one launch per step); the other cases (INT8) run the append
 * kernel first. */
int32_t kvq_append_decode_attn(const kvq_cache_desc* desc, const kvq_cache* cache,
                               const void* k_f16, const void* v_f16, const void* q_f16,
                               int32_t q_heads, const int32_t* lens, int32_t window,
                               float softmax_scale, int32_t num_splits, float* out,
                               void* workspace, size_t ws_bytes, kvq_stream stream);

/* kvq_append_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step, arguments, result and errors, without the workspace arguments.  The split
 * counters and partials live instead in a scratch array of KVQ_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends (a static
 * device array; nothing is allocated, by this call or any other).
 *   - KVQ_ERR_WORKSPACE, before any launch, when the call needs more than the array
 *     holds: kvq_decode_workspace_bytes(desc, q_heads, max(lens), window, num_splits)
 *     > KVQ_NOALLOC_SCRATCH_BYTES.
 *   - Every call on a GPU shares that GPU's array, and each leaves its counters zero:
 *     calls that may overlap in time on one GPU (other streams, concurrent graph
 *     replays) race on it and give wrong results.  Serialize them (one stream).
 *   - The first call on a device looks the array's address up once
 *     (hipGetSymbolAddress; KVQ_ERR_LAUNCH if that fails) and enqueues a small kernel
 *     on `stream` that zeroes the counters. */
int32_t kvq_append_decode_attn_noalloc(const kvq_cache_desc* desc, const kvq_cache* cache,
                                       const void* k_f16, const void* v_f16, const void* q_f16,
                                       int32_t q_heads, const int32_t* lens, int32_t window,
                                       float softmax_scale, int32_t num_splits, float* out,
                                       kvq_stream stream);

/* Chunked-prefill attention over the packed cache ([KV-4bit] §1.1: the prefill computes
 * every position of the prompt at once, where decode computes one): n_query tokens per
 * sequence, at positions [len_b - n_query, len_b), whose K/V rows are already in the
 * cache (kvq_quantize_prefill of the chunk), attend causally:
 *   out[b, h, i] = sum_t softmax_t(scale * q[b,h,i] . x_K[b,kv,t]) * x_V[b,kv,t],
 *   t over [lo, len_b - n_query + i], lo = max(0, len_b - n_query + i - window + 1) with
 *   a window (window > 0), else 0; kv = h / (q_heads / Hkv); x = dequantized values.
 *   q_f16: device, [B, q_heads, n_query, D] fp16; out: device, [B, q_heads, n_query, D]
 *   fp32.  lens: host, [B], n_query <= len_b; len_b <= C, or (a window ring, contiguous
 *   layout) window > 0 and window + n_query - 1 <= C - S.  softmax_scale as in
 *   kvq_decode_attn.
 * INT4 formats (fp32 or fp16 scales) with head_dim 128, V group 128 and K group 64 or
 * 128, q_heads / Hkv in {1, 2, 4, 8}, no sinks or recent rows (KVQ_ERR_UNSUPPORTED
 * otherwise); contiguous or paged.  Runs on the matrix cores; needs no workspace. */
int32_t kvq_prefill_attn(const kvq_cache_desc* desc, const kvq_cache* cache, const void* q_f16,
                         int32_t q_heads, int32_t n_query, const int32_t* lens, int32_t window,
                         float softmax_scale, float* out, kvq_stream stream);

/* Dequantize positions [start_pos, start_pos + n) of K (kv = 0) or V (kv = 1)
 * ([KV-4bit] §2.1 dequantize_4bit_group: code * scale; codec: s * H c[idx] / sqrt(D)).
 *   out: device, [B, Hkv, n, D] fp32.  Requires start_pos >= 0, n >= 1 and at most C - S
 *   of the positions at or after S (the rows must be distinct slots).  Reads the INT4
 *   codes also where recent fp16 rows exist. */
int32_t kvq_dequant(const kvq_cache_desc* desc, const kvq_cache* cache, int32_t kv,
                    int32_t start_pos, int32_t n, float* out, kvq_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
