// api.hip -- the C ABI declared in include/kvq.h: argument validation, size queries,
// split planning and kernel dispatch.  Every check runs before anything is enqueued.
#include <cmath>
#include <cstring>
#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

namespace {

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t check_desc(const kvq_cache_desc* d) {
  if (!d) return KVQ_ERR_ARG;
  if (d->format < KVQ_INT4_G || d->format > KVQ_INT4_G16) return KVQ_ERR_ARG;
  if (d->batch < 1 || d->kv_heads < 1 || d->head_dim < 1 || d->capacity < 1)
    return KVQ_ERR_ARG;
  if (d->sinks < 0 || d->sinks >= d->capacity || d->recent < 0 || d->page_size < 0) return KVQ_ERR_ARG;
  if (d->page_size > 0) {   // paged layout: pages of 16 .. 256 positions, no ring
    if (d->num_pages < 1) return KVQ_ERR_ARG;
    if (!pow2(d->page_size) || d->page_size < 16 || d->page_size > 256 ||
        d->capacity % d->page_size != 0 || d->sinks > 0 || d->recent > 0)
      return KVQ_ERR_UNSUPPORTED;
  }
  // recent fp16 rows: INT4 only, without sinks, at most KVQ_MAX_RECENT
  if (d->recent > 0 && (d->format != KVQ_INT4_G || d->sinks > 0 || d->recent > KVQ_MAX_RECENT))
    return KVQ_ERR_UNSUPPORTED;
  if (d->batch > KVQ_MAX_BATCH) return KVQ_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (d->format == KVQ_INT4_G || d->format == KVQ_INT4_G16) {
    for (int32_t g : {d->group_k, d->group_v}) {
      if (g < 1) return KVQ_ERR_ARG;
      if (!pow2(g) || g < 32 || g > d->head_dim) return KVQ_ERR_UNSUPPORTED;
    }
  }
  // 32-bit lane indexing inside the kernels
  const uint64_t rows = d->page_size > 0
                            ? (uint64_t)d->num_pages * d->kv_heads * d->page_size
                            : (uint64_t)d->batch * d->kv_heads * d->capacity;
  if (rows * (uint64_t)(d->head_dim / 8) >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

bool cache_ok(const kvq_cache_desc* d, const kvq_cache* c) {
  return c && c->k_codes && c->k_scales && c->v_codes && c->v_scales &&
         (d->recent == 0 || (c->k_recent && c->v_recent)) &&
         (d->page_size == 0 || c->block_table);
}

// Rows of each codes / scales buffer: the pool's pages, or B * Hkv * C.
size_t cache_rows(const kvq_cache_desc* d) {
  return d->page_size > 0 ? (size_t)d->num_pages * d->kv_heads * d->page_size
                          : (size_t)d->batch * d->kv_heads * d->capacity;
}

Pages make_pages(const kvq_cache_desc* d, const kvq_cache* c) {
  Pages p;
  std::memset(&p, 0, sizeof(p));
  if (d->page_size > 0) {
    p.table = c->block_table;
    p.size = d->page_size;
    p.shift = __builtin_ctz((unsigned)d->page_size);
    p.pps = d->capacity / d->page_size;
    p.count = d->num_pages;
  }
  return p;
}

int32_t scales_per_row(const kvq_cache_desc* d, int32_t kv) {
  if (d->format == KVQ_INT4_G || d->format == KVQ_INT4_G16)
    return d->head_dim / (kv ? d->group_v : d->group_k);
  return 1;
}

int32_t launch_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

int32_t quant_common(const kvq_cache_desc* desc, const kvq_cache* cache, const void* k,
                     const void* v, const SlotMap& map, int32_t n, hipStream_t stream) {
  QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_codes = cache->k_codes;
  a.k_scales = static_cast<float*>(cache->k_scales);
  a.v_codes = cache->v_codes;
  a.v_scales = static_cast<float*>(cache->v_scales);
  a.B = desc->batch;
  a.Hkv = desc->kv_heads;
  a.D = desc->head_dim;
  a.gk = desc->group_k;
  a.gv = desc->group_v;
  a.rows = desc->batch * desc->kv_heads * n;
  a.map = map;
  a.pages = make_pages(desc, cache);
  if (desc->recent > 0) {
    a.k_recent = static_cast<uint16_t*>(cache->k_recent);
    a.v_recent = static_cast<uint16_t*>(cache->v_recent);
    a.recent = desc->recent;
  }
  if (is_codec(desc->format)) {
    float lv[16];
    codec_codebook(codec_bits(desc->format), lv, a.thr);
    return launch_status(launch_codec_encode(codec_bits(desc->format), a, stream));
  }
  return launch_status(launch_quant_intq(desc->format, a, stream));
}

// Workspace: the split-arrival counters first (KVQ_WS_COUNTER_BYTES, [B, Hkv] uint32,
// zero between calls), then nsplit partial slots per query head (weighted V sums
// [B, Hq, nsplit, D], then (max, sum) pairs [B, Hq, nsplit, 2]).
constexpr size_t partials_offset() { return KVQ_WS_COUNTER_BYTES; }
constexpr int64_t max_units() { return KVQ_WS_COUNTER_BYTES / sizeof(uint32_t); }
size_t partials_bytes(int32_t batch, int32_t q_heads, int32_t ns, int32_t head_dim) {
  return (size_t)batch * q_heads * ns * (head_dim + 2) * sizeof(float);
}

// Positions a decode step at length L attends: L, or with a window W < L the window
// and the sinks before it.
int32_t attended_span(int32_t L, int32_t window, int32_t sinks) {
  if (window <= 0 || window >= L) return L;
  return window + (sinks < L - window ? sinks : L - window);
}

// Longest attended span over the batch; KVQ_ERR_* (negative) if a length is invalid.
int32_t check_lens(const kvq_cache_desc* d, const int32_t* lens, int32_t window) {
  int32_t span = 0;
  for (int32_t b = 0; b < d->batch; ++b) {
    const int32_t L = lens[b];
    if (L < 1) return KVQ_ERR_ARG;
    if (window == 0 || d->page_size > 0) {   // (a paged cache has no ring)
      if (L > d->capacity) return KVQ_ERR_CAPACITY;
    } else if (L > d->capacity && window > d->capacity - d->sinks) {
      return KVQ_ERR_CAPACITY;   // the window's rows would not all be in the ring
    }
    const int32_t s = attended_span(L, window, d->sinks);
    if (s > span) span = s;
  }
  return span;
}

// Positions [start, start + n) map to distinct slots: at most C - S of them at or after S
// (paged: all of them below C).
bool rows_fit(const kvq_cache_desc* d, int32_t start, int32_t n) {
  if (d->page_size > 0) return (int64_t)start + n <= d->capacity;
  const int64_t first_ring = start > d->sinks ? start : d->sinks;
  return (int64_t)start + n - first_ring <= d->capacity - d->sinks;
}

}  // namespace

extern "C" {

int32_t kvq_version(void) { return KVQ_VERSION; }

const char* kvq_status_str(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported shape or format";
    case KVQ_ERR_CAPACITY: return "positions do not fit the cache";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int32_t kvq_check_desc(const kvq_cache_desc* desc) { return check_desc(desc); }

size_t kvq_codes_bytes(const kvq_cache_desc* d, int32_t kv) {
  if (check_desc(d) != KVQ_OK || (kv != 0 && kv != 1)) return 0;
  const size_t rows = cache_rows(d);
  if (d->format == KVQ_INT8_TOKEN) return rows * d->head_dim;
  if (d->format == KVQ_WHT_LM3) return rows * (3 * d->head_dim / 8);
  return rows * (d->head_dim / 2);
}

size_t kvq_scales_bytes(const kvq_cache_desc* d, int32_t kv) {
  if (check_desc(d) != KVQ_OK || (kv != 0 && kv != 1)) return 0;
  const size_t rows = cache_rows(d);
  return rows * scales_per_row(d, kv) * (d->format == KVQ_INT4_G16 ? sizeof(uint16_t) : sizeof(float));
}

size_t kvq_recent_bytes(const kvq_cache_desc* d) {
  if (check_desc(d) != KVQ_OK) return 0;
  return (size_t)d->batch * d->kv_heads * d->recent * d->head_dim * sizeof(uint16_t);
}

int32_t kvq_plan_splits(const kvq_cache_desc* d, int32_t q_heads, int32_t span) {
  if (check_desc(d) != KVQ_OK || q_heads < 1 || q_heads % d->kv_heads || span < 1) return 0;
  return plan_splits(d, q_heads / d->kv_heads, span);
}

size_t kvq_decode_workspace_bytes(const kvq_cache_desc* d, int32_t q_heads, int32_t max_len,
                                  int32_t window, int32_t num_splits) {
  if (check_desc(d) != KVQ_OK || q_heads < 1 || q_heads % d->kv_heads || max_len < 1 ||
      window < 0 || num_splits < 0)
    return 0;
  const int32_t span = attended_span(max_len, window, d->sinks);
  const int32_t ns = num_splits ? num_splits : kvq_plan_splits(d, q_heads, span);
  return partials_offset() + partials_bytes(d->batch, q_heads, ns, d->head_dim);
}

int32_t kvq_codec_codebook(float* levels16, float* thresholds15) {
  if (!levels16 || !thresholds15) return KVQ_ERR_ARG;
  codec_codebook(4, levels16, thresholds15);
  return KVQ_OK;
}

int32_t kvq_codec_codebook_bits(int32_t bits, float* levels, float* thresholds) {
  if (!levels || !thresholds || (bits != 3 && bits != 4)) return KVQ_ERR_ARG;
  float lv[16], th[15];
  codec_codebook(bits, lv, th);
  for (int32_t j = 0; j < (1 << bits); ++j) levels[j] = lv[j];
  for (int32_t j = 0; j + 1 < (1 << bits); ++j) thresholds[j] = th[j];
  return KVQ_OK;
}

int32_t kvq_quantize_prefill(const kvq_cache_desc* desc, const kvq_cache* cache,
                             const void* k_f16, const void* v_f16, int32_t start_pos,
                             int32_t n, kvq_stream stream) {
  const int32_t st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!cache_ok(desc, cache) || !k_f16 || !v_f16 || start_pos < 0 || n < 1) return KVQ_ERR_ARG;
  if (!rows_fit(desc, start_pos, n)) return KVQ_ERR_CAPACITY;
  if ((uint64_t)desc->batch * desc->kv_heads * n * (desc->head_dim / 8) >= (1ull << 31))
    return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)start_pos + n - 1 > INT32_MAX) return KVQ_ERR_ARG;
  SlotMap map;
  std::memset(&map, 0, sizeof(map));
  map.append = 0;
  map.start = start_pos;
  map.n = n;
  map.cap = desc->capacity;
  map.sinks = desc->sinks;
  return quant_common(desc, cache, k_f16, v_f16, map, n, static_cast<hipStream_t>(stream));
}

int32_t kvq_append(const kvq_cache_desc* desc, const kvq_cache* cache, const void* k_f16,
                   const void* v_f16, const int32_t* pos, kvq_stream stream) {
  const int32_t st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!cache_ok(desc, cache) || !k_f16 || !v_f16 || !pos) return KVQ_ERR_ARG;
  SlotMap map;
  std::memset(&map, 0, sizeof(map));
  for (int32_t b = 0; b < desc->batch; ++b) {
    if (pos[b] < 0) return KVQ_ERR_ARG;
    if (desc->page_size > 0 && pos[b] >= desc->capacity) return KVQ_ERR_CAPACITY;
    map.pos[b] = pos[b];
  }
  map.append = 1;
  map.n = 1;
  map.cap = desc->capacity;
  map.sinks = desc->sinks;
  return quant_common(desc, cache, k_f16, v_f16, map, 1, static_cast<hipStream_t>(stream));
}

// ---- the scratch of kvq_append_decode_attn_noalloc: the split counters and partials in
// a static device array (one copy per GPU, held until the process ends) instead of a
// caller workspace.
namespace {

__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag scratch_once[MAX_DEVICES];
void* scratch_addr[MAX_DEVICES];   // the array's device address on each GPU (set once)

__global__ void zero_words(uint32_t* p, int32_t n) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The array's address on the current device, looked up once per device (in host code
// the array's name is only a stand-in; kernels get this address).  The first lookup also
// zeroes the counters with a fill kernel on `stream` (the array starts zeroed when the
// code object loads; this makes that explicit, with no memset node under capture).
void* scratch_on_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::call_once(scratch_once[dev], [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
    const int32_t words = KVQ_WS_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return;
    scratch_addr[dev] = p;
  });
  return scratch_addr[dev];
}

// Workspace argument of decode_common that selects the scratch array.
char scratch_tag;
void* const USE_SCRATCH = &scratch_tag;

}  // namespace

namespace {

// Shared by kvq_decode_attn and kvq_append_decode_attn: validate, then append (when
// k_new is set) and attend.
int32_t decode_common(const kvq_cache_desc* desc, const kvq_cache* cache, const void* k_new,
                      const void* v_new, const void* q_f16, int32_t q_heads,
                      const int32_t* lens, int32_t window, float softmax_scale,
                      int32_t num_splits, float* out, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  const int32_t st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!cache_ok(desc, cache) || !q_f16 || !lens || !out || window < 0 || num_splits < 0 ||
      q_heads < 1 || !std::isfinite(softmax_scale) || softmax_scale < 0.0f)
    return KVQ_ERR_ARG;
  if (q_heads % desc->kv_heads) return KVQ_ERR_ARG;
  const int32_t G = q_heads / desc->kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)desc->batch * desc->kv_heads > max_units()) return KVQ_ERR_UNSUPPORTED;
  const int32_t span = check_lens(desc, lens, window);
  if (span < 0) return span;
  // recent fp16 rows: the INT4 matrix-core kernel only (its splits share them out)
  if (desc->recent > 0 && !mfma_int4_eligible(desc->head_dim, desc->group_k, desc->group_v,
                                              desc->capacity, G))
    return KVQ_ERR_UNSUPPORTED;
  const int32_t ns = num_splits ? num_splits : kvq_plan_splits(desc, q_heads, span);
  if (ns < 1 || ns > MAX_SPLITS) return KVQ_ERR_ARG;
  const size_t need = partials_offset() + partials_bytes(desc->batch, q_heads, ns, desc->head_dim);
  if (workspace == USE_SCRATCH) {   // kvq_append_decode_attn_noalloc, all else checked
    if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
    workspace = scratch_on_current_device(stream);
    if (!workspace) return KVQ_ERR_LAUNCH;
    ws_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16)
    return KVQ_ERR_WORKSPACE;
#ifdef KVQ_TIMELINE
  // the probe build: 32 timestamp slots per workgroup after the partials, when the
  // workspace has room for them
  const size_t tl_off = (need + 255) & ~(size_t)255;
  const size_t tl_bytes = (size_t)ns * desc->kv_heads * desc->batch * 32 * sizeof(uint64_t);
  uint64_t* stamps = ws_bytes >= tl_off + tl_bytes
                         ? reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + tl_off)
                         : nullptr;
#endif

  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k_codes = cache->k_codes;
  a.k_scales = static_cast<const float*>(cache->k_scales);
  a.v_codes = cache->v_codes;
  a.v_scales = static_cast<const float*>(cache->v_scales);
  a.q = static_cast<const uint16_t*>(q_f16);
  a.counters = static_cast<uint32_t*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + partials_offset());
  a.ws_ml = a.ws_acc + (size_t)desc->batch * q_heads * ns * desc->head_dim;
  a.out = out;
  a.B = desc->batch;
  a.Hkv = desc->kv_heads;
  a.Hq = q_heads;
  a.D = desc->head_dim;
  a.cap = desc->capacity;
  a.gk = desc->group_k;
  a.gv = desc->group_v;
  a.window = window;
  a.nsplit = ns;
  a.pages = make_pages(desc, cache);

#ifdef KVQ_TIMELINE
  a.stamps = stamps;
#endif
  a.sinks = desc->sinks;
  if (desc->recent > 0) {
    a.k_recent = static_cast<uint16_t*>(cache->k_recent);
    a.v_recent = static_cast<uint16_t*>(cache->v_recent);
    a.recent = desc->recent;
  }
  const float scale = softmax_scale != 0.0f ? softmax_scale
                                            : 1.0f / std::sqrt((float)desc->head_dim);
  a.qscale = scale * 1.4426950408889634f;  // log2(e): scores in base-2 units
  if (is_codec(desc->format)) codec_codebook(codec_bits(desc->format), a.levels, a.thr);
  for (int32_t b = 0; b < desc->batch; ++b) a.lens[b] = lens[b];

  if (k_new) {
    if (fused_append_supported(desc, G)) {
      a.k_new = static_cast<const uint16_t*>(k_new);
      a.v_new = static_cast<const uint16_t*>(v_new);
    } else {
      // the other kernels attend over the cache only: append first
      SlotMap map;
      std::memset(&map, 0, sizeof(map));
      for (int32_t b = 0; b < desc->batch; ++b) map.pos[b] = lens[b] - 1;
      map.append = 1;
      map.n = 1;
      map.cap = desc->capacity;
      map.sinks = desc->sinks;
      const int32_t r = quant_common(desc, cache, k_new, v_new, map, 1, stream);
      if (r != KVQ_OK) return r;
    }
  }
  return launch_status(launch_decode(desc->format, a, G, stream));
}

}  // namespace

int32_t kvq_decode_attn(const kvq_cache_desc* desc, const kvq_cache* cache, const void* q_f16,
                        int32_t q_heads, const int32_t* lens, int32_t window,
                        float softmax_scale, int32_t num_splits, float* out, void* workspace,
                        size_t ws_bytes, kvq_stream stream) {
  return decode_common(desc, cache, nullptr, nullptr, q_f16, q_heads, lens, window,
                       softmax_scale, num_splits, out, workspace, ws_bytes,
                       static_cast<hipStream_t>(stream));
}

int32_t kvq_append_decode_attn(const kvq_cache_desc* desc, const kvq_cache* cache,
                               const void* k_f16, const void* v_f16, const void* q_f16,
                               int32_t q_heads, const int32_t* lens, int32_t window,
                               float softmax_scale, int32_t num_splits, float* out,
                               void* workspace, size_t ws_bytes, kvq_stream stream) {
  if (!k_f16 || !v_f16) return KVQ_ERR_ARG;
  return decode_common(desc, cache, k_f16, v_f16, q_f16, q_heads, lens, window,
                       softmax_scale, num_splits, out, workspace, ws_bytes,
                       static_cast<hipStream_t>(stream));
}

int32_t kvq_append_decode_attn_noalloc(const kvq_cache_desc* desc, const kvq_cache* cache,
                                       const void* k_f16, const void* v_f16, const void* q_f16,
                                       int32_t q_heads, const int32_t* lens, int32_t window,
                                       float softmax_scale, int32_t num_splits, float* out,
                                       kvq_stream stream) {
  if (!k_f16 || !v_f16) return KVQ_ERR_ARG;
  return decode_common(desc, cache, k_f16, v_f16, q_f16, q_heads, lens, window, softmax_scale,
                       num_splits, out, USE_SCRATCH, 0, static_cast<hipStream_t>(stream));
}

int32_t kvq_prefill_attn(const kvq_cache_desc* desc, const kvq_cache* cache, const void* q_f16,
                         int32_t q_heads, int32_t n_query, const int32_t* lens, int32_t window,
                         float softmax_scale, float* out, kvq_stream stream) {
  const int32_t st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!cache_ok(desc, cache) || !q_f16 || !lens || !out || window < 0 || n_query < 1 ||
      q_heads < 1 || !std::isfinite(softmax_scale) || softmax_scale < 0.0f)
    return KVQ_ERR_ARG;
  if (q_heads % desc->kv_heads) return KVQ_ERR_ARG;
  const int32_t G = q_heads / desc->kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  if ((desc->format != KVQ_INT4_G && desc->format != KVQ_INT4_G16) || desc->head_dim != 128 ||
      desc->group_v != 128 ||
      (desc->group_k != 64 && desc->group_k != 128) || desc->sinks > 0 || desc->recent > 0 ||
      desc->capacity < 32)
    return KVQ_ERR_UNSUPPORTED;
  for (int32_t b = 0; b < desc->batch; ++b) {
    const int32_t L = lens[b];
    if (L < n_query) return KVQ_ERR_ARG;
    if (L > desc->capacity) {   // a window ring must hold every position the chunk attends
      if (desc->page_size > 0 || window == 0 || (int64_t)window + n_query - 1 > desc->capacity)
        return KVQ_ERR_CAPACITY;
    }
  }
  if ((uint64_t)desc->batch * q_heads * n_query * 128 >= (1ull << 31)) return KVQ_ERR_UNSUPPORTED;
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k_codes = cache->k_codes;
  a.k_scales = static_cast<const float*>(cache->k_scales);
  a.v_codes = cache->v_codes;
  a.v_scales = static_cast<const float*>(cache->v_scales);
  a.q = static_cast<const uint16_t*>(q_f16);
  a.out = out;
  a.B = desc->batch;
  a.Hkv = desc->kv_heads;
  a.Hq = q_heads;
  a.D = desc->head_dim;
  a.cap = desc->capacity;
  a.gk = desc->group_k;
  a.gv = desc->group_v;
  a.window = window;
  a.nq = n_query;
  a.pages = make_pages(desc, cache);
  const float scale = softmax_scale != 0.0f ? softmax_scale
                                            : 1.0f / std::sqrt((float)desc->head_dim);
  a.qscale = scale * 1.4426950408889634f;
  for (int32_t b = 0; b < desc->batch; ++b) a.lens[b] = lens[b];
  return launch_status(launch_prefill_int4_mfma(a, G, desc->format == KVQ_INT4_G16, static_cast<hipStream_t>(stream)));
}

int32_t kvq_dequant(const kvq_cache_desc* desc, const kvq_cache* cache, int32_t kv,
                    int32_t start_pos, int32_t n, float* out, kvq_stream stream) {
  const int32_t st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (!cache_ok(desc, cache) || !out || (kv != 0 && kv != 1) || start_pos < 0 || n < 1)
    return KVQ_ERR_ARG;
  if (!rows_fit(desc, start_pos, n)) return KVQ_ERR_CAPACITY;
  if ((uint64_t)desc->batch * desc->kv_heads * n * (desc->head_dim / 8) >= (1ull << 31))
    return KVQ_ERR_UNSUPPORTED;
  DequantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.codes = kv ? cache->v_codes : cache->k_codes;
  a.scales = static_cast<const float*>(kv ? cache->v_scales : cache->k_scales);
  a.out = out;
  a.B = desc->batch;
  a.Hkv = desc->kv_heads;
  a.D = desc->head_dim;
  a.g = kv ? desc->group_v : desc->group_k;
  a.cap = desc->capacity;
  a.start = start_pos;
  a.n = n;
  a.sinks = desc->sinks;
  a.pages = make_pages(desc, cache);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (is_codec(desc->format)) {
    float thr[15];
    codec_codebook(codec_bits(desc->format), a.levels, thr);
    return launch_status(launch_codec_dequant(codec_bits(desc->format), a, s));
  }
  return launch_status(launch_dequant_intq(desc->format, a, s));
}

}  // extern "C"
