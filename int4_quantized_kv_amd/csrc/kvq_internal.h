// kvq_internal.h -- launch interfaces between the C-ABI layer (api.hip) and the kernel
// translation units.  Not installed; not part of the ABI.
#ifndef KVQ_INTERNAL_H
#define KVQ_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// Where row (b, h, t) of a quantize call lands: slot (start + t) % cap for a prefill,
// slot pos[b] % cap for an append (n == 1).
// Slot of position p in a cache of `cap` slots whose first `sinks` slots hold positions
// 0 .. sinks - 1 and the rest a ring: p below sinks, else sinks + (p - sinks) mod
// (cap - sinks) (p mod cap without sinks).
__host__ __device__ inline int32_t cache_slot(int32_t p, int32_t cap, int32_t sinks) {
  return p < sinks ? p : sinks + (p - sinks) % (cap - sinks);
}

// The paged layout (include/kvq.h): the row of position p of sequence b, kv head h,
// through the block table; an entry outside the pool is clamped into it.
struct Pages {
  const int32_t* table;  // [B, pps] (device), or null: contiguous layout
  int32_t size;          // page size P (a power of two), 0 when contiguous
  int32_t shift;         // log2(P)
  int32_t pps;           // pages per sequence (table row length) = capacity / P
  int32_t count;         // pages in the pool
};
__device__ inline size_t paged_row(const Pages& pg, int32_t Hkv, int32_t b, int32_t h,
                                   int32_t p) {
  const uint32_t id = min((uint32_t)pg.table[(size_t)b * pg.pps + (p >> pg.shift)],
                          (uint32_t)(pg.count - 1));
  return ((size_t)id * Hkv + h) * pg.size + (p & (pg.size - 1));
}

struct SlotMap {
  int32_t append;   // 0: prefill, 1: append
  int32_t start;
  int32_t n;        // rows per (b, h) in the source tensor
  int32_t cap;
  int32_t sinks;    // slots ahead of the ring (cache_slot)
  int32_t pos[KVQ_MAX_BATCH];
};

struct QuantArgs {
  const uint16_t* k;     // fp16 source [B, Hkv, n, D]
  const uint16_t* v;
  void* k_codes;
  float* k_scales;
  void* v_codes;
  float* v_scales;
  int32_t B, Hkv, D, gk, gv;
  int32_t rows;          // B * Hkv * n
  float thr[15];         // codec decision thresholds (codec format only)
  uint16_t* k_recent;    // fp16 rings [B, Hkv, recent, D] (INT4 with recent > 0), else null
  uint16_t* v_recent;
  int32_t recent;
  Pages pages;
  SlotMap map;
};

struct DequantArgs {
  const void* codes;
  const float* scales;
  float* out;            // [B, Hkv, n, D]
  int32_t B, Hkv, D, g, cap, start, n;
  int32_t sinks;         // slots ahead of the ring (cache_slot)
  Pages pages;
  float levels[16];      // codec output levels (codec format only)
};

struct DecodeArgs {
  const void* k_codes;
  const float* k_scales;
  const void* v_codes;
  const float* v_scales;
  const uint16_t* q;     // [B, Hq, D] fp16
  float* ws_acc;         // [B, Hq, nsplit, D]
  float* ws_ml;          // [B, Hq, nsplit, 2] (running max in log2 units, sum)
  float* out;            // [B, Hq, D]
  uint32_t* counters;    // [B, Hkv] split arrival counters (zero between calls)
  const uint16_t* k_new; // [B, Hkv, D] fp16 rows appended at position lens[b] - 1, or null
  const uint16_t* v_new;
  int32_t B, Hkv, Hq, D, cap, gk, gv, window, nsplit;
  int32_t sinks;         // slots ahead of the ring; with a window, positions 0 .. sinks - 1
                         // are attended too (before the window)
  float qscale;          // softmax scale * log2(e)
  float levels[16];      // codec output levels
  float thr[15];         // codec decision thresholds (the fused codec append)
  int32_t merge_inline;  // split-K kernel: the last split of a unit merges (no merge kernel)
  uint16_t* k_recent;    // fp16 rings [B, Hkv, recent, D], position p in row p % recent
  uint16_t* v_recent;    // (INT4 matrix-core kernel with recent > 0), else null
  int32_t recent;        // positions [len - recent, len) are read from the rings (each
                         // split takes a share of them)
  Pages pages;           // paged layout (pages.size > 0), else contiguous [B, Hkv, cap, .]
  int32_t nq;            // chunked prefill: queries per sequence (q [B, Hq, nq, D])
  uint64_t* stamps;      // timeline probe builds only (-DKVQ_TIMELINE): phase timestamps
                         // of each workgroup of the matrix-core kernel, else null
  int32_t lens[KVQ_MAX_BATCH];
};

hipError_t launch_quant_intq(int32_t format, const QuantArgs& a, hipStream_t s);
hipError_t launch_dequant_intq(int32_t format, const DequantArgs& a, hipStream_t s);
hipError_t launch_codec_encode(int32_t bits, const QuantArgs& a, hipStream_t s);
hipError_t launch_codec_dequant(int32_t bits, const DequantArgs& a, hipStream_t s);
// Decode attention.  When the matrix-core kernel applies, the splits are merged inside
// it (a.counters must then point at zeroed counters).  a.k_new / a.v_new, if set, fuse
// the append of position lens[b] - 1 into the INT4 matrix-core kernel and into the
// codec's split-K kernel (see fused_append_supported); the other kernels require the
// append to have been launched separately.
hipError_t launch_decode(int32_t format, const DecodeArgs& a, int32_t q_group, hipStream_t s);

// Split plan of the decode kernels for the cache `d`, `q_group` query heads per KV
// head and a longest attended span of `span` positions (the kernel that will run
// decides the plan, so the workspace query and the launch always agree).
int32_t plan_splits(const kvq_cache_desc* d, int32_t q_group, int32_t span);

// The INT4 matrix-core kernel (decode_mfma.hip) and when it applies.
bool mfma_int4_eligible(int32_t head_dim, int32_t group_k, int32_t group_v, int32_t cap,
                        int32_t q_group);
int32_t plan_splits_mfma(int32_t units, int32_t span);
bool fused_append_supported(const kvq_cache_desc* d, int32_t q_group);
// INT4 with fp16 scales on the matrix-core kernel: its shapes, without sinks
bool mfma_int4h_eligible(const kvq_cache_desc* d, int32_t q_group);
hipError_t launch_decode_int4_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s);
hipError_t launch_decode_int4h_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s);
// Chunked-prefill (multi-query causal) attention over the INT4 cache on the matrix cores
// (head_dim 128, V group 128, K group 64 or 128; fp32 or fp16 scales): a.q [B, Hq, nq, D],
// a.out the same in fp32; no workspace.
hipError_t launch_prefill_int4_mfma(const DecodeArgs& a, int32_t q_group, bool fp16_scales,
                                    hipStream_t s);
// The same kernel for the INT8 per-token format (head_dim 128, capacity >= 16).
bool mfma_int8_eligible(int32_t head_dim, int32_t cap, int32_t q_group);
hipError_t launch_decode_int8_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s);

// Largest split count a decode call accepts (the merge kernel keeps one weight per
// split in LDS).
constexpr int32_t MAX_SPLITS = 1024;

// The library's own Lloyd-Max codebooks of N(0,1) at 4 or 3 bits (computed once, then
// constant): 2^bits levels (the rest 0) and 2^bits - 1 thresholds (the rest +inf, so
// that a count of the thresholds below a value stays below 2^bits).
void codec_codebook(int32_t bits, float levels[16], float thresholds[15]);
inline bool is_codec(int32_t format) { return format == KVQ_WHT_LM4 || format == KVQ_WHT_LM3; }
inline int32_t codec_bits(int32_t format) { return format == KVQ_WHT_LM3 ? 3 : 4; }

}  // namespace kvq

#endif  // KVQ_INTERNAL_H
