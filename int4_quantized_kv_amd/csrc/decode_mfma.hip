// decode_mfma.hip -- split-K decode attention over the packed cache on the gfx950 matrix
// cores, for head_dim 128 and GQA groups of 1, 2, 4 or 8 query heads per KV head: the
// INT4 format with one V scale per row (V group 128) and any K group that is a multiple
// of 32, and the INT8 per-token format (see "INT8 per-token tiles").
//
// Semantics as decode.hip (bxzpzcl.cn/news/2871434 section 3.2; lpnh.cn/news/2042373
// sections 1.1 and 2.1; in-operator dequantization, pwwt.cn/news/4219524 section 5).
//
// Why MFMA: one decode step reads every cached position once; with the G query heads
// of a KV head sharing that read, q.K and P.V are G x 128 contractions per position.
// Done with fp32 FMAs they cost ~8 VALU ops per cached byte, above what the vector ALUs
// sustain at HBM speed (~5 per byte), so both contractions go to the matrix cores and
// the VALU only unpacks codes and runs the softmax.
//
// INT4, per wave, per tile of 32 positions (two 16-position halves T = 0, 1):
//   q.K   A = K codes (rows = 16 positions, k = 32 head dims), B = q, v_mfma_f32_16x16x32_f16.
//         The K group scale differs per group, so the 16 B columns are (query head,
//         K group) pairs: column head * NGK + g carries q only in the k slots of dims in
//         group g.  Each column's result is scaled by its group's scale and the NGK
//         adjacent columns are summed with a lane shuffle: z = sum_g sK[t, g] (q . codes_g).
//         With at most 8 columns in use, the other 8 score the second half of the tile
//         in the same MFMAs (see "Position sets").
//   P.V   computed transposed: A = V codes (rows = 16 head dims, k = 32 positions),
//         B = P (k = positions, columns = heads).  Lane (r, j) loads dword r of the 8
//         positions {4j..4j+3, 16+4j..16+4j+3} whose scores it already holds from q.K, so
//         P needs no data movement.  MFMA e (e = 0..7) covers dims {8r + e}.  The V row
//         scale is folded into P (p' = p * sV[t]); p' is split into fp16 hi + lo, which
//         ride in a head's two columns of one MFMA, so P.V keeps ~22 bits (fp16 P alone
//         would lose ~1e-4).
// Codes become exact MFMA operands: K nibbles as biased fp16 subnormals (the bias is
// removed after the MFMA), V nibbles as fp16 integers via the 1024 exponent bias and a
// packed subtract (see v_pair_f16 and unpack_word_u).
// The online softmax keeps the running maximum of the unscaled scores and forms
// p = 2^(s * (z - m)) with s = softmax scale * log2 e (one fma + exp per score); it
// rescales the accumulators only when some head's running maximum grows.
// The eight waves of a workgroup (one per CU) claim tiles of the split from an LDS
// counter and merge their (max, sum, weighted V) through LDS; the workgroup that
// finishes last for a (sequence, KV head) then combines the splits' partials (no
// separate merge launch).  Tiles are staged through LDS by direct global->LDS
// transfers (see "LDS staging").
#include <cmath>
#include <type_traits>

#include "kvq_arith.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float NEG_INF = -__builtin_huge_valf();
// Initial running maximum: finite and below every score (|q . k| < 128 * 65504^2 for fp16
// q and K values), so a column that sees only masked positions keeps p = 2^-inf = 0,
// a zero sum and zero accumulators (with -inf it would form 2^(-inf + inf) = NaN), and
// enters the combine with weight 0.  Raised for very large softmax scales so that
// M_EMPTY * scale stays finite.
constexpr float M_EMPTY = -1.0e30f;
__device__ __forceinline__ float empty_max(float qscale) { return fmaxf(M_EMPTY, -1.0e37f / qscale); }
constexpr int HD = 128;     // head_dim of this kernel
constexpr int TILE = 32;    // positions per wave iteration
constexpr int WAVES = 8;    // one workgroup per CU (see the tile schedule below)
constexpr int NT = WAVES * 64;

union H8 {
  half8 h;
  uint32_t u[4];
};

// Nibble pairs -> MFMA operands.  A dword holds two 16-bit halves of four
// two's-complement nibbles each (nibble p at bits 4p .. 4p+3 of a half).  Nibbles 0 and
// 1 of both halves are taken in place and nibbles 2 and 3 after one shift by 8, so each
// dword costs one shift.  A nibble taken at bits 4..7 lands in the fp16 encoding 16
// times larger than one at bits 0..3; the caller compensates with exact powers of two
// (q scaled by 1/16 in those MFMA slots for K, the V accumulators of those dims by
// 1/16 at the end).  In every bitop3, the immediate 0x6A is the truth table
// f(0xF0, 0xCC, 0xAA) of f(a, b, c) = (a & b) ^ c: keep the nibble, flip its sign bit
// (u = q + 8) and set the bits of c outside the nibble.

// V: (1024 + u) or (1024 + 16 u) as fp16 (exponent bits set by c), then a packed
// subtract of 1032 (or 1152) leaves q (or 16 q) exactly.
__device__ __forceinline__ uint32_t pk_sub_f16(uint32_t x, float k) {
  f16x2 v = __builtin_bit_cast(f16x2, x);
  const f16x2 kk = {(_Float16)k, (_Float16)k};
  v = v - kk;
  return __builtin_bit_cast(uint32_t, v);
}
template <int P>   // nibble P (0..3) of both halves of x
__device__ __forceinline__ uint32_t v_pair_f16(uint32_t x, uint32_t x8) {
  if (P == 0) return pk_sub_f16(__builtin_amdgcn_bitop3_b32(x, 0x000F000Fu, 0x64086408u, 0x6A), 1032.0f);
  if (P == 1) return pk_sub_f16(__builtin_amdgcn_bitop3_b32(x, 0x00F000F0u, 0x64806480u, 0x6A), 1152.0f);
  if (P == 2) return pk_sub_f16(__builtin_amdgcn_bitop3_b32(x8, 0x000F000Fu, 0x64086408u, 0x6A), 1032.0f);
  return pk_sub_f16(__builtin_amdgcn_bitop3_b32(x8, 0x00F000F0u, 0x64806480u, 0x6A), 1152.0f);
}

// K: the eight nibbles of `w` as fp16 subnormals u * 2^-24 (slots 0, 1, 4, 5) or
// 16 u * 2^-24 (slots 2, 3, 6, 7), which the matrix cores take exactly; slot 2p holds
// nibble p of the low half, slot 2p + 1 nibble p of the high half.  The + 8 offset is
// removed after the MFMA: sum q_k (u_k - 8) = 2^24 C - 8 sum q_k.
__device__ __forceinline__ half8 unpack_word_u(uint32_t w) {
  H8 r;
  const uint32_t w8 = w >> 8;
  r.u[0] = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x00080008u, 0x6A);
  r.u[1] = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x00800080u, 0x6A);
  r.u[2] = __builtin_amdgcn_bitop3_b32(w8, 0x000F000Fu, 0x00080008u, 0x6A);
  r.u[3] = __builtin_amdgcn_bitop3_b32(w8, 0x00F000F0u, 0x00800080u, 0x6A);
  return r.h;
}

// Max / sum over the 4 lanes j (lane, lane ^ 16, lane ^ 32, lane ^ 48) that share a
// column, with the gfx950 row-swap permutes (VALU, no LDS round trip).  Swapping a
// register with a copy of itself leaves [r0, r0, r2, r2] / [r1, r1, r3, r3] (16-lane
// rows) for v_permlane16_swap and [r0, r1, r0, r1] / [r2, r3, r2, r3] for
// v_permlane32_swap.  The swaps are written as inline assembly with both registers
// read-write (the compiler builtin returns its first result for both elements of the
// pair); the s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Maxima of scores and scales, none of which is ever NaN: the hardware max, one
// instruction (fmaxf also quiets signalling NaNs first, an extra max of each operand
// with itself).
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_over_j(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  uint32_t c = __builtin_bit_cast(uint32_t, max_raw(__builtin_bit_cast(float, a),
                                                    __builtin_bit_cast(float, b)));
  uint32_t d = c;
  swap32(c, d);
  return max_raw(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
__device__ __forceinline__ float sum_over_j(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) +
                                                __builtin_bit_cast(float, b));
  uint32_t d = c;
  swap32(c, d);
  return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(1))) void* gbl_vptr;

// ---------------------------------------------------------------------------------------
// LDS staging.  Each wave owns a ring of NB tile slots and keeps NB - 1 tiles in flight:
// tiles arrive by direct HBM -> LDS transfers (buffer loads into LDS for full tiles,
// global_load_lds otherwise) that do not pass through VGPRs, so the prefetch depth does
// not cost registers.  The decode kernel keeps one tile in flight behind the one being
// processed (8 per CU, ~9 MB over the chip): the same transfers with no arithmetic
// stream equally fast at one, two or three tiles per wave, and with the arithmetic one
// is the fastest (Llama-3-8B step 2-3% faster than two, which was 3-4% faster than
// three), since fewer requests queued ahead of each tile shorten its latency.  The
// chunked prefill has a ring of its own (PF_NB), shared by its waves.  The compiler does
// not track these transfers, so the pipeline waits on them explicitly with s_waitcnt
// vmcnt (every tile issues the same number of transfers, and no other vector-memory
// load is issued inside the loop).
//
// Slot layout (bytes): K codes [0, 2048), V codes [2048, 4096), K scales [4096, +SKB),
// V scales [.., +256).  A 16-row half of K or V is 1 KB: LDS row position P holds tile
// row rowperm(P) of the half, and its 16-byte chunk slot S holds chunk S ^ f(P).  The
// row permutation and the chunk swizzle make the q.K reads (lane (r, j): chunk j of row
// r, ds_read_b128) and the P.V reads (lane (r, j): dword r of row 4j + i, ds_read_b32)
// free of bank conflicts for 32- and for 64-bank LDS.  K scales are stored group-major
// ([g][32 rows]) so a lane reads its 4 rows of its group with one ds_read_b128.
constexpr int NB = 2;
constexpr int DEPTH = NB - 1;   // tiles in flight behind the one being processed

__device__ __forceinline__ int rowinv(int rho) { return 4 * (rho >> 2) + ((rho + (rho >> 2)) & 3); }
__device__ __forceinline__ int rowperm(int P) { return 4 * (P >> 2) + (((P & 3) - (P >> 2)) & 3); }
__device__ __forceinline__ int chunk_swz(int P) { return ((P >> 1) ^ (P >> 3)) & 3; }

template <int NGK>
struct Slot {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2048;
  static constexpr int SK_OFF = 4096;
  static constexpr int SK_BYTES = NGK <= 2 ? 256 : 512;
  static constexpr int SV_OFF = SK_OFF + SK_BYTES;
  static constexpr int BYTES = SV_OFF + 256;
  static constexpr int DMA = 4 + (NGK <= 2 ? 1 : 2) + 1;   // transfers per tile
};

// Cache policy of the tile transfers: non-temporal ("nt"), since every cache byte is read
// once per step.  A plain streaming-read kernel on this machine moves ~12% more bytes per
// second with nt loads than with plain ones (6.2 -> 7.0 TB/s at its best launch shape).
constexpr int CPOL_NT = 2;
template <int AUX = 0>
__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gbl_vptr)g, (lds_vptr)l, 16, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void dma4(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gbl_vptr)g, (lds_vptr)l, 4, 0, AUX);
}
// The transfer of one scale per lane into one LDS dword per lane.  fp32 scales: a
// 4-byte transfer.  fp16 scales (H16): a 2-byte transfer, which lands zero-extended in
// the low half of the lane's dword (lane stride 4 bytes, checked on gfx950), so the
// LDS tile layout and its reads are the same for both and the reader converts.
template <bool H16>
__device__ __forceinline__ void dma_scale(const uint8_t* g, uint8_t* l) {
  if constexpr (H16) __builtin_amdgcn_global_load_lds((gbl_vptr)g, (lds_vptr)l, 2, 0, CPOL_NT);
  else __builtin_amdgcn_global_load_lds((gbl_vptr)g, (lds_vptr)l, 4, 0, CPOL_NT);
}
// bytes of one stored scale, and the shift from a 4-byte scale offset to the stored one
template <bool H16> constexpr int SCB = H16 ? 2 : 4;
template <bool H16> constexpr int SCSH = H16 ? 1 : 0;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most n tiles' transfers (DMA each) are outstanding, n in 0 .. D <= 3
// (uniform; the immediate must be a constant, hence the cases).
template <int DMA, int D>
__device__ __forceinline__ void wait_vmcnt_tiles(int n) {
  static_assert(D >= 1 && D <= 3, "pipeline depth");
  if (D >= 3 && n >= 3) wait_vmcnt<3 * DMA>();
  else if (D >= 2 && n == 2) wait_vmcnt<2 * DMA>();
  else if (n == 1) wait_vmcnt<DMA>();
  else wait_vmcnt<0>();
}

// Workgroup barrier over LDS data: waits for this wave's LDS operations only.
// __syncthreads()'s fence also waits for every outstanding global load (vmcnt 0), here
// the transfers of the first tiles, which held the loop start back by ~1.5 us.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------
// Timeline probe (a separate build, -DKVQ_TIMELINE: libkvq_timeline.so; the library itself
// is built without it).  Each workgroup records the 100 MHz real-time counter at its phase
// points into a.stamps[workgroup * TL_SLOTS + i]:
//   0 entry (wave 0)   1 XCC id << 32 | HW_ID   2 q in LDS (after the prologue barrier)
//   3 wave 0's loop start   4 .. 11 loop end of waves 0 .. 7
//   12 partial published (thread 0)   13 arrival counted (thread 0)
//   14 exit (thread 0: after the merge in the last workgroup of a unit)
//   15 tiles processed by waves 0 .. 7, 8 bits each
//   16 kernel arguments read (wave 0)   17 wave 0's first tile landed
#ifdef KVQ_TIMELINE
constexpr int TL_SLOTS = 32;
__device__ __forceinline__ uint64_t tl_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ void tl_put(const DecodeArgs& a, int i, uint64_t v) {
  if (a.stamps) {
    const size_t wg = blockIdx.x + (size_t)gridDim.x * (blockIdx.y + (size_t)gridDim.y * blockIdx.z);
    a.stamps[wg * TL_SLOTS + i] = v;
  }
}
#endif

// Per-lane byte offsets of the transfers, fixed for the whole kernel: lane l fills LDS
// row position P = l / 4, chunk slot l % 4 with chunk (l % 4) ^ f(P) of tile row
// rowperm(P) (+16 for the second half); scale transfers take row l % 32.
struct DmaOffs {
  int kv[2];    // K / V codes, half T: row (16T + rowperm(P)) * 64 + 16 * chunk
  int rho[2];   // the tile rows behind kv[T] (for the clamped path)
  int kap16;    // 16 * chunk
  int sk[2];    // K scale h: (l % 32) * NGK * 4 + g * 4
  int sv;       // V scale: (l % 32) * 4
};

template <int NGK>
__device__ __forceinline__ DmaOffs dma_offsets(int lane) {
  DmaOffs o;
  const int P = lane >> 2;
  o.kap16 = 16 * ((lane & 3) ^ chunk_swz(P));
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    o.rho[T] = 16 * T + rowperm(P);
    o.kv[T] = o.rho[T] * (HD / 2) + o.kap16;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) o.sk[h] = ((lane & 31) * NGK + min((lane >> 5) + 2 * h, NGK - 1)) * 4;
  o.sv = (lane & 31) * 4;
  return o;
}

// Issue the transfers of tile t0 (positions t0 .. t0 + 31 of a split ending at pe) into
// the LDS slot `lb`.  A full tile whose 32 slots are contiguous is addressed from one
// scalar base row plus the fixed lane offsets; otherwise each row is clamped to pe - 1
// (masked positions read a valid row) and wrapped around the ring.
// The unit's four streams as buffer resources (base at the unit's first row), so that a
// full tile's transfers take a scalar byte offset plus the fixed lane offsets and need no
// per-lane address arithmetic.  Word 3 is the gfx9 raw-buffer configuration; the record
// count is the unit's bytes (used only for units below 4 GiB per stream: cap <= 2^26).
struct UnitBufs {
  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
};
constexpr int BUF_CFG = 0x00020000;
constexpr int BUF_MAX_CAP = 1 << 26;
template <int NGK, bool H16>
__device__ __forceinline__ UnitBufs unit_bufs(const DecodeArgs& a, size_t row0) {
  const uint32_t cap = (uint32_t)min(a.cap, BUF_MAX_CAP);
  auto mk = [&](const void* base, size_t row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(base) + row0 * row_bytes), (short)0,
        (int)(cap * row_bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)(cap * row_bytes)), BUF_CFG);
  };
  return {mk(a.k_codes, HD / 2), mk(a.v_codes, HD / 2), mk(a.k_scales, NGK * SCB<H16>),
          mk(a.v_scales, SCB<H16>)};
}
template <int SIZE>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        uint8_t* l) {
  static_assert(SIZE == 16 || SIZE == 4 || SIZE == 2, "transfer size");
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)l, 16, voff, soff, 0, CPOL_NT);
  else if constexpr (SIZE == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)l, 4, voff, soff, 0, CPOL_NT);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)l, 2, voff, soff, 0, CPOL_NT);
}

template <int NGK, bool SK, bool H16 = false>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, size_t row0, int t0, int pe,
                                           int lo, int vlo, uint8_t* lb, int lane,
                                           const DmaOffs& o, const UnitBufs& ub) {
  using L = Slot<NGK>;
  const int cap = a.cap;
  // the tile's first slot; with sinks, a tile at or past the window start holds
  // positions t0 .. t0 + 31 themselves, in consecutive ring slots unless it wraps
  // (tiles below the window start, which hold sinks, take the general path)
  const int sbase = SK ? (t0 >= lo ? cache_slot(t0, cap, a.sinks) : cap)
                       : (t0 < cap ? t0 : t0 % cap);
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_codes);
  const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_scales);
  const uint8_t* vs = reinterpret_cast<const uint8_t*>(a.v_scales);
  if (t0 + TILE <= pe && sbase + TILE <= cap && cap <= BUF_MAX_CAP) {
    const uint32_t sb = (uint32_t)sbase;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      dma_buf<16>(ub.kc, (uint32_t)o.kv[T], sb * (HD / 2), lb + L::K_OFF + 1024 * T);
      dma_buf<16>(ub.vc, (uint32_t)o.kv[T], sb * (HD / 2), lb + L::V_OFF + 1024 * T);
    }
#pragma unroll
    for (int h = 0; h < (NGK <= 2 ? 1 : 2); ++h)
      dma_buf<SCB<H16>>(ub.ks, (uint32_t)(o.sk[h] >> SCSH<H16>), sb * (NGK * SCB<H16>),
                        lb + L::SK_OFF + 256 * h);
    dma_buf<SCB<H16>>(ub.vs, (uint32_t)(o.sv >> SCSH<H16>), sb * SCB<H16>, lb + L::SV_OFF);
    return;
  }
  auto row_of = [&](int rho) -> size_t {
    int off = rho;
    if (t0 + off > pe - 1) off = pe - 1 - t0;
    if constexpr (SK) {   // virtual index u: [vlo, lo) stands for the sinks 0 .. lo - vlo - 1
      const int u = t0 + off;
      return row0 + (size_t)cache_slot(u >= lo ? u : u - vlo, cap, a.sinks);
    }
    int sl = sbase + off;
    if (sl >= cap) sl -= cap;
    return row0 + (size_t)sl;
  };
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const size_t row = row_of(o.rho[T]);
    dma16<CPOL_NT>(kc + row * (HD / 2) + o.kap16, lb + L::K_OFF + 1024 * T);
    dma16<CPOL_NT>(vc + row * (HD / 2) + o.kap16, lb + L::V_OFF + 1024 * T);
  }
  const size_t srow = row_of(lane & 31);
#pragma unroll
  for (int h = 0; h < (NGK <= 2 ? 1 : 2); ++h)
    dma_scale<H16>(ks + (srow * (NGK * 4) + (o.sk[h] - (lane & 31) * NGK * 4)) / (4 / SCB<H16>),
                   lb + L::SK_OFF + 256 * h);
  dma_scale<H16>(vs + srow * SCB<H16>, lb + L::SV_OFF);
}

// ---------------------------------------------------------------------------------------
// Paged layout (include/kvq.h; "AI 推理性能调优：KV Cache 优化与显存管理的工程实践",
// bxzpzcl.cn/news/2871434, section 3.1 KVCacheManager: fixed pages from a pool).  The
// paged instance aligns its tiles to TL positions, so a tile lies in one page (P >= TL)
// or in two (P = 16 with 32-position tiles, one page per 16-row half).  Page ids are
// read with scalar loads written in asm: a vector load would join the tile transfers'
// vmcnt count, which the pipeline's waits assume holds transfers only.
__device__ __forceinline__ uint32_t page_id(const Pages& pg, int b, int e) {
  const int32_t* p = pg.table + (size_t)b * pg.pps + e;
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return min(v, (uint32_t)(pg.count - 1));   // an entry outside the pool stays inside it
}

// The rows of a tile [t0, t0 + TL) in the paged layout: positions below pb or at pe and
// beyond are clamped into [pb, pe) (their scores are masked), which keeps them in the
// tile's page(s).
struct PageRows {
  uint32_t id0, id1;   // pages of positions t0 .. and t0 + 16 .. (P = 16)
  int e0;
  __device__ __forceinline__ size_t row(const Pages& pg, int Hkv, int h, int p) const {
    const uint32_t id = (p >> pg.shift) == e0 ? id0 : id1;
    return ((size_t)id * Hkv + h) * pg.size + (p & (pg.size - 1));
  }
};
template <int TLN>
__device__ __forceinline__ PageRows page_rows(const DecodeArgs& a, int b, int t0, int pe) {
  PageRows r;
  r.e0 = t0 >> a.pages.shift;
  r.id0 = page_id(a.pages, b, r.e0);
  r.id1 = (a.pages.size < TLN && t0 + 16 < pe) ? page_id(a.pages, b, r.e0 + 1) : r.id0;
  return r;
}

template <int NGK, bool H16 = false>
__device__ __forceinline__ void issue_tile_pg(const DecodeArgs& a, int b, int h, int t0, int pb,
                                              int pe, uint8_t* lb, int lane, const DmaOffs& o) {
  using L = Slot<NGK>;
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_codes);
  const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_scales);
  const uint8_t* vs = reinterpret_cast<const uint8_t*>(a.v_scales);
  const PageRows pr = page_rows<TILE>(a, b, t0, pe);
  auto row_of = [&](int rho) -> size_t {   // tile row -> cache row, clamped into [pb, pe)
    return pr.row(a.pages, a.Hkv, h, min(max(t0 + rho, pb), pe - 1));
  };
  if (t0 >= pb && t0 + TILE <= pe) {   // (uniform) every row in range: one base per half
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const size_t rb = pr.row(a.pages, a.Hkv, h, t0 + 16 * T);   // rows 16 T .. 16 T + 15
      dma16<CPOL_NT>(kc + rb * (HD / 2) + o.kv[T] - 16 * T * (HD / 2), lb + L::K_OFF + 1024 * T);
      dma16<CPOL_NT>(vc + rb * (HD / 2) + o.kv[T] - 16 * T * (HD / 2), lb + L::V_OFF + 1024 * T);
    }
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const size_t row = row_of(o.rho[T]);
      dma16<CPOL_NT>(kc + row * (HD / 2) + o.kap16, lb + L::K_OFF + 1024 * T);
      dma16<CPOL_NT>(vc + row * (HD / 2) + o.kap16, lb + L::V_OFF + 1024 * T);
    }
  }
  const size_t srow = row_of(lane & 31);
#pragma unroll
  for (int hh = 0; hh < (NGK <= 2 ? 1 : 2); ++hh)
    dma_scale<H16>(ks + (srow * (NGK * 4) + (o.sk[hh] - (lane & 31) * NGK * 4)) / (4 / SCB<H16>),
                   lb + L::SK_OFF + 256 * hh);
  dma_scale<H16>(vs + srow * SCB<H16>, lb + L::SV_OFF);
}

// Position sets.  A head's q.K needs G * NGK of the 16 MFMA columns.  When that is at
// most 8 (S = 2), the other 8 columns score the second 16-position half of the tile in
// the same MFMAs: A row r then carries position r of half 0 in the k slots of lane
// quarters j = 0, 1 and position 16 + r in those of quarters 2, 3 (two chunks of K
// codes per lane instead of one chunk of each half), and the q of columns 8 .. 15 sits
// in quarters 2, 3 (columns 0 .. 7: quarters 0, 1).  Column r then scores positions
// 16 (r / 8) + 4j + i in lane (r, j): each lane holds 4 scores instead of 8 (the same 8
// MFMAs per tile, half the softmax arithmetic), and P.V keeps its layout: a column's B
// is its 4 values of P' in its set's k slots and zeros in the other set's.
__host__ __device__ constexpr int position_sets(int g, int ngk) { return g * ngk <= 8 ? 2 : 1; }

// Online-softmax state of one wave (per lane: query head of column r).
// P' = p * sV enters P.V as fp16 hi + lo parts; with small V scales (a head whose values
// are ~1e-3) the lo part would fall below fp16's normal range and lose its low bits.  So
// the wave carries a power-of-two normalizer 2^lvs of the V scales (wave-uniform): the
// exponent takes it as an added integer, so p~ = p * 2^lvs and l, oacc hold 2^lvs times
// their plain values; the combine entry's maximum subtracts lvs again, which cancels it.
// lvs moves (and l, oacc by the same exact power of two) only when a tile's largest V
// scale times 2^lvs leaves [1/16, 16]; it then puts that product in [1, 2).
struct State {
  floatx4 oacc[8];
  float m, l;
  int lvs;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
// fp32 pair -> fp16 pair, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pk_f16_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
// P' = p~ * sV as fp16 hi (round to nearest) + lo (the exact fp32 remainder, rounded to
// nearest): ~22 significant bits while p~ * sV stays within fp16's normal range.
__device__ __forceinline__ void split_hi_lo(float q0, float q1, uint32_t& hi, uint32_t& lo) {
  hi = pk_f16_rne(q0, q1);
  const f16x2 h = __builtin_bit_cast(f16x2, hi);
  lo = pk_f16_rne(__builtin_fmaf((float)h.x, -1.0f, q0), __builtin_fmaf((float)h.y, -1.0f, q1));
}

// Four scales stored as fp16 in the low halves of four dwords -> their fp32 values (exact).
__device__ __forceinline__ u32x4 f16lo_to_f32(const u32x4& w) {
  const floatx4 f = {(float)__builtin_bit_cast(_Float16, (uint16_t)w.x),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)w.y),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)w.z),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)w.w)};
  return __builtin_bit_cast(u32x4, f);
}

// The softmax / V-scale update of one tile.  `mx` is the tile's score maximum of the
// lane's column (over the 4 lanes j) and `svmax` the largest V scale among the rows the
// lane holds.  Returns mq = m * scale - lvs, the exponent offset of this tile's p~.
__device__ __forceinline__ float tile_update(State& st, float mx, float svmax, float qscale) {
  const float m_new = max_raw(st.m, mx);
  // V-scale band, by ballots: some lane above 16, or every lane below 1/16
  const float x = __builtin_amdgcn_ldexpf(svmax, st.lvs);
  const bool vmove = __any(x > 16.0f) || !__any(x >= 0.0625f);
  if (__any(m_new > st.m) || vmove) {
    int nl = st.lvs;
    if (vmove) {   // (rare) the wave's largest V scale of the tile
      float t = max_over_j(svmax);
      t = fmaxf(t, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       0, __builtin_bit_cast(int, t), 0x128, 0xF, 0xF, false)));   // lane r ^ 8
      t = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t)));
      nl = 1 - __builtin_amdgcn_frexp_expf(t);   // t * 2^nl in [1, 2)
    }
    const float corr = fast_exp2(__builtin_fmaf(st.m - m_new, qscale, (float)(nl - st.lvs)));
    st.l *= corr;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.oacc[e] *= corr;
    st.m = m_new;
    st.lvs = nl;
  }
  return __builtin_fmaf(st.m, qscale, -(float)st.lvs);
}

// Per-lane LDS offsets, fixed for the whole kernel (see position_sets).
struct LaneOffs {
  int k[2];     // q.K: the lane's two 16-byte chunks of K codes
  int v[4];     // P.V: dword r of row 4j + i (half 0)
  int sk;       // K scales of the lane's group and first 4 rows
  int sv;       // V scales of the lane's first 4 rows
};

// Next value of a workgroup's LDS tile counter (lane 0 adds, the wave reads its result).
// Written in asm that waits for its own result, for the same reason as read_tile.
__device__ __forceinline__ uint32_t lds_claim(uint32_t* ctr, int lane) {
  uint32_t old = 0;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_vptr)ctr;
  if (lane == 0)
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(old)
                 : "v"(addr), "v"(1u)
                 : "memory");
  return __builtin_amdgcn_readfirstlane(old);
}

// The LDS reads of one tile for one lane: two chunks of K codes, the K and V scales of
// the rows whose scores the lane holds (S = 1: rows 4j .. 4j+3 of both halves; S = 2:
// of its column's half only) and the V dwords of rows 4j + i of both halves.
struct TileData {
  u32x4 k[2], sk[2], sv[2];
  uint32_t v[2][4];
};

// A lane's read addresses in slot 0 of its wave's ring, computed once before the loop;
// the loop is unrolled over the ring's slots, so a slot's offset is an immediate of the
// read instructions and a tile costs no address arithmetic.
struct TileAddr {
  uint32_t k0, k1, sk, sv, v0, v1, v2, v3;
};
template <int NGK>
__device__ __forceinline__ TileAddr tile_addr(const uint8_t* ring, const LaneOffs& lo) {
  using L = Slot<NGK>;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_vptr)ring;
  return {base + L::K_OFF + lo.k[0], base + L::K_OFF + lo.k[1], base + L::SK_OFF + lo.sk,
          base + L::SV_OFF + lo.sv,  base + L::V_OFF + lo.v[0], base + L::V_OFF + lo.v[1],
          base + L::V_OFF + lo.v[2], base + L::V_OFF + lo.v[3]};
}

// All 14 (S = 2: 12) reads are issued in one asm statement that ends by waiting for them.  Written
// this way the compiler sees no LDS read here, so it does not add a wait for every
// transfer in flight before the tile (it cannot tell which LDS bytes a global->LDS
// transfer writes); the caller's vmcnt wait is what orders this tile's own transfers
// before the reads.  OFF: the byte offset of the tile's slot in the ring.
template <int NGK, int S, int OFF>
__device__ __forceinline__ TileData read_tile(const TileAddr& ad) {
  static_assert(OFF + 1024 + 64 < 65536, "the slot offset fits the reads' immediate");
  TileData d;
  if (S == 1) {
    asm volatile(
        "ds_read_b128 %0, %14 offset:%22\n\t"
        "ds_read_b128 %1, %15 offset:%22\n\t"
        "ds_read_b128 %2, %16 offset:%22\n\t"
        "ds_read_b128 %3, %16 offset:%23\n\t"
        "ds_read_b128 %4, %17 offset:%22\n\t"
        "ds_read_b128 %5, %17 offset:%23\n\t"
        "ds_read_b32 %6, %18 offset:%22\n\t"
        "ds_read_b32 %7, %19 offset:%22\n\t"
        "ds_read_b32 %8, %20 offset:%22\n\t"
        "ds_read_b32 %9, %21 offset:%22\n\t"
        "ds_read_b32 %10, %18 offset:%24\n\t"
        "ds_read_b32 %11, %19 offset:%24\n\t"
        "ds_read_b32 %12, %20 offset:%24\n\t"
        "ds_read_b32 %13, %21 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d.k[0]), "=&v"(d.k[1]), "=&v"(d.sk[0]), "=&v"(d.sk[1]), "=&v"(d.sv[0]),
          "=&v"(d.sv[1]), "=&v"(d.v[0][0]), "=&v"(d.v[0][1]), "=&v"(d.v[0][2]),
          "=&v"(d.v[0][3]), "=&v"(d.v[1][0]), "=&v"(d.v[1][1]), "=&v"(d.v[1][2]),
          "=&v"(d.v[1][3])
        : "v"(ad.k0), "v"(ad.k1), "v"(ad.sk), "v"(ad.sv), "v"(ad.v0), "v"(ad.v1), "v"(ad.v2),
          "v"(ad.v3), "n"(OFF), "n"(OFF + 64), "n"(OFF + 1024)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %12 offset:%20\n\t"
        "ds_read_b128 %1, %13 offset:%20\n\t"
        "ds_read_b128 %2, %14 offset:%20\n\t"
        "ds_read_b128 %3, %15 offset:%20\n\t"
        "ds_read_b32 %4, %16 offset:%20\n\t"
        "ds_read_b32 %5, %17 offset:%20\n\t"
        "ds_read_b32 %6, %18 offset:%20\n\t"
        "ds_read_b32 %7, %19 offset:%20\n\t"
        "ds_read_b32 %8, %16 offset:%21\n\t"
        "ds_read_b32 %9, %17 offset:%21\n\t"
        "ds_read_b32 %10, %18 offset:%21\n\t"
        "ds_read_b32 %11, %19 offset:%21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d.k[0]), "=&v"(d.k[1]), "=&v"(d.sk[0]), "=&v"(d.sv[0]), "=&v"(d.v[0][0]),
          "=&v"(d.v[0][1]), "=&v"(d.v[0][2]), "=&v"(d.v[0][3]), "=&v"(d.v[1][0]),
          "=&v"(d.v[1][1]), "=&v"(d.v[1][2]), "=&v"(d.v[1][3])
        : "v"(ad.k0), "v"(ad.k1), "v"(ad.sk), "v"(ad.sv), "v"(ad.v0), "v"(ad.v1), "v"(ad.v2),
          "v"(ad.v3), "n"(OFF), "n"(OFF + 1024)
        : "memory");
  }
  return d;
}

// State::m is the running maximum of the unscaled scores z = q . k; since the scale
// (softmax scale * log2 e) is positive, p = 2^(scale * (z - m)).
// S = 1: the lane's scores are positions 16T + 4j + i (T = 0, 1); S = 2: positions
// soff + 4j + i, soff = 16 * (the half of the lane's column set), see position_sets.
// masked (uniform): the tile reaches past pe (a split's last tile) or, in the paged
// layout, starts below pmin (the first tile of an aligned plan); those positions get
// score -inf.  One code path serves both kinds of tile, and the masking only rewrites
// the scores in place: with two instances of the tile in the loop, the compiler gave
// the accumulators of each its own registers and copied all 32 of them twice per tile.
template <int G, int NGK, int S, bool H16, int OFF>
__device__ __forceinline__ void process_tile(const TileAddr& ad, State& st,
                                             const half8 (&qb)[4 * S], float qbias, int t0,
                                             int pmin, int pe, int j, float qscale, bool lo_col,
                                             int soff, bool masked) {
  constexpr int NTB = 2 / S;   // 16-row blocks of q.K results per lane
  TileData td = read_tile<NGK, S, OFF>(ad);
  if constexpr (H16) {   // fp16 scales sit in the low halves of their dwords (dma_scale)
#pragma unroll
    for (int T = 0; T < NTB; ++T) {
      td.sk[T] = f16lo_to_f32(td.sk[T]);
      td.sv[T] = f16lo_to_f32(td.sv[T]);
    }
  }
  // ---- q.K: lane (r, j) gets rows 4j + i of block T for column r = (set, head, group)
  const uint32_t kw8[8] = {td.k[0].x, td.k[0].y, td.k[0].z, td.k[0].w,
                           td.k[1].x, td.k[1].y, td.k[1].z, td.k[1].w};
  float z[NTB][4];
#pragma unroll
  for (int T = 0; T < NTB; ++T) {
    const floatx4 sk = __builtin_bit_cast(floatx4, td.sk[T]);
    floatx4 cg = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4 * S; ++c)
      cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_word_u(kw8[4 * S * T + c]), qb[c], cg,
                                                  0, 0, 0);
    // q . codes_g = 2^24 C - 8 sum_g(q); then the group scale
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = __builtin_fmaf(cg[i], 16777216.0f, qbias) * sk[i];
    // the NGK columns of a head are adjacent (column = head * NGK + group): DPP adds over
    // lane pairs (and quads), in assembly so that each is one instruction (from the
    // builtin the compiler formed a DPP move and recomputed the product into it); each
    // block starts with the two wait states a DPP read needs after a VALU write
    if constexpr (NGK >= 2)
      asm volatile(
          "s_nop 1\n\t"
          "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
          : "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]));
    if constexpr (NGK >= 4)
      asm volatile(
          "s_nop 1\n\t"
          "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_add_f32_dpp %3, %3, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
          : "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) z[T][i] = sc[i];
  }
  if (masked) {
#pragma unroll
    for (int T = 0; T < NTB; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 16 * T + soff + 4 * j + i >= pe || t0 + 16 * T + soff + 4 * j + i < pmin)
          z[T][i] = NEG_INF;
  }

  // ---- online softmax (the 4 lanes j of a column share a head)
  float mx = max3_raw(z[0][0], z[0][1], max_raw(z[0][2], z[0][3]));
  if (NTB == 2) mx = max3_raw(mx, max_raw(z[NTB - 1][0], z[NTB - 1][1]),
                              max_raw(z[NTB - 1][2], z[NTB - 1][3]));
  mx = max_over_j(mx);
  float svmax;
  {
    const floatx4 v0 = __builtin_bit_cast(floatx4, td.sv[0]);
    svmax = max3_raw(v0[0], v0[1], max_raw(v0[2], v0[3]));
    if (NTB == 2) {
      const floatx4 v1 = __builtin_bit_cast(floatx4, td.sv[NTB - 1]);
      svmax = max3_raw(svmax, max_raw(v1[0], v1[1]), max_raw(v1[2], v1[3]));
    }
  }
  const float mq = tile_update(st, mx, svmax, qscale);

  // ---- P' = p~ * sV as fp16 hi + lo, in the B layout: k slot 4T + i (S = 1) or
  // 4 * set + i (S = 2, zeros in the other set's four slots)
  H8 phi, plo;
#pragma unroll
  for (int T = 0; T < NTB; ++T) {
    const floatx4 sv = __builtin_bit_cast(floatx4, td.sv[T]);
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(z[T][i], qscale, -mq));
      const float p1 = fast_exp2(__builtin_fmaf(z[T][i + 1], qscale, -mq));
      st.l += p0 + p1;
      split_hi_lo(p0 * sv[i], p1 * sv[i + 1], phi.u[2 * T + i / 2], plo.u[2 * T + i / 2]);
    }
  }
  // S = 2: the lane's two dwords go to its set's slots (the other two are zero)
  auto place = [&](H8& x) {
    const bool s1 = soff != 0;
    x.u[2] = s1 ? x.u[0] : 0u;
    x.u[3] = s1 ? x.u[1] : 0u;
    x.u[0] = s1 ? 0u : x.u[0];
    x.u[1] = s1 ? 0u : x.u[1];
  };
  H8 pb;
  if (NGK >= 2) {
#pragma unroll
    for (int w = 0; w < 2 * NTB; ++w) pb.u[w] = lo_col ? plo.u[w] : phi.u[w];
    if (S == 2) place(pb);
  } else if (S == 2) {
    place(phi);
    place(plo);
  }

  // ---- P.V: byte halves of two rows' dwords give the (row, row + 1) pairs of 4 dims
  uint32_t xlo[4], xhi[4];
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const int T = pr >> 1, i = 2 * (pr & 1);
    const uint32_t w0 = td.v[T][i];
    const uint32_t w1 = td.v[T][i + 1];
    xlo[pr] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);   // w0.b0 w0.b1 w1.b0 w1.b1
    xhi[pr] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);   // w0.b2 w0.b3 w1.b2 w1.b3
  }
  // V codes as exact fp16 (q, via the 1024 bias and a packed subtract): the matrix
  // cores do not keep full fp32 precision when adding a 32-term dot product whose terms
  // carry a common +8 offset, so V (unlike K) is not fed as biased subnormals.
  uint32_t xlo8[4], xhi8[4];
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    xlo8[pr] = xlo[pr] >> 8;
    xhi8[pr] = xhi[pr] >> 8;
  }
  // (dims with e & 3 in {1, 3} accumulate 16 times their value; see v_pair_f16)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    H8 va;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const uint32_t x = e < 4 ? xlo[pr] : xhi[pr];
      const uint32_t x8 = e < 4 ? xlo8[pr] : xhi8[pr];
      switch (e & 3) {
        case 0: va.u[pr] = v_pair_f16<0>(x, x8); break;
        case 1: va.u[pr] = v_pair_f16<1>(x, x8); break;
        case 2: va.u[pr] = v_pair_f16<2>(x, x8); break;
        default: va.u[pr] = v_pair_f16<3>(x, x8); break;
      }
    }
    if (NGK >= 2) {
      // a head's NGK columns carry the same P: columns g = 0, 2 take P'_hi and g = 1, 3
      // take P'_lo, so one MFMA gives both parts (summed over columns g = 0, 1 at the end)
      st.oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.h, pb.h, st.oacc[e], 0, 0, 0);
    } else {
      st.oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.h, phi.h, st.oacc[e], 0, 0, 0);
      st.oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.h, plo.h, st.oacc[e], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------------------
// INT8 per-token tiles (bxzpzcl.cn/news/2871434 section 3.1: one scale per row and head).
// A row is 128 bytes of codes for K and for V, so a tile is 16 positions (4352 bytes
// with the scales: the same LDS ring and the same bytes in flight as the INT4 tiles).
//   q.K   A = K codes (rows = 16 positions, k = 32 dims) in 4 MFMAs; lane (r, j) holds
//         dims 32j .. 32j + 31 of position r (two 16-byte chunks) and feeds dims
//         32j + 8c .. + 7 to MFMA c.  Columns are (head, part) pairs: both carry the
//         whole q of the head (there are no K groups), so lane (column, j) gets the
//         score of positions 4j + i of its head directly, times the row scale.
//   P.V   A = V codes (rows = 16 dims, k = 4 positions per lane quarter) in 8
//         v_mfma_f32_16x16x16_f16; lane (r, j) feeds dim 8r + e of positions 4j .. 4j+3,
//         which are the positions of the 4 scores the lane holds, so B is the lane's own
//         4 values of P'_hi (part 0) or P'_lo (part 1); the two parts are summed at
//         the end as for INT4.
// Codes become exact fp16 integers with the 1024 bias: byte b with its sign bit
// flipped is q + 128; (0x64 << 8 | (q + 128)) is the fp16 1152 + q; a packed subtract of
// 1152 leaves q.  (Fed as biased subnormals like the INT4 keys, the +128 offset would
// cost ~16 times the INT4 keys' accumulation error.)
// LDS: tile row rho lives in row slot P = rho ^ ((rho >> 2) & 1) and its 16-byte chunk c
// in chunk slot c ^ g(P), g(P) = ((P >> 1) ^ ((P & 1) << 2)) & 7: the K reads (16 rows,
// one chunk) and the V reads (the 16 eight-byte pieces of a row; two rows an XOR 4 apart
// per 32 lanes) are then free of bank conflicts for 32- and 64-bank LDS.
struct Slot8 {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 2048;
  static constexpr int SK_OFF = 4096;   // 16 K scales, then 16 V scales, then 128 spare
  static constexpr int SV_OFF = 4160;
  static constexpr int BYTES = 4352;
  static constexpr int DMA = 5;
};
constexpr int TILE8 = 16;
__device__ __forceinline__ int rowslot8(int rho) { return rho ^ ((rho >> 2) & 1); }
__device__ __forceinline__ int chunk_swz8(int P) { return ((P >> 1) ^ ((P & 1) << 2)) & 7; }

struct DmaOffs8 {
  int kv[2];    // K / V codes, transfer T: tile row rho_T, chunk (byte offset)
  int rho[2];
  int ch16[2];  // 16 * logical chunk of transfer T
  int srow;     // the tile row whose scale this lane moves
  bool sv;      // lanes 16..31 move V scales, the others K scales
};

__device__ __forceinline__ DmaOffs8 dma_offsets8(int lane) {
  DmaOffs8 o;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int P = 8 * T + (lane >> 3), pc = lane & 7;
    o.rho[T] = rowslot8(P);                   // (an involution)
    o.ch16[T] = 16 * (pc ^ chunk_swz8(P));
    o.kv[T] = o.rho[T] * 128 + o.ch16[T];
  }
  o.srow = lane & 15;
  o.sv = (lane >> 4) == 1;
  return o;
}

template <bool SK>
__device__ __forceinline__ void issue_tile8(const DecodeArgs& a, size_t row0, int t0, int pe,
                                            int lo, int vlo, uint8_t* lb, const DmaOffs8& o) {
  using L = Slot8;
  const int cap = a.cap;
  const int sbase = t0 % cap;
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_codes);
  if (!SK && t0 + TILE8 <= pe && sbase + TILE8 <= cap) {
    const size_t rb = row0 + (size_t)sbase;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      dma16<CPOL_NT>(kc + rb * HD + o.kv[T], lb + L::K_OFF + 1024 * T);
      dma16<CPOL_NT>(vc + rb * HD + o.kv[T], lb + L::V_OFF + 1024 * T);
    }
    const float* sc = o.sv ? a.v_scales : a.k_scales;
    dma4<CPOL_NT>(sc + rb + o.srow, lb + L::SK_OFF);
    return;
  }
  auto row_of = [&](int rho) -> size_t {
    int off = rho;
    if (t0 + off > pe - 1) off = pe - 1 - t0;
    if constexpr (SK) {   // as in issue_tile
      const int u = t0 + off;
      return row0 + (size_t)cache_slot(u >= lo ? u : u - vlo, cap, a.sinks);
    }
    int sl = sbase + off;
    if (sl >= cap) sl -= cap;
    return row0 + (size_t)sl;
  };
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const size_t row = row_of(o.rho[T]);
    dma16<CPOL_NT>(kc + row * HD + o.ch16[T], lb + L::K_OFF + 1024 * T);
    dma16<CPOL_NT>(vc + row * HD + o.ch16[T], lb + L::V_OFF + 1024 * T);
  }
  const float* sc = o.sv ? a.v_scales : a.k_scales;
  dma4<CPOL_NT>(sc + row_of(o.srow), lb + L::SK_OFF);
}

// The paged layout's INT8 tile: 16 positions from a multiple of 16, so one page.
__device__ __forceinline__ void issue_tile8_pg(const DecodeArgs& a, int b, int h, int t0, int pb,
                                               int pe, uint8_t* lb, const DmaOffs8& o) {
  using L = Slot8;
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_codes);
  const PageRows pr = page_rows<TILE8>(a, b, t0, pe);
  auto row_of = [&](int rho) -> size_t {
    return pr.row(a.pages, a.Hkv, h, min(max(t0 + rho, pb), pe - 1));
  };
  if (t0 >= pb && t0 + TILE8 <= pe) {   // (uniform) 16 consecutive rows of one page
    const size_t rb = pr.row(a.pages, a.Hkv, h, t0);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      dma16<CPOL_NT>(kc + rb * HD + o.kv[T], lb + L::K_OFF + 1024 * T);
      dma16<CPOL_NT>(vc + rb * HD + o.kv[T], lb + L::V_OFF + 1024 * T);
    }
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const size_t row = row_of(o.rho[T]);
      dma16<CPOL_NT>(kc + row * HD + o.ch16[T], lb + L::K_OFF + 1024 * T);
      dma16<CPOL_NT>(vc + row * HD + o.ch16[T], lb + L::V_OFF + 1024 * T);
    }
  }
  const float* sc = o.sv ? a.v_scales : a.k_scales;
  dma4<CPOL_NT>(sc + row_of(o.srow), lb + L::SK_OFF);
}

struct LaneOffs8 {
  int k[2];     // chunks 2j, 2j + 1 of row r
  int v[4];     // bytes 8r .. 8r + 7 of rows 4j + i
  int sk, sv;   // scales of rows 4j .. 4j + 3
};

__device__ __forceinline__ LaneOffs8 lane_offsets8(int r, int j) {
  LaneOffs8 lo;
  const int P = rowslot8(r);
#pragma unroll
  for (int h = 0; h < 2; ++h) lo.k[h] = P * 128 + 16 * ((2 * j + h) ^ chunk_swz8(P));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int Pv = rowslot8(4 * j + i);
    lo.v[i] = Pv * 128 + 16 * ((r >> 1) ^ chunk_swz8(Pv)) + 8 * (r & 1);
  }
  lo.sk = 16 * j;
  lo.sv = 16 * j;
  return lo;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct TileData8 {
  u32x4 k[2];
  u32x4 sk, sv;
  u32x2 v[4];
};

// The 8 LDS reads of an INT8 tile, in one asm statement that waits for them (see
// read_tile).
__device__ __forceinline__ TileData8 read_tile8(const uint8_t* lb, const LaneOffs8& lo) {
  using L = Slot8;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_vptr)lb;
  const uint32_t ak0 = base + L::K_OFF + lo.k[0], ak1 = base + L::K_OFF + lo.k[1];
  const uint32_t ask = base + L::SK_OFF + lo.sk, asv = base + L::SV_OFF + lo.sv;
  const uint32_t av0 = base + L::V_OFF + lo.v[0], av1 = base + L::V_OFF + lo.v[1];
  const uint32_t av2 = base + L::V_OFF + lo.v[2], av3 = base + L::V_OFF + lo.v[3];
  TileData8 d;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b64 %4, %12\n\t"
      "ds_read_b64 %5, %13\n\t"
      "ds_read_b64 %6, %14\n\t"
      "ds_read_b64 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d.k[0]), "=&v"(d.k[1]), "=&v"(d.sk), "=&v"(d.sv), "=&v"(d.v[0]), "=&v"(d.v[1]),
        "=&v"(d.v[2]), "=&v"(d.v[3])
      : "v"(ak0), "v"(ak1), "v"(ask), "v"(asv), "v"(av0), "v"(av1), "v"(av2), "v"(av3)
      : "memory");
  return d;
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
union H4 {
  half4 h;
  uint32_t u[2];
};

// Bytes 0, 1 (SEL = 0x04010400) or 2, 3 (0x04030402) of a sign-flipped code word with
// 0x64 above each: the fp16 pair (1152 + q0, 1152 + q1), then q0, q1 exactly.
template <uint32_t SEL>
__device__ __forceinline__ uint32_t k8_pair(uint32_t xflip) {
  return pk_sub_f16(__builtin_amdgcn_perm(0x64646464u, xflip, SEL), 1152.0f);
}
// Byte e of two rows' code words (positions p, p + 1) as the fp16 pair (q_p, q_p+1).
__device__ __forceinline__ uint32_t v8_pair(uint32_t w0, uint32_t w1, uint32_t sel) {
  return pk_sub_f16(__builtin_amdgcn_perm(w1, w0, sel) ^ 0x64806480u, 1152.0f);
}

template <int G>
__device__ __forceinline__ void process_tile8(const uint8_t* lb, const LaneOffs8& lo, State& st,
                                              const half8 (&qb)[4], int t0, int pmin, int pe,
                                              int j, float qscale, bool lo_col, bool masked) {
  const TileData8 td = read_tile8(lb, lo);
  // ---- q.K: the lane's 32 dims in 4 MFMAs, 8 dims each
  const uint32_t kw[8] = {td.k[0].x, td.k[0].y, td.k[0].z, td.k[0].w,
                          td.k[1].x, td.k[1].y, td.k[1].z, td.k[1].w};
  floatx4 cg = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x0 = kw[2 * c] ^ 0x80808080u, x1 = kw[2 * c + 1] ^ 0x80808080u;
    H8 ka;
    ka.u[0] = k8_pair<0x04010400u>(x0);
    ka.u[1] = k8_pair<0x04030402u>(x0);
    ka.u[2] = k8_pair<0x04010400u>(x1);
    ka.u[3] = k8_pair<0x04030402u>(x1);
    cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka.h, qb[c], cg, 0, 0, 0);
  }
  const floatx4 sk = __builtin_bit_cast(floatx4, td.sk);
  float z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = cg[i] * sk[i];
  if (masked) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + 4 * j + i >= pe || t0 + 4 * j + i < pmin) z[i] = NEG_INF;
  }

  // ---- online softmax (the 4 lanes j of a column share a head)
  float mx = max3_raw(z[0], z[1], max_raw(z[2], z[3]));
  mx = max_over_j(mx);
  const floatx4 sv = __builtin_bit_cast(floatx4, td.sv);
  const float mq = tile_update(st, mx, max3_raw(sv[0], sv[1], max_raw(sv[2], sv[3])), qscale);

  // ---- P' = p~ * sV as fp16 hi + lo; the column's part goes to B
  H4 pb;
#pragma unroll
  for (int i = 0; i < 4; i += 2) {
    const float p0 = fast_exp2(__builtin_fmaf(z[i], qscale, -mq));
    const float p1 = fast_exp2(__builtin_fmaf(z[i + 1], qscale, -mq));
    st.l += p0 + p1;
    uint32_t hi, lo;
    split_hi_lo(p0 * sv[i], p1 * sv[i + 1], hi, lo);
    pb.u[i / 2] = lo_col ? lo : hi;
  }

  // ---- P.V: dim 8r + e of positions 4j .. 4j + 3
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int wsel = e >> 2, b = e & 3;
    const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
    H4 va;
    va.u[0] = v8_pair(td.v[0][wsel], td.v[1][wsel], sel);
    va.u[1] = v8_pair(td.v[2][wsel], td.v[3][wsel], sel);
    st.oacc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(va.h, pb.h, st.oacc[e], 0, 0, 0);
  }
}

// Device-scope (all XCDs) store / load of one float of the split partials.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// an 8-byte-aligned (max, sum) pair in one load
__device__ __forceinline__ uint64_t fetch_pair(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The new token's row when the append is fused into the attention.  Wave 0 of the
// first workgroup of each (sequence, KV head) copies the fp16 K and V rows into LDS at
// the start (with the workgroup's one copy of the G query rows), quantizes them to the
// append kernel's codes (the same scale and fp32 quotient, rounded half to even) while
// its first tiles are in flight (lanes 0..15: K dims 8c .. 8c+7, c = lane; lanes
// 16..31: V), and keeps the result in LDS: the row
// enters this step's softmax as one more entry of the workgroup's combine (no tile
// reads it back from memory), and its codes and scales are written to the cache at the
// end.
struct NewLds {
  uint16_t k[HD], v[HD];  // the new token's fp16 K and V rows (staged by transfers)
  float m[8];          // the new row's score per head (base-2 units)
  float o[HD];         // its dequantized V row
  uint32_t w[32];      // packed codes of lanes 0..31 (K dims 8c.., then V dims 8c..)
  float sc[32];        // the group scale each of those lanes holds
};

struct NewRow {
  float z[8];     // unscaled score per query head (K lanes)
  float v[8];     // dequantized V values of dims 8c .. 8c+7 (V lanes)
  uint32_t w;     // the 8 packed codes of this lane
  float sc;       // the group scale of this lane
};

__device__ __forceinline__ void f16x8_to_f32(const u32x4& r, float x[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    x[2 * i] = (float)h.x;
    x[2 * i + 1] = (float)h.y;
  }
}

// Reductions within aligned groups of 2^n lanes of a 16-lane row, by DPP (VALU, no LDS
// round trip): quad swaps for partners 1 and 2, then the half-row and row mirrors, each
// of which pairs a lane with one in the other half of its group of 8 / 16.
template <bool MAX, int CTRL>
__device__ __forceinline__ float dpp_step(float x) {
  const float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
  return MAX ? fmaxf(x, y) : x + y;
}
template <bool MAX, int LANES>   // LANES: 1, 2, 4, 8 or 16
__device__ __forceinline__ float row_reduce(float x) {
  if (LANES >= 2) x = dpp_step<MAX, 0xB1>(x);    // quad_perm [1, 0, 3, 2]
  if (LANES >= 4) x = dpp_step<MAX, 0x4E>(x);    // quad_perm [2, 3, 0, 1]
  if (LANES >= 8) x = dpp_step<MAX, 0x141>(x);   // row_half_mirror
  if (LANES >= 16) x = dpp_step<MAX, 0x140>(x);  // row_mirror
  return x;
}

// H16: the fp16-scale format's arithmetic (the append kernel's): scale fl16(amax / 7),
// 1 when that is 0, and each quotient rounded to fp16 before it is rounded to an integer.
template <int G, int NGK, bool H16 = false>
__device__ __forceinline__ NewRow append_row(const DecodeArgs& a, const NewLds* s,
                                             const uint8_t* qrows, int lane) {
  NewRow nr;
  const bool isv = lane >= 16;
  const int c = lane & 15;
  constexpr int LPG_K = 16 / NGK;                       // lanes per K group (V: 16)
  float x[8];
  f16x8_to_f32(*reinterpret_cast<const u32x4*>((isv ? s->v : s->k) + 8 * c), x);
  float am = abs_max8(x);
  const float am_row = row_reduce<true, 16>(am);
  am = isv ? am_row : row_reduce<true, LPG_K>(am);
  float sc;
  if constexpr (H16) {
    const float s16 = (float)(_Float16)(am / 7.0f);
    sc = s16 == 0.0f ? 1.0f : s16;
  } else {
    sc = kvq_int4_scale(am);
  }
  const float rc = 1.0f / sc;
  uint32_t w = 0;
  float code[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const float y = H16 ? (float)(_Float16)(x[jj] / sc) : kvq_div_exact(x[jj], sc, rc);
    const float q = fminf(fmaxf(rintf(y), -7.0f), 7.0f);
    code[jj] = q;
    w |= ((uint32_t)(int)q & 15u) << (4 * jj);
  }
  nr.w = w;
  nr.sc = sc;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) nr.v[jj] = code[jj] * sc;
  // score of every query head (K lanes): sum over K groups of (group scale) * (q . codes)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float qv[8];
    f16x8_to_f32(*reinterpret_cast<const u32x4*>(qrows + h * 2 * HD + 16 * c), qv);
    float d = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) d = __builtin_fmaf(qv[jj], code[jj], d);
    d = row_reduce<false, LPG_K>(d) * sc;               // within the K group, scaled
    if (LPG_K < 2) d = dpp_step<false, 0xB1>(d);         // then over the K groups
    if (LPG_K < 4) d = dpp_step<false, 0x4E>(d);
    if (LPG_K < 8) d = dpp_step<false, 0x141>(d);
    if (LPG_K < 16) d = dpp_step<false, 0x140>(d);
    nr.z[h] = d;
  }
  return nr;
}

// Write the new row's codes and scales (kept in LDS by lanes 0..31) to cache row `row`.
template <int NGK, bool H16 = false>
__device__ __forceinline__ void store_new_row(const DecodeArgs& a, const NewLds* s, size_t row,
                                              int lane) {
  const bool isv = lane >= 16;
  const int c = lane & 15;
  const uint32_t w = s->w[lane];
  const float sc = s->sc[lane];
  auto put = [](const float* base, size_t i, float v) {   // (fp16 scales: v is exact in fp16)
    if constexpr (H16) reinterpret_cast<_Float16*>(const_cast<float*>(base))[i] = (_Float16)v;
    else const_cast<float*>(base)[i] = v;
  };
  if (isv) {
    static_cast<uint32_t*>(const_cast<void*>(a.v_codes))[row * (HD / 8) + c] = w;
    if (c == 0) put(a.v_scales, row, sc);
  } else {
    const int lpg = a.gk >> 3;
    static_cast<uint32_t*>(const_cast<void*>(a.k_codes))[row * (HD / 8) + c] = w;
    if ((c & (lpg - 1)) == 0) put(a.k_scales, row * NGK + c / lpg, sc);
  }
}

// I8: the INT8 per-token format (NGK = 2 then counts the (head, part) columns of a head,
// both carrying the whole q; 16-position tiles, one position set).
// SK: the cache keeps attention-sink slots ahead of its ring (a separate instance, so
// that the common case carries no sink arithmetic).
// ---------------------------------------------------------------------------------------
// Recent fp16 rows ("LLM长上下文推理优化：用INT4状态机管理KV Cache", pwwt.cn/news/4219524,
// section 8.3: older tokens in INT4, recent ones in FP16).  Positions [rlo, len),
// rlo = max(window start, len - recent), are read from the fp16 rings instead of the
// codes.  Every split workgroup takes a chunk of them (extra workgroups would not be
// resident with the splits: the plan gives each CU one), and its wave w the rows
// t = r0 + w, r0 + w + WAVES, ... of the chunk, RPW at a time.  A wave issues the loads
// of its first RPW rows right after the q barrier, behind its first tile, so their
// latency passes under the tile stream (up to RPRE rows; any further ones are loaded
// after the loop, RPW at a time), and attends the rows after its tile loop.
// Lane l holds dims 2l, 2l + 1 of a row.  A batch's G * RPW scores are wave sums (DPP),
// reduced stage by stage over the whole batch so that the independent sums overlap;
// the batch then updates each head's running (max, sum) once (max over the batch
// first, then independent exponentials), and the lane keeps its two dims of the
// weighted V sum.  The result is a second combine entry of the wave (entry WAVES + w),
// in the same form as a tile entry (max in base-2 units), so the combine, the partial,
// the arrival and the merge are unchanged.  With the append fused, position len - 1 is
// the new token's row (read from the caller's buffer); the appending wave stores it
// into its ring row from LDS before the loop (no workgroup of the launch reads that row
// of the ring: the attended positions before len - 1 are the recent - 1 others).
constexpr int RPW = 4;            // rows per wave and batch
constexpr int RPRE = 16;          // rows per wave loaded before the tile loop

struct RecentBatch {
  uint32_t kw[RPW], vw[RPW];      // the lane's two fp16 of K and of V of RPW rows
};
struct RecentRows {
  int t0, r1;                     // this wave's first row and the chunk's end (stride WAVES)
  RecentBatch b[RPRE / RPW];
};

// rows t0, t0 + WAVES, ... (RPW of them; zero past r1)
__device__ __forceinline__ void recent_load(const DecodeArgs& a, int unit, int len, bool fused,
                                            int lane, int t0, int r1, RecentBatch& rb) {
  const size_t base = (size_t)unit * a.recent * (HD / 2) + lane;
  const uint32_t* kring = reinterpret_cast<const uint32_t*>(a.k_recent) + base;
  const uint32_t* vring = reinterpret_cast<const uint32_t*>(a.v_recent) + base;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int t = t0 + i * WAVES;
    if (t < r1) {   // (uniform)
      if (fused && t == len - 1) {   // (uniform) the new token's row
        rb.kw[i] = reinterpret_cast<const uint32_t*>(a.k_new)[(size_t)unit * (HD / 2) + lane];
        rb.vw[i] = reinterpret_cast<const uint32_t*>(a.v_new)[(size_t)unit * (HD / 2) + lane];
      } else {
        const size_t o = (size_t)(t % a.recent) * (HD / 2);
        rb.kw[i] = kring[o];
        rb.vw[i] = vring[o];
      }
    } else {
      rb.kw[i] = 0u;
      rb.vw[i] = 0u;
    }
  }
}

__device__ __forceinline__ RecentRows recent_preload(const DecodeArgs& a, int unit, int len,
                                                     int lo_pos, int rw, int nwg, int wave,
                                                     int lane, bool fused) {
  RecentRows rr;
  const int rlo = max(lo_pos, len - a.recent);
  const int rchunk = (len - rlo + nwg - 1) / nwg;
  const int r0 = rlo + rw * rchunk;
  rr.r1 = min(len, r0 + rchunk);
  rr.t0 = r0 + wave;
#pragma unroll
  for (int bi = 0; bi < RPRE / RPW; ++bi)
    recent_load(a, unit, len, fused, lane, rr.t0 + bi * RPW * WAVES, rr.r1, rr.b[bi]);
  return rr;
}

template <int G>
__device__ __forceinline__ void recent_entry(const DecodeArgs& a, int unit, int len, int lane,
                                             bool fused, const RecentRows& rr,
                                             const uint8_t* s_q, float* s_o, float* s_m,
                                             float* s_l, int ors, int ne, int slot) {
  float q0[G], q1[G], m[G], l[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const f16x2 qq = __builtin_bit_cast(f16x2, reinterpret_cast<const uint32_t*>(s_q + h * 2 * HD)[lane]);
    q0[h] = (float)qq[0];
    q1[h] = (float)qq[1];
    m[h] = empty_max(a.qscale) * a.qscale;
    l[h] = 0.0f;
    o0[h] = 0.0f;
    o1[h] = 0.0f;
  }
  // one batch of RPW rows starting at row t0 (the rows past the chunk score -inf)
  auto batch = [&](int t0, const RecentBatch& rb) {
    float v0[RPW], v1[RPW], z[RPW][G];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const f16x2 kk = __builtin_bit_cast(f16x2, rb.kw[i]), vv = __builtin_bit_cast(f16x2, rb.vw[i]);
      v0[i] = (float)vv[0];
      v1[i] = (float)vv[1];
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = __builtin_fmaf(q0[h], (float)kk[0], q1[h] * (float)kk[1]);
    }
    // the wave sums, one reduction stage at a time over the batch
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = dpp_add<0xB1>(z[i][h]);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = dpp_add<0x4E>(z[i][h]);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = dpp_add<0x141>(z[i][h]);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = dpp_add<0x140>(z[i][h]);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) {   // each 16-lane row's sum is in all its lanes
        const float lo16 = readlane_f(z[i][h], 0) + readlane_f(z[i][h], 16);
        const float hi16 = readlane_f(z[i][h], 32) + readlane_f(z[i][h], 48);
        const bool in = t0 + i * WAVES < rr.r1;   // (uniform)
        z[i][h] = in ? (lo16 + hi16) * a.qscale : NEG_INF;
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = m[h];
#pragma unroll
      for (int i = 0; i < RPW; ++i) mb = fmaxf(mb, z[i][h]);
      const float f = fast_exp2(m[h] - mb);
      float ls = l[h] * f, a0 = o0[h] * f, a1 = o1[h] * f;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const float p = fast_exp2(z[i][h] - mb);   // 0 for a row past the chunk
        ls += p;
        a0 = __builtin_fmaf(p, v0[i], a0);
        a1 = __builtin_fmaf(p, v1[i], a1);
      }
      m[h] = mb;
      l[h] = ls;
      o0[h] = a0;
      o1[h] = a1;
    }
  };
#pragma unroll
  for (int bi = 0; bi < RPRE / RPW; ++bi) {   // the preloaded rows
    const int t0 = rr.t0 + bi * RPW * WAVES;
    if (t0 < rr.r1) batch(t0, rr.b[bi]);   // (uniform)
  }
  for (int t0 = rr.t0 + RPRE * WAVES; t0 < rr.r1; t0 += RPW * WAVES) {   // any further ones
    RecentBatch nb;
    recent_load(a, unit, len, fused, lane, t0, rr.r1, nb);
    batch(t0, nb);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int d = 2 * lane;
    s_o[h * ors + d + (d >> 5)] = o0[h];
    s_o[h * ors + d + 1 + ((d + 1) >> 5)] = o1[h];
    if (lane == 0) {
      s_m[h * ne + slot] = m[h];
      s_l[h * ne + slot] = l[h];
    }
  }
}

// PG: the paged layout (page-aligned tiles, rows through the block table; a separate
// instance, so that the contiguous case carries none of it).
// H16: INT4 with fp16 scales (KVQ_INT4_G16): 2-byte scale transfers into the same tile
// layout, converted after the LDS reads; the fused append codes the new row with the
// format's fp16 arithmetic.
template <int G, int NGK, bool I8, bool SK, bool RC = false, bool PG = false, bool H16 = false>
__global__ void __launch_bounds__(NT) decode_int4_mfma_kernel(DecodeArgs a) {
  using L = std::conditional_t<I8, Slot8, Slot<NGK>>;
  constexpr int TL = I8 ? TILE8 : TILE;       // positions per tile
  constexpr int S = I8 ? 1 : position_sets(G, NGK);
  constexpr int DMA = L::DMA;
  // the wave rings; after the loop, the merge's staging of up to MAX_SPLITS partials
  constexpr int RING_BYTES = WAVES * NB * L::BYTES;
  constexpr int MERGE_BYTES = (3 * G * MAX_SPLITS + G) * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) uint8_t smem[RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES];
  __shared__ __attribute__((aligned(16))) NewLds s_new;
  __shared__ int s_last;
  __shared__ uint32_t s_claim;
  constexpr int NE = RC ? 2 * WAVES : WAVES;   // combine entries (a second per wave: recent rows)
  __shared__ __attribute__((aligned(16))) float s_mlc[2 * NE * G];      // combine max / sum
  __shared__ __attribute__((aligned(16))) uint8_t s_q[G * 2 * HD];      // the G query rows
#ifdef KVQ_TIMELINE
  __shared__ uint32_t s_tl_tiles[WAVES];
#endif

#ifdef KVQ_TIMELINE
  const uint64_t tl_entry = tl_now();
#endif
  const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps tile positions, ring addresses and base pointers in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // fp16 inputs, copied into LDS by wave 0's first transfers, ahead of every tile and
  // of the kernel arguments the tile schedule needs: the G query rows, one copy shared
  // by the workgroup, and in the appending workgroup the new K/V rows into s_new.
  // (Loading them into registers inside the loop would make the compiler wait for them
  // wherever it reuses those registers; a load before the loop would make it wait ahead
  // of every transfer.)
  uint8_t* qstage = s_q;
#ifdef KVQ_TIMELINE
  // (an empty asm that consumes the q pointer: the stamp follows its kernel-argument load)
  asm volatile("" ::"s"(a.q), "s"(a.k_codes));
  const uint64_t tl_karg = tl_now();
#endif
  if (wave == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      dma4(a.q + ((size_t)b * a.Hq + kvh * G + h) * HD + 2 * lane, qstage + h * 2 * HD);
    if (!I8 && sp == 0 && a.k_new != nullptr) {
      const size_t u = (size_t)b * a.Hkv + kvh;
      dma4(a.k_new + u * HD + 2 * lane, reinterpret_cast<uint8_t*>(s_new.k));
      dma4(a.v_new + u * HD + 2 * lane, reinterpret_cast<uint8_t*>(s_new.v));
    }
  }
  const int r = lane & 15, j = lane >> 4;
  // q.K column r = (set r / 8 when S = 2, head, group) with head = rr / NGK and
  // group = rr % NGK for rr = r % (16 / S); junk columns beyond G * NGK
  const int rr = S == 2 ? (r & 7) : r;
  const int cset = S == 2 ? (r >> 3) : 0;   // the half whose positions the column scores
  const int qhead = (rr / NGK) % G;
  const int qgrp = rr % NGK;
  const bool lo_col = (qgrp & 1) != 0;   // column carries P'_lo in P.V (NGK >= 2)
  const int unit = b * a.Hkv + kvh;
  const int len = a.lens[b];
  const int lo_pos = a.window > 0 ? max(0, len - a.window) : 0;
  // with the append fused, position len - 1 comes from the new token, not from a tile
  // (INT4 only: the INT8 step is appended by the quantize kernel first)
  const bool fused = !I8 && a.k_new != nullptr;
  const bool appender = fused && sp == 0;
  // tiles cover [lo_pos, pt); with recent fp16 rows, only the positions before them
  const int pt = RC ? max(lo_pos, len - a.recent) : (fused ? len - 1 : len);

  // ---- tile schedule: split sp covers positions [ps, pe) of [lo_pos, pt), nts tiles
  // of 32 positions.  Wave w starts with tile w; every further tile is
  // claimed from the workgroup's LDS counter, so faster waves take more tiles.  One
  // workgroup of 8 waves per CU: with two workgroups of 4 waves sharing a CU, one of the
  // pair was measured to lag the other by up to a third of the kernel, a split no LDS
  // counter can rebalance.
  // with a window, the attention sinks [0, nsk) come first: the splits share out the
  // virtual range [vlo, pt), where u in [vlo, lo_pos) stands for position u - vlo
  const int nsk = SK && a.window > 0 ? min(a.sinks, lo_pos) : 0;
  const int vlo = lo_pos - nsk;
  // paged layout: tiles start at multiples of TL (so each lies in one page, or two of 16),
  // from the multiple of TL below the horizon; positions below it are masked
  const int vbase = PG ? (vlo & ~(TL - 1)) : vlo;
  const int span = pt - vbase;
  int chunk = span > 0 ? (span + a.nsplit - 1) / a.nsplit : 0;
  if (PG) chunk = (chunk + TL - 1) & ~(TL - 1);
  const int ps = min(pt, vbase + sp * chunk);
  const int pe = min(pt, ps + chunk);
  const int pb = PG ? vlo : -2147483647;   // positions below are masked (paged plan)
  const int nts = (pe - ps + TL - 1) / TL;
  const size_t row0 = (size_t)unit * a.cap;
  uint8_t* ring = smem + wave * NB * L::BYTES;
  const auto dof = [&] {
    if constexpr (I8) return dma_offsets8(lane);
    else return dma_offsets<NGK>(lane);
  }();
  // (contiguous INT4 layout: the unit's streams as buffer resources)
  [[maybe_unused]] UnitBufs ubufs;
  if constexpr (!I8 && !PG) ubufs = unit_bufs<NGK, H16>(a, row0);
  auto issue = [&](int t0, uint8_t* lb) {
    if constexpr (PG) {
      if constexpr (I8) issue_tile8_pg(a, b, kvh, t0, pb, pe, lb, dof);
      else issue_tile_pg<NGK, H16>(a, b, kvh, t0, pb, pe, lb, lane, dof);
    } else {
      if constexpr (I8) issue_tile8<SK>(a, row0, t0, pe, lo_pos, vlo, lb, dof);
      else issue_tile<NGK, SK, H16>(a, row0, t0, pe, lo_pos, vlo, lb, lane, dof, ubufs);
    }
  };
  if (threadIdx.x == 0) s_claim = 0;   // ordered before the first claim by the q barrier

  const bool app_wave = appender && wave == 0;

  const auto lo = [&] {
  if constexpr (I8) {
    return lane_offsets8(r, j);
  } else {
  LaneOffs lo;
  {
    const int P = rowinv(r);
    if (S == 1) {   // chunk j of row r in both halves
      lo.k[0] = P * 64 + 16 * (j ^ chunk_swz(P));
      lo.k[1] = lo.k[0] + 1024;
    } else {        // chunks j % 2 and j % 2 + 2 of row r in half j / 2
      lo.k[0] = (j >> 1) * 1024 + P * 64 + 16 * ((j & 1) ^ chunk_swz(P));
      lo.k[1] = (j >> 1) * 1024 + P * 64 + 16 * (((j & 1) + 2) ^ chunk_swz(P));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int Pv = rowinv(4 * j + i);
      lo.v[i] = Pv * 64 + 16 * ((r >> 2) ^ chunk_swz(Pv)) + 4 * (r & 3);
    }
    lo.sk = (min(qgrp, NGK - 1) * 32 + 16 * cset + 4 * j) * 4;
    lo.sv = (16 * cset + 4 * j) * 4;
  }
  return lo;
  }
  }();

  State st;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.oacc[e] = (floatx4){0.f, 0.f, 0.f, 0.f};
  st.m = empty_max(a.qscale);
  st.l = 0.0f;
  st.lvs = 0;
  half8 qb[4 * S];
  float qbias = 0.0f;

  // The pipeline: the first DEPTH tiles start before the loop; step k claims tile
  // k + DEPTH, starts it into slot (k + DEPTH) % NB and processes tile k from slot k % NB,
  // so DEPTH tiles stay in flight behind the one being processed.  tq[i] is the tile of
  // step k + i (NONE past the end; claims only grow, so once a claim is past the end
  // every later one is too).  Only the first tile starts here, behind q; with a deeper
  // ring the others start after the q barrier: an opening burst of one tile per wave
  // brings q and the first tiles in sooner (with two tiles in flight, starting the
  // second after the barrier made the Llama-3-8B step 2% faster; a third tile started
  // early made it 2% slower).
  constexpr int NONE = -1;
  int tq[DEPTH];
  int nq = 0;   // tiles started before the q barrier (0 or 1)
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    const int id = wave + i * WAVES;
    tq[i] = id < nts ? id : NONE;
  }
  if (tq[0] != NONE) {
    issue(ps + TL * tq[0], ring);
    ++nq;
  }

  // wave 0 waits for its q (and new-row) transfers alone, which are older than its
  // tiles'; the barrier then publishes them (and the zeroed claim counter) to every wave
  if (wave == 0) wait_vmcnt_tiles<DMA, DEPTH>(nq);
  lds_barrier();
#ifdef KVQ_TIMELINE
  const uint64_t tl_q = tl_now();
#endif
#pragma unroll
  for (int i = 1; i < DEPTH; ++i)
    if (tq[i] != NONE) issue(ps + TL * tq[i], ring + i * L::BYTES);
  // (recent fp16 rows: the first batch's loads go out behind the first tiles)
  [[maybe_unused]] RecentRows rrows;
  if constexpr (RC) rrows = recent_preload(a, unit, len, lo_pos, sp, a.nsplit, wave, lane, fused);
  // q into MFMA layout (and the appending wave's quantization of the new row) while
  // the first tiles are in flight (asm reads: plain reads would make the compiler wait
  // for them as well)
  // the chunk of q feeding MFMA c: S = 1: chunk j (all c); S = 2: chunk j % 2 + 2 (c / 4)
  u32x4 qraw[4 * S];
  {
    const int ch0 = S == 1 ? j : (j & 1);
    const uint32_t aq = (uint32_t)(uintptr_t)(lds_vptr)(qstage + qhead * 2 * HD + 64 * ch0);
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:16\n\t"
        "ds_read_b128 %2, %4 offset:32\n\t"
        "ds_read_b128 %3, %4 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(qraw[0]), "=&v"(qraw[1]), "=&v"(qraw[2]), "=&v"(qraw[3])
        : "v"(aq)
        : "memory");
    if constexpr (S == 2)
      asm volatile(
          "ds_read_b128 %0, %4 offset:128\n\t"
          "ds_read_b128 %1, %4 offset:144\n\t"
          "ds_read_b128 %2, %4 offset:160\n\t"
          "ds_read_b128 %3, %4 offset:176\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(qraw[4]), "=&v"(qraw[5]), "=&v"(qraw[6]), "=&v"(qraw[7])
          : "v"(aq)
          : "memory");
  }
  // q as the B operand of MFMA c: lane quarter j holds dims 32 ch + 8 (c % 4) + {p, p+4}
  // (ch its chunk for c) in slots {2p, 2p + 1} (the order unpack_word_u produces) when
  // those dims lie in the column's K group and (S = 2) quarter j feeds the column's
  // set, zeros otherwise; qbias = -8 * (sum of those q entries)
  constexpr int QPG = 4 / NGK;   // chunks (32 dims) per K group
  float qs = 0.0f;
  if constexpr (I8) {   // INT8: dims 32j + 8c .. + 7 in order, every column of a head
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      H8 o;
      const uint32_t w[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) o.u[p] = rr < G * NGK ? w[p] : 0u;
      qb[c] = o.h;
    }
  } else {
#pragma unroll
  for (int c = 0; c < 4 * S; ++c) {
    const int ch = S == 1 ? j : (j & 1) + 2 * (c >> 2);
    const bool live = rr < G * NGK && ch / QPG == qgrp && (S == 1 || (j >> 1) == cset);
    const uint32_t w[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
    H8 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // element p is half (p&1) of word p/2; element p+4 is half (p&1) of word 2+p/2
      const uint32_t lo16 = (w[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
      const uint32_t hi16 = (w[2 + (p >> 1)] >> (16 * (p & 1))) & 0xFFFFu;
      o.u[p] = live ? (lo16 | (hi16 << 16)) : 0u;
      f16x2 h2 = __builtin_bit_cast(f16x2, o.u[p]);
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
      qs = __builtin_amdgcn_fdot2(h2, one2, qs, false);   // qs += h2.x + h2.y (one dot2)
      if (p & 1) {   // slots of nibbles taken at bits 4..7 (16 times larger): q / 16
        const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        h2 = h2 * sixteenth;
        o.u[p] = __builtin_bit_cast(uint32_t, h2);
      }
    }
    qb[c] = o.h;
  }
  qbias = -8.0f * sum_over_j(qs);
  }
  if constexpr (!I8) if (app_wave && lane < 32) {
    const NewRow nr = append_row<G, NGK, H16>(a, &s_new, qstage, lane);
    s_new.w[lane] = nr.w;
    s_new.sc[lane] = nr.sc;
    if (lane >= 16) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) s_new.o[8 * (lane - 16) + jj] = nr.v[jj];
    } else if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) s_new.m[h] = nr.z[h] * a.qscale;
    }
    if constexpr (RC) {   // the new row's fp16 K (lanes 0-15) / V (16-31) to its ring row
      const int c = lane & 15;
      const u32x4 raw = *reinterpret_cast<const u32x4*>((lane >= 16 ? s_new.v : s_new.k) + 8 * c);
      uint16_t* rrow = (lane >= 16 ? a.v_recent : a.k_recent) +
                       ((size_t)unit * a.recent + (len - 1) % a.recent) * HD;
      reinterpret_cast<u32x4*>(rrow)[c] = raw;
    }
  }

#ifdef KVQ_TIMELINE
  const uint64_t tl_loop = tl_now();
  int tl_tiles = 0;
  uint64_t tl_first = 0;
#endif
  // lane read addresses of slot 0 (INT4 tiles; the INT8 reader forms its own)
  [[maybe_unused]] TileAddr tad;
  if constexpr (!I8) tad = tile_addr<NGK>(ring, lo);
  // step k: processes slot k % NB, so the loop is unrolled NB times with the slot a
  // compile-time constant (SL)
  static_assert(NB == 2 || NB == 3, "the loop below is unrolled over a 2- or 3-slot ring");
  auto step = [&](auto slot) {
    constexpr int SL = decltype(slot)::value;
#ifdef KVQ_TIMELINE
    ++tl_tiles;
#endif
    int nn = NONE;
    if (tq[DEPTH - 1] != NONE) {
      const int id = DEPTH * WAVES + (int)lds_claim(&s_claim, lane);
      nn = id < nts ? id : NONE;
    }
    if (nn != NONE) {
      issue(ps + TL * nn, ring + ((SL + DEPTH) % NB) * L::BYTES);
      wait_vmcnt<DEPTH * DMA>();   // after tile k: the transfers of tiles k + 1 .. k + DEPTH
    } else {
      int later = 0;   // tiles still in flight behind tile k
#pragma unroll
      for (int i = 1; i < DEPTH; ++i) later += tq[i] != NONE;
      wait_vmcnt_tiles<DMA, DEPTH>(later);
    }
#ifdef KVQ_TIMELINE
    if (tl_tiles == 1) tl_first = tl_now();
#endif
    const int t0 = ps + TL * tq[0];
    const bool masked = t0 + TL > pe || (PG && t0 < pb);
    if constexpr (I8)
      process_tile8<G>(ring + SL * L::BYTES, lo, st, qb, t0, pb, pe, j, a.qscale, lo_col, masked);
    else
      process_tile<G, NGK, S, H16, SL * L::BYTES>(tad, st, qb, qbias, t0, pb, pe, j, a.qscale,
                                                  lo_col, 16 * cset, masked);
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i) tq[i] = tq[i + 1];
    tq[DEPTH - 1] = nn;
  };
  while (tq[0] != NONE) {
    step(std::integral_constant<int, 0>{});
    if (tq[0] == NONE) break;
    step(std::integral_constant<int, 1>{});
    if constexpr (NB == 3) {
      if (tq[0] == NONE) break;
      step(std::integral_constant<int, 2>{});
    }
  }
  wait_vmcnt<0>();   // (also the q staging, when this wave had no tile)
#ifdef KVQ_TIMELINE
  {
    const uint64_t tl_end = tl_now();
    if (lane == 0) {
      tl_put(a, 4 + wave, tl_end);
      s_tl_tiles[wave] = (uint32_t)tl_tiles;
      if (wave == 0) {
        uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);   // HW_REG_XCC_ID
        uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_REG_HW_ID
        tl_put(a, 0, tl_entry);
        tl_put(a, 1, ((uint64_t)xcc << 32) | hw);
        tl_put(a, 2, tl_q);
        tl_put(a, 3, tl_loop);
        tl_put(a, 16, tl_karg);
        tl_put(a, 17, tl_first);
      }
    }
    wait_vmcnt<0>();
  }
#endif

  // ---- combine the waves' column sets (and, in the appending workgroup, the new row)
  // through LDS: lane (r, j) holds O[column r][8(4j + i) + e] in oacc[e][i]; a head sits
  // in column head * NGK of each set, and each set has its own running maximum.  A wave
  // first merges its two sets (S = 2: lanes r and r ^ 8 hold the same head and dims for
  // the two halves of every tile), so it enters the combine as one entry, and writes that
  // entry into its own ring as soon as its loop ends (no other wave transfers into that
  // ring or reads it): only the last wave's writes come after the workgroup barrier.
  // Entry rows of 132 words (a pad word after every 32 dims): one write instruction
  // stores dims 32j + const of up to 8 (entry, head) rows, which then fall in 32 distinct
  // banks (unpadded they all share one bank)
  constexpr int ORS = HD + HD / 32;                             // padded row stride
  auto opad = [](int d) { return d + (d >> 5); };
  static_assert((NE / WAVES) * G * ORS * sizeof(float) <= NB * L::BYTES,
                "a wave's entries fit its ring");
  float* s_o = reinterpret_cast<float*>(ring);                 // this wave's [G][ORS]
  float* s_m = s_mlc;                                           // [G][NE]
  float* s_l = s_mlc + NE * G;                                  // [G][NE]
  if constexpr (!I8) {
#pragma unroll
    for (int e = 1; e < 8; e += 2) st.oacc[e] *= 0.0625f;   // see v_pair_f16
  }
  if (NGK >= 2) {   // column g = 0 of a head: P'_hi part + (column g = 1) P'_lo part
    // (one DPP add per value, in assembly: written with the builtin, the compiler moved
    // the adds below the branch that follows and kept a zeroed copy per value; each
    // block starts with the two wait states a DPP read needs after a VALU write)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x0 = st.oacc[e][0], x1 = st.oacc[e][1], x2 = st.oacc[e][2], x3 = st.oacc[e][3];
      asm volatile(
          "s_nop 1\n\t"
          "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
          "v_add_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
          "v_add_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
          "v_add_f32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
      st.oacc[e] = (floatx4){x0, x1, x2, x3};
    }
  }
  float l_run = sum_over_j(st.l);
  if constexpr (S == 2) {   // the partner set from lane r ^ 8 (DPP rotation by 8 in the row)
    const auto partner = [](float x) {
      return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   0x128, 0xF, 0xF, false));
    };
    const float mo = partner(st.m), lo_run = partner(l_run);
    const float mx = fmaxf(st.m, mo);
    const float f0 = fast_exp2((st.m - mx) * a.qscale), f1 = fast_exp2((mo - mx) * a.qscale);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.oacc[e][i] = __builtin_fmaf(st.oacc[e][i], f0, partner(st.oacc[e][i]) * f1);
    l_run = __builtin_fmaf(l_run, f0, lo_run * f1);
    st.m = mx;
  }
  if (rr < G * NGK && qgrp == 0 && cset == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_o[qhead * ORS + opad(8 * (4 * j + i) + e)] = st.oacc[e][i];
    if (j == 0) {   // base-2 units; - lvs cancels the V-scale normalizer in l and o
      s_m[qhead * NE + wave] = __builtin_fmaf(st.m, a.qscale, -(float)st.lvs);
      s_l[qhead * NE + wave] = l_run;
    }
  }
  if constexpr (RC)
    recent_entry<G>(a, unit, len, lane, fused, rrows, qstage, s_o + G * ORS, s_m, s_l,
                    ORS, NE, WAVES + wave);
  __syncthreads();
  const int nps = a.nsplit;                                     // partials per query head
  const size_t pbase = (size_t)(b * a.Hq + kvh * G) * nps;     // slot of (head 0, split 0)
  for (int idx = threadIdx.x; idx < G * HD; idx += NT) {
    const int h = idx / HD, d = idx % HD;
    // every entry's (max, sum, value) first, so the reads issue together (the per-head
    // max and sum are 16-byte broadcast reads); an entry that saw no position has max
    // empty_max * scale and zero sum and value, so it adds nothing whatever its weight
    float mw[NE], lw[NE], ow[NE];
#pragma unroll
    for (int w = 0; w < NE; w += 4) {
      const floatx4 m4 = *reinterpret_cast<const floatx4*>(s_m + h * NE + w);
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(s_l + h * NE + w);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mw[w + u] = m4[u];
        lw[w + u] = l4[u];
      }
    }
#pragma unroll
    for (int w = 0; w < NE; ++w)   // entry w: wave w % WAVES's, in that wave's ring
      ow[w] = reinterpret_cast<const float*>(smem + (w % WAVES) * NB * L::BYTES)[(w / WAVES) * G * ORS +
                                                                                h * ORS + opad(d)];
    // (with recent fp16 rows the new row is attended among them, not here)
    const float mn = appender && !RC ? s_new.m[h] : NEG_INF;
    const float on = appender && !RC ? s_new.o[d] : 0.0f;
    float M = mn;
#pragma unroll
    for (int w = 0; w < NE; ++w) M = fmaxf(M, mw[w]);
    float Acc = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NE; ++w) {
      const float f = fast_exp2(mw[w] - M);
      Acc = __builtin_fmaf(ow[w], f, Acc);
      Lsum = __builtin_fmaf(lw[w], f, Lsum);
    }
    if (mn != NEG_INF) {
      const float f = fast_exp2(mn - M);
      Acc = __builtin_fmaf(on, f, Acc);
      Lsum += f;
    }
    const size_t o = pbase + (size_t)h * nps + sp;
    publish(a.ws_acc + o * HD + d, Acc);
    if (d == 0) {
      publish(a.ws_ml + 2 * o, M);
      publish(a.ws_ml + 2 * o + 1, Lsum);
    }
  }

  // ---- arrivals.  The partials are device-scope stores (written through to the point
  // where every XCD sees them); each wave waits until its own have completed before the
  // barrier, so when the counting thread bumps the (device-scope) arrival counter the
  // whole partial is visible.  This avoids a release fence, which on this chip writes
  // back the XCD's whole L2 and costs microseconds per workgroup.  Ordering: (1) an
  // acknowledged device-scope store has been performed where every XCD's device-scope
  // loads see it; (2) each workgroup's increment comes after its acknowledgements; (3)
  // the increments of one counter are totally ordered, so the workgroup that reads
  // count - 1 comes after every other workgroup's stores; (4) it issues its
  // device-scope partial loads only once its increment has returned (they depend on
  // the returned value through the branch below).  These are properties of the hardware
  // rather than of the C++ memory model, in which relaxed atomics order nothing; an
  // acquire on the increment adds a cache invalidation costing 2-3% per decode step.
  // the new row's codes and scales go to the cache here, so that the wait below covers
  // them together with the partials (a barrier right after the loop would wait for them
  // alone); no tile of this step reads that row
  if (app_wave && lane < 32) {
    size_t nrow;
    if constexpr (PG) nrow = page_rows<TL>(a, b, len - 1, len).row(a.pages, a.Hkv, kvh, len - 1);
    else nrow = row0 + (size_t)(SK ? cache_slot(len - 1, a.cap, a.sinks) : (len - 1) % a.cap);
    store_new_row<NGK, H16>(a, &s_new, nrow, lane);
  }
  uint32_t* cnt = a.counters + unit;
#ifdef KVQ_TIMELINE
  const uint64_t tl_pub = tl_now();
#endif
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int np = nps;                                    // partials to merge
#ifdef KVQ_TIMELINE
  const uint64_t tl_arr = tl_now();
  if (threadIdx.x == 0) {
    uint64_t packed = 0;
    for (int w = 0; w < WAVES; ++w) packed |= (uint64_t)(s_tl_tiles[w] & 255u) << (8 * w);
    tl_put(a, 12, tl_pub);
    tl_put(a, 13, tl_arr);
    tl_put(a, 15, packed);
    if (s_last != np - 1) tl_put(a, 14, tl_now());
  }
#endif
  if (s_last != np - 1) return;

  // ---- the last arrival merges the np partials of its G heads with the log-sum-exp
  // rule (device-scope loads: the partials come from other XCDs) and resets the arrival
  // counter.
  constexpr int OPT = (G * HD + NT - 1) / NT;           // outputs per thread
  // Up to SM splits: every thread loads its outputs' partials and the (max, sum) pairs of
  // their heads (repeated across a head's threads: one request per wave) in one round
  // trip and forms the weights itself, with no LDS staging and no barrier.
  constexpr int SM = 8;
  if (np <= SM) {
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int idx = threadIdx.x + NT * u;
      const int ic = min(idx, G * HD - 1);
      const int h = ic / HD, d = ic % HD;
      const size_t o0 = pbase + (size_t)h * nps;
      // (branch-free: the split index clamped to np - 1, its weight zeroed below)
      float pv[SM];
      uint64_t ml[SM];
#pragma unroll
      for (int sI = 0; sI < SM; ++sI) {
        const size_t o = o0 + (size_t)min(sI, np - 1);
        pv[sI] = fetch(a.ws_acc + o * HD + d);
        ml[sI] = fetch_pair(a.ws_ml + 2 * o);
      }
      float M = NEG_INF;
#pragma unroll
      for (int sI = 0; sI < SM; ++sI) M = max_raw(M, __builtin_bit_cast(float, (uint32_t)ml[sI]));
      float A = 0.0f, L = 0.0f;
#pragma unroll
      for (int sI = 0; sI < SM; ++sI) {
        const float ms = __builtin_bit_cast(float, (uint32_t)ml[sI]);
        const float w = sI < np && ms != NEG_INF ? fast_exp2(ms - M) : 0.0f;
        A = __builtin_fmaf(pv[sI], w, A);
        L = __builtin_fmaf(__builtin_bit_cast(float, (uint32_t)(ml[sI] >> 32)), w, L);
      }
      if (idx < G * HD) a.out[(size_t)(b * a.Hq + kvh * G + h) * HD + d] = A / L;
    }
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#ifdef KVQ_TIMELINE
    if (threadIdx.x == 0) tl_put(a, 14, tl_now());
#endif
    return;
  }
  // More splits: each thread first issues the loads of its outputs' first PF partials, so
  // their latency overlaps the maxima's (32: a 128K-position sequence's 32 splits in one
  // round trip, 2% on that step over 16; plans with fewer splits issue fewer loads).
  constexpr int PF = 32;
  // (branch-free: the loads go in groups of 4 under a uniform test, the split index
  // clamped to np - 1 inside a group and the output index to the last output)
  float pre[OPT][PF];
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = min((int)threadIdx.x + NT * u, G * HD - 1);
    const float* src = a.ws_acc + (pbase + (size_t)(idx / HD) * nps) * HD + idx % HD;
#pragma unroll
    for (int s4 = 0; s4 < PF; s4 += 4) {
      if (s4 < np) {
#pragma unroll
        for (int sI = s4; sI < s4 + 4; ++sI) pre[u][sI] = fetch(src + (size_t)min(sI, np - 1) * HD);
      } else {
#pragma unroll
        for (int sI = s4; sI < s4 + 4; ++sI) pre[u][sI] = 0.0f;
      }
    }
  }
  const int sws = np > PF ? (np + 3) & ~3 : PF;         // weight row stride (>= PF)
  static_assert(MERGE_BYTES <= sizeof(smem),
                "the merge stages up to MAX_SPLITS partials per head in the tile rings");
  float* s_mx = reinterpret_cast<float*>(smem);          // [G][np] split maxima
  float* s_ls = s_mx + G * np;                           // [G][np] split sums
  float* s_w = s_ls + G * np;                           // [G][sws] weights (0 past np)
  float* s_L = s_w + G * sws;                           // [G]
  for (int idx = threadIdx.x; idx < G * np; idx += NT) {
    const int h = idx / np, sI = idx % np;
    const uint64_t ml = fetch_pair(a.ws_ml + 2 * (pbase + (size_t)h * nps + sI));
    s_mx[idx] = __builtin_bit_cast(float, (uint32_t)ml);
    s_ls[idx] = __builtin_bit_cast(float, (uint32_t)(ml >> 32));
  }
  __syncthreads();
  // one wave per head: maximum and weighted sum of the split sums by DPP reductions
  // (splits strided over the lanes), weights 2^(m_s - M) into s_w
  for (int h = wave; h < G; h += WAVES) {
    float mx = NEG_INF;
    for (int sI = lane; sI < np; sI += 64) mx = fmaxf(mx, s_mx[h * np + sI]);
    mx = lane_group_max<32>(mx);
    const float M = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 0)),
                          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 32)));
    float ls = 0.0f;
    for (int sI = lane; sI < sws; sI += 64) {
      float wgt = 0.0f;
      if (sI < np) {
        const float ms = s_mx[h * np + sI];
        wgt = ms != NEG_INF ? fast_exp2(ms - M) : 0.0f;
        ls = __builtin_fmaf(wgt, s_ls[h * np + sI], ls);
      }
      s_w[h * sws + sI] = wgt;
    }
    ls = lane_group_sum<32>(ls);
    // (read by every lane: inside the lane-0 branch the compiler computed the half
    // sums in lane 0 alone, and lane 32 was read before its own sum)
    const float L = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 0)) +
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 32));
    if (lane == 0) s_L[h] = L;
  }
  __syncthreads();
  // every output: the weighted sum of its partials (the first PF branch-free: weights
  // past np are 0; the rest, for plans above PF splits, in chunks of PF loads)
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = threadIdx.x + NT * u;
    if (idx < G * HD) {
      const int h = idx / HD, d = idx % HD;
      const float* wh = s_w + h * sws;
      float A = 0.0f;
#pragma unroll
      for (int sI = 0; sI < PF; ++sI) A = __builtin_fmaf(pre[u][sI], wh[sI], A);
      for (int s0 = PF; s0 < np; s0 += PF) {
        float x[PF];
#pragma unroll
        for (int t = 0; t < PF; ++t)
          x[t] = s0 + t < np ? fetch(a.ws_acc + (pbase + (size_t)h * nps + s0 + t) * HD + d) : 0.0f;
#pragma unroll
        for (int t = 0; t < PF; ++t)
          if (s0 + t < np) A = __builtin_fmaf(x[t], wh[s0 + t], A);
      }
      a.out[(size_t)(b * a.Hq + kvh * G + h) * HD + d] = A / s_L[h];
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#ifdef KVQ_TIMELINE
  if (threadIdx.x == 0) tl_put(a, 14, tl_now());
#endif
}

template <int G, bool SK, bool RC, bool PG = false, bool H16 = false>
hipError_t launch_gs(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  switch (HD / a.gk) {
    case 1: return launch_kernel(decode_int4_mfma_kernel<G, 1, false, SK, RC, PG, H16>, grid, dim3(NT), a, s);
    case 2: return launch_kernel(decode_int4_mfma_kernel<G, 2, false, SK, RC, PG, H16>, grid, dim3(NT), a, s);
    case 4:
      if constexpr (G <= 4) return launch_kernel(decode_int4_mfma_kernel<G, 4, false, SK, RC, PG, H16>, grid, dim3(NT), a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// (sinks, recent fp16 rows and pages are not combined: the library rejects such caches;
// fp16 scales take the contiguous and the paged instances, a cache with sinks the
// split-K kernel)
template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  if (a.pages.size) return a.sinks || a.recent ? hipErrorInvalidValue : launch_gs<G, false, false, true>(a, s);
  if (a.recent) return a.sinks ? hipErrorInvalidValue : launch_gs<G, false, true>(a, s);
  return a.sinks ? launch_gs<G, true, false>(a, s) : launch_gs<G, false, false>(a, s);
}
template <int G>
hipError_t launch_g16(const DecodeArgs& a, hipStream_t s) {
  if (a.sinks || a.recent) return hipErrorInvalidValue;
  return a.pages.size ? launch_gs<G, false, false, true, true>(a, s)
                      : launch_gs<G, false, false, false, true>(a, s);
}

// ---------------------------------------------------------------------------------------
// Chunked prefill: multi-query causal attention over the INT4 cache
// (lpnh.cn/news/2042373 section 1.1: the prefill computes every position of a prompt
// at once, where decode computes one).  A chunk of nq new tokens per sequence, whose
// K/V rows are already in the cache at positions [len - nq, len), attends causally:
// query i, at position len - nq + i, sees positions [lo_i, len - nq + i] with
// lo_i = max(0, len - nq + i - window + 1) under a window, else 0.  Every cached row now
// meets G * nq query rows, so the work is a dense contraction and the matrix cores bound
// it, not HBM.
//
// Workgroup: (query block, KV head, sequence), PF_WAVES waves.  Wave w owns NCB column
// blocks of 16 query rows: column c of block cb is head c % G of query
// qb0 + (w * NCB + cb) * 16 / G + c / G.  All waves walk the same K/V tiles (the decode
// kernel's 32-position LDS tile layout and transfers): tile t is staged by wave
// t % PF_WAVES into slot t % PF_NB of one ring, and one barrier per tile both publishes it
// (its wave waited for its transfers first) and frees the slot the next transfer reuses.
//   q.K   per tile half T and K group g (64 dims): A = the half's 16 K rows, k = 32 dims
//         of group g (lane quarter j: dims 64 g + 16 j + 8 c2 + 0..7, c2 = 0, 1),
//         B = q of the block's 16 columns at the same dims; two MFMAs per (T, g), whose
//         sum is scaled by the group's K scale: z = sum_g sK(g) (q . codes_g).  (With
//         one K group of 128 the scale slot holds the same scale twice.)
//   P.V   as in decode: A = V codes (rows = 16 dims, k = 32 positions), B = the lane's
//         own 8 values of P' = p~ * sV as fp16 hi and lo, in two MFMAs per dim group
//         (every column is a query row, so the parts cannot share one MFMA here).
// The online softmax, the V-scale normalizer and the masks are the decode kernel's, with
// each column's own horizon.
constexpr int PF_WAVES = 4;
constexpr int PF_NB = 2;      // the prefill's ring: one tile ahead of the one in use
constexpr int PF_NT = PF_WAVES * 64;
constexpr int PF_NCB = 2;   // column blocks (16 query rows each) per wave: each wave's
                            // K and V operand conversions serve 32 columns (232 VGPRs, two
                            // waves per SIMD): 508 vs 454 TFLOP/s with one block

struct TileDataPF {
  u32x2 k[2][2];     // [T][g]: dims 64 g + 16 j .. + 15 of tile row r of half T
  u32x4 sk[2][2];    // [T][g]: K scales of rows 16 T + 4 j .. + 3, group g
  uint32_t v[2][4];  // [T][i]: dword r of V row 16 T + 4 j + i
  u32x4 sv[2];       // [T]: V scales of rows 16 T + 4 j .. + 3
};

struct LaneOffsPF {
  int k[2];          // group g's 8-byte piece of row r (half 0; + 1024 for half 1)
  int v[4];
};

// The 18 LDS reads of a tile for one lane, in one asm statement that waits for them
// (for the reason given at read_tile).
template <int NGK>
__device__ __forceinline__ TileDataPF read_tile_pf(const uint8_t* lb, const LaneOffsPF& lo, int j) {
  using L = Slot<NGK>;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_vptr)lb;
  const uint32_t ak0 = base + L::K_OFF + lo.k[0], ak1 = base + L::K_OFF + lo.k[1];
  const uint32_t ask = base + L::SK_OFF + 16 * j, asv = base + L::SV_OFF + 16 * j;
  const uint32_t av0 = base + L::V_OFF + lo.v[0], av1 = base + L::V_OFF + lo.v[1];
  const uint32_t av2 = base + L::V_OFF + lo.v[2], av3 = base + L::V_OFF + lo.v[3];
  TileDataPF d;
  asm volatile(
      "ds_read_b64 %0, %18\n\t"
      "ds_read_b64 %1, %19\n\t"
      "ds_read_b64 %2, %18 offset:1024\n\t"
      "ds_read_b64 %3, %19 offset:1024\n\t"
      "ds_read_b128 %4, %20\n\t"
      "ds_read_b128 %5, %20 offset:128\n\t"
      "ds_read_b128 %6, %20 offset:64\n\t"
      "ds_read_b128 %7, %20 offset:192\n\t"
      "ds_read_b32 %8, %22\n\t"
      "ds_read_b32 %9, %23\n\t"
      "ds_read_b32 %10, %24\n\t"
      "ds_read_b32 %11, %25\n\t"
      "ds_read_b32 %12, %22 offset:1024\n\t"
      "ds_read_b32 %13, %23 offset:1024\n\t"
      "ds_read_b32 %14, %24 offset:1024\n\t"
      "ds_read_b32 %15, %25 offset:1024\n\t"
      "ds_read_b128 %16, %21\n\t"
      "ds_read_b128 %17, %21 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d.k[0][0]), "=&v"(d.k[0][1]), "=&v"(d.k[1][0]), "=&v"(d.k[1][1]),
        "=&v"(d.sk[0][0]), "=&v"(d.sk[0][1]), "=&v"(d.sk[1][0]), "=&v"(d.sk[1][1]),
        "=&v"(d.v[0][0]), "=&v"(d.v[0][1]), "=&v"(d.v[0][2]), "=&v"(d.v[0][3]),
        "=&v"(d.v[1][0]), "=&v"(d.v[1][1]), "=&v"(d.v[1][2]), "=&v"(d.v[1][3]),
        "=&v"(d.sv[0]), "=&v"(d.sv[1])
      : "v"(ak0), "v"(ak1), "v"(ask), "v"(asv), "v"(av0), "v"(av1), "v"(av2), "v"(av3)
      : "memory");
  return d;
}

// H16: fp16 scales (KVQ_INT4_G16), transferred and converted as in the decode kernel.
template <int G, int NGK, int NCB, bool PG, bool H16 = false>
// (at least two workgroups per CU: at most 256 registers per lane, two waves per SIMD)
__global__ void __launch_bounds__(PF_NT, 2) prefill_int4_mfma_kernel(DecodeArgs a) {
  using L = Slot<NGK>;
  constexpr int QPC = 16 / G;                  // queries per column block
  constexpr int QWG = PF_WAVES * NCB * QPC;    // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t ring[PF_NB * L::BYTES];

  // Workgroups reach the 8 XCDs in turn, in dispatch order (x fastest).  They are
  // renumbered so that each XCD runs whole (sequence, KV head) units, all query blocks of
  // a unit side by side: those walk the same K/V tiles at about the same pace, so a tile
  // comes from HBM into that XCD's L2 once rather than once per XCD.  (Any order is
  // correct; this one only saves traffic.)
  const int nqb = gridDim.x;
  const int nwg = nqb * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + nqb * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xcd = lin & 7, per = nwg >> 3, rem = nwg & 7;
  const int vid = xcd * per + min(xcd, rem) + (lin >> 3);
  const int unit = vid / nqb;
  const int qb0 = (vid - unit * nqb) * QWG, kvh = unit % a.Hkv, b = unit / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int len = a.lens[b];
  const int nq = a.nq;
  const int p0 = len - nq;                     // position of query 0
  const int W = a.window;
  // the workgroup's queries [qb0, qe) and the positions they attend
  const int qe = min(nq, qb0 + QWG);
  const int hi_last = p0 + qe - 1;
  const int lo_first = W > 0 ? max(0, p0 + qb0 - W + 1) : 0;
  const int min_hi = p0 + qb0;                 // the first query's position
  const int max_lo = W > 0 ? max(0, hi_last - W + 1) : 0;
  const int tbase = lo_first & ~(TILE - 1);    // tiles from a multiple of 32 (paged layout)
  const int pe = hi_last + 1;
  const int ntiles = (pe - tbase + TILE - 1) / TILE;
  const size_t row0 = (size_t)(b * a.Hkv + kvh) * a.cap;
  const auto dof = dma_offsets<NGK>(lane);
  [[maybe_unused]] UnitBufs ubufs;
  if constexpr (!PG) ubufs = unit_bufs<NGK, H16>(a, row0);
  auto issue = [&](int t) {
    uint8_t* lb = ring + (t % PF_NB) * L::BYTES;
    const int t0 = tbase + TILE * t;
    if constexpr (PG) issue_tile_pg<NGK, H16>(a, b, kvh, t0, lo_first, pe, lb, lane, dof);
    else issue_tile<NGK, false, H16>(a, row0, t0, pe, 0, 0, lb, lane, dof, ubufs);
  };

  // ---- the columns: q as the B operands of the four (g, c2) MFMAs, -8 * (sum of each
  // group's q) for the nibble bias, and each column's horizon [clo, chi]
  half8 qop[NCB][4];
  float qbias[NCB][2];
  int chi[NCB], clo[NCB], cq[NCB];
  const int hh = r % G;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int qi = qb0 + (wave * NCB + cb) * QPC + r / G;
    const bool live = qi < qe;
    cq[cb] = live ? qi : -1;
    const int pq = p0 + qi;
    chi[cb] = live ? pq : -1;                  // (a junk column attends nothing)
    clo[cb] = W > 0 ? max(0, pq - W + 1) : 0;
    const uint16_t* qrow = a.q + (((size_t)b * a.Hq + kvh * G + hh) * nq + (live ? qi : 0)) * HD;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float qs = 0.0f;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 raw = live ? *reinterpret_cast<const u32x4*>(qrow + 64 * g + 16 * j + 8 * c2)
                               : (u32x4){0u, 0u, 0u, 0u};
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        H8 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {   // slot 2p: element p, slot 2p + 1: element p + 4
          const uint32_t lo16 = (w[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
          const uint32_t hi16 = (w[2 + (p >> 1)] >> (16 * (p & 1))) & 0xFFFFu;
          o.u[p] = lo16 | (hi16 << 16);
          f16x2 h2 = __builtin_bit_cast(f16x2, o.u[p]);
          const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
          qs = __builtin_amdgcn_fdot2(h2, one2, qs, false);
          if (p & 1) {   // slots of nibbles taken at bits 4..7 (16 times larger): q / 16
            const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
            h2 = h2 * sixteenth;
            o.u[p] = __builtin_bit_cast(uint32_t, h2);
          }
        }
        qop[cb][2 * g + c2] = o.h;
      }
      qbias[cb][g] = -8.0f * sum_over_j(qs);
    }
  }

  // per-lane LDS offsets: K rows r (group g's 8-byte piece), V dwords r of rows 4 j + i
  LaneOffsPF lo;
  {
    const int P = rowinv(r);
#pragma unroll
    for (int g = 0; g < 2; ++g) lo.k[g] = P * 64 + 16 * ((2 * g + (j >> 1)) ^ chunk_swz(P)) + 8 * (j & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int Pv = rowinv(4 * j + i);
      lo.v[i] = Pv * 64 + 16 * ((r >> 2) ^ chunk_swz(Pv)) + 4 * (r & 3);
    }
  }

  State st[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) st[cb].oacc[e] = (floatx4){0.f, 0.f, 0.f, 0.f};
    st[cb].m = empty_max(a.qscale);
    st[cb].l = 0.0f;
    st[cb].lvs = 0;
  }

  // ---- the tile loop: tile t staged by wave t % PF_WAVES, one tile ahead (two ahead, in a
  // 3-slot ring, was 1.7% slower)
  if (wave == 0 && ntiles > 0) issue(0);
  for (int k = 0; k < ntiles; ++k) {
    // a wave has at most one tile in flight (its tiles are PF_WAVES apart and it waits
    // for each before the next is issued), so vmcnt(0) waits for exactly tile k
    if (wave == k % PF_WAVES) wait_vmcnt<0>();
    lds_barrier();   // tile k visible to every wave; every wave done with tile k - 1
    if (k + 1 < ntiles && wave == (k + 1) % PF_WAVES) issue(k + 1);   // into tile k - 1's slot
    const int t0 = tbase + TILE * k;
    TileDataPF td = read_tile_pf<NGK>(ring + (k % PF_NB) * L::BYTES, lo, j);
    if constexpr (H16) {   // fp16 scales in the low halves of their dwords (dma_scale)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        td.sk[T][0] = f16lo_to_f32(td.sk[T][0]);
        td.sk[T][1] = f16lo_to_f32(td.sk[T][1]);
        td.sv[T] = f16lo_to_f32(td.sv[T]);
      }
    }
    // K operands of the tile (shared by the column blocks): [T][g][c2]
    half8 ka[2][2][2];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        ka[T][g][0] = unpack_word_u(td.k[T][g].x);
        ka[T][g][1] = unpack_word_u(td.k[T][g].y);
      }
    const floatx4 sk00 = __builtin_bit_cast(floatx4, td.sk[0][0]), sk01 = __builtin_bit_cast(floatx4, td.sk[0][1]);
    const floatx4 sk10 = __builtin_bit_cast(floatx4, td.sk[1][0]), sk11 = __builtin_bit_cast(floatx4, td.sk[1][1]);
    const floatx4 sv0 = __builtin_bit_cast(floatx4, td.sv[0]), sv1 = __builtin_bit_cast(floatx4, td.sv[1]);
    float svmax = max3_raw(max3_raw(sv0[0], sv0[1], sv0[2]), max3_raw(sv0[3], sv1[0], sv1[1]),
                           max_raw(sv1[2], sv1[3]));
    // (uniform) positions past the earliest query or before the latest window start
    const bool masked = t0 + TILE - 1 > min_hi || t0 < max_lo;
    H8 phi[NCB], plo[NCB];   // each column block's P' (fp16 hi and lo parts), B operands of P.V
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float z[2][4];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        floatx4 c0 = (floatx4){0.f, 0.f, 0.f, 0.f}, c1 = c0;
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[T][0][0], qop[cb][0], c0, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[T][0][1], qop[cb][1], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[T][1][0], qop[cb][2], c1, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[T][1][1], qop[cb][3], c1, 0, 0, 0);
        const floatx4 s0 = T ? sk10 : sk00, s1 = T ? sk11 : sk01;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          z[T][i] = __builtin_fmaf(__builtin_fmaf(c0[i], 16777216.0f, qbias[cb][0]), s0[i],
                                   __builtin_fmaf(c1[i], 16777216.0f, qbias[cb][1]) * s1[i]);
      }
      if (masked) {
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = t0 + 16 * T + 4 * j + i;
            if (p > chi[cb] || p < clo[cb]) z[T][i] = NEG_INF;
          }
      }
      float mx = max3_raw(max3_raw(z[0][0], z[0][1], z[0][2]), max3_raw(z[0][3], z[1][0], z[1][1]),
                          max_raw(z[1][2], z[1][3]));
      mx = max_over_j(mx);
      const float mq = tile_update(st[cb], mx, svmax, a.qscale);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const floatx4 sv = T ? sv1 : sv0;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float pa = fast_exp2(__builtin_fmaf(z[T][i], a.qscale, -mq));
          const float pb = fast_exp2(__builtin_fmaf(z[T][i + 1], a.qscale, -mq));
          st[cb].l += pa + pb;
          split_hi_lo(pa * sv[i], pb * sv[i + 1], phi[cb].u[2 * T + i / 2], plo[cb].u[2 * T + i / 2]);
        }
      }
    }
    // ---- P.V, one dim group at a time (its V operand converted just before its MFMAs,
    // so that only one group's operand is live): byte halves of two rows' dwords give the
    // (row, row + 1) pairs of 4 dims
    uint32_t xlo[4], xhi[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const int T = pr >> 1, i = 2 * (pr & 1);
      xlo[pr] = __builtin_amdgcn_perm(td.v[T][i + 1], td.v[T][i], 0x05040100u);
      xhi[pr] = __builtin_amdgcn_perm(td.v[T][i + 1], td.v[T][i], 0x07060302u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      H8 v;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t x = e < 4 ? xlo[pr] : xhi[pr];
        const uint32_t x8 = x >> 8;
        switch (e & 3) {
          case 0: v.u[pr] = v_pair_f16<0>(x, x8); break;
          case 1: v.u[pr] = v_pair_f16<1>(x, x8); break;
          case 2: v.u[pr] = v_pair_f16<2>(x, x8); break;
          default: v.u[pr] = v_pair_f16<3>(x, x8); break;
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        st[cb].oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v.h, phi[cb].h, st[cb].oacc[e], 0, 0, 0);
        st[cb].oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v.h, plo[cb].h, st[cb].oacc[e], 0, 0, 0);
      }
    }
  }

  // ---- outputs: lane (column r, j) holds dims 8 (4 j + i) + e of its column
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int e = 1; e < 8; e += 2) st[cb].oacc[e] *= 0.0625f;   // see v_pair_f16
    const float inv = 1.0f / sum_over_j(st[cb].l);
    if (cq[cb] >= 0) {
      float* orow = a.out + (((size_t)b * a.Hq + kvh * G + hh) * nq + cq[cb]) * HD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4* dst = reinterpret_cast<float4*>(orow + 8 * (4 * j + i));
        dst[0] = make_float4(st[cb].oacc[0][i] * inv, st[cb].oacc[1][i] * inv,
                             st[cb].oacc[2][i] * inv, st[cb].oacc[3][i] * inv);
        dst[1] = make_float4(st[cb].oacc[4][i] * inv, st[cb].oacc[5][i] * inv,
                             st[cb].oacc[6][i] * inv, st[cb].oacc[7][i] * inv);
      }
    }
  }
}

template <int G, int NCB, bool PG, bool H16>
hipError_t launch_pf_g(const DecodeArgs& a, hipStream_t s) {
  constexpr int QWG = PF_WAVES * NCB * (16 / G);
  const dim3 grid((a.nq + QWG - 1) / QWG, a.Hkv, a.B);
  switch (HD / a.gk) {
    case 1: return launch_kernel(prefill_int4_mfma_kernel<G, 1, NCB, PG, H16>, grid, dim3(PF_NT), a, s);
    case 2: return launch_kernel(prefill_int4_mfma_kernel<G, 2, NCB, PG, H16>, grid, dim3(PF_NT), a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool PG, bool H16>
hipError_t launch_pf(const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  switch (q_group) {
    case 1: return launch_pf_g<1, PF_NCB, PG, H16>(a, s);
    case 2: return launch_pf_g<2, PF_NCB, PG, H16>(a, s);
    case 4: return launch_pf_g<4, PF_NCB, PG, H16>(a, s);
    case 8: return launch_pf_g<8, PF_NCB, PG, H16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool SK, bool PG = false>
hipError_t launch_i8(const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  switch (q_group) {
    case 1: return launch_kernel(decode_int4_mfma_kernel<1, 2, true, SK, false, PG>, grid, dim3(NT), a, s);
    case 2: return launch_kernel(decode_int4_mfma_kernel<2, 2, true, SK, false, PG>, grid, dim3(NT), a, s);
    case 4: return launch_kernel(decode_int4_mfma_kernel<4, 2, true, SK, false, PG>, grid, dim3(NT), a, s);
    case 8: return launch_kernel(decode_int4_mfma_kernel<8, 2, true, SK, false, PG>, grid, dim3(NT), a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_int4_eligible(int32_t head_dim, int32_t group_k, int32_t group_v, int32_t cap,
                        int32_t q_group) {
  if (head_dim != HD || group_v != HD || group_k < 32 || group_k > HD || cap < TILE) return false;
  if (q_group != 1 && q_group != 2 && q_group != 4 && q_group != 8) return false;
  return q_group * (HD / group_k) <= 16;   // (K group, head) pairs fit the 16 MFMA columns
}

int32_t plan_splits_mfma(int32_t units, int32_t span) {
  const int32_t target_wg = 256;        // one 8-wave workgroup per CU on 256 CUs
  const int32_t min_rows = 1024;        // >= 4 tiles per wave
  int32_t n = (target_wg + units - 1) / units;
  const int32_t by_span = (span + min_rows - 1) / min_rows;
  if (n > by_span) n = by_span;
  if (n > 1024) n = 1024;
  return n < 1 ? 1 : n;
}

bool mfma_int4h_eligible(const kvq_cache_desc* d, int32_t q_group) {
  return d->format == KVQ_INT4_G16 && d->sinks == 0 && d->recent == 0 &&
         mfma_int4_eligible(d->head_dim, d->group_k, d->group_v, d->capacity, q_group);
}

bool fused_append_supported(const kvq_cache_desc* d, int32_t q_group) {
  // the matrix-core kernel codes the row for INT4 (either scale type); the split-K
  // kernel for the codecs and for INT4 with fp16 scales beside sinks or other shapes
  if (is_codec(d->format) || d->format == KVQ_INT4_G16) return true;
  return d->format == KVQ_INT4_G &&
         mfma_int4_eligible(d->head_dim, d->group_k, d->group_v, d->capacity, q_group);
}

hipError_t launch_decode_int4_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  switch (q_group) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_int4h_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  switch (q_group) {
    case 1: return launch_g16<1>(a, s);
    case 2: return launch_g16<2>(a, s);
    case 4: return launch_g16<4>(a, s);
    case 8: return launch_g16<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

bool mfma_int8_eligible(int32_t head_dim, int32_t cap, int32_t q_group) {
  return head_dim == HD && cap >= TILE8 &&
         (q_group == 1 || q_group == 2 || q_group == 4 || q_group == 8);
}

hipError_t launch_prefill_int4_mfma(const DecodeArgs& a, int32_t q_group, bool fp16_scales,
                                    hipStream_t s) {
  if (fp16_scales)
    return a.pages.size ? launch_pf<true, true>(a, q_group, s) : launch_pf<false, true>(a, q_group, s);
  return a.pages.size ? launch_pf<true, false>(a, q_group, s) : launch_pf<false, false>(a, q_group, s);
}

hipError_t launch_decode_int8_mfma(const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  if (a.pages.size) return a.sinks ? hipErrorInvalidValue : launch_i8<false, true>(a, q_group, s);
  return a.sinks ? launch_i8<true>(a, q_group, s) : launch_i8<false>(a, q_group, s);
}

}  // namespace kvq
