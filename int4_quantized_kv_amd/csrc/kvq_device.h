// kvq_device.h -- small device helpers shared by the gfx950 kernels.
#ifndef KVQ_DEVICE_H
#define KVQ_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kvq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Eight consecutive fp16 values (one 16-byte load) widened to fp32 (exact).
__device__ __forceinline__ void load8_f16(const uint16_t* p, float x[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    x[2 * i] = (float)h.x;
    x[2 * i + 1] = (float)h.y;
  }
}

// Eight fp16 values already loaded as one 16-byte word, widened to fp32 (exact).
__device__ __forceinline__ void f16x8_unpack(const uint4& r, float x[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    x[2 * i] = (float)h.x;
    x[2 * i + 1] = (float)h.y;
  }
}

// Signed 4-bit field j (0..7) of a packed word, as an int in -8..7.
__device__ __forceinline__ int nib_s(uint32_t w, int j) {
  return (int32_t)(w << (28 - 4 * j)) >> 28;
}

// Unsigned 4-bit field j of a packed word.
__device__ __forceinline__ int nib_u(uint32_t w, int j) { return (w >> (4 * j)) & 15; }

// x from lane (lane ^ M) within aligned groups of 2M lanes (M = 1, 2, 4, 8, 16), by DPP
// and the gfx950 row-pair swap (VALU, no LDS round trip): partners 1 and 2 are quad
// permutes, 4 is a quad xor-3 followed by a half-row mirror (lane i ^ 7), 8 is a
// rotation by 8 within a 16-lane row, 16 is v_permlane16_swap of a register with a copy
// of itself (one copy then holds row r, the other row r ^ 1) and a select.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float xor_lane(float x, int lane_in_group) {
  if constexpr (M == 1) return dpp_mov<0xB1>(x);            // quad_perm [1, 0, 3, 2]
  else if constexpr (M == 2) return dpp_mov<0x4E>(x);       // quad_perm [2, 3, 0, 1]
  else if constexpr (M == 4) return dpp_mov<0x141>(dpp_mov<0x1B>(x));   // xor 3, mirror 8
  else if constexpr (M == 8) return dpp_mov<0x128>(x);      // row_ror:8
  else {
    static_assert(M == 16, "partners 1 .. 16");
    uint32_t p = __builtin_bit_cast(uint32_t, x), q = p;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(p), "+v"(q));
    return __builtin_bit_cast(float, (lane_in_group & 16) ? p : q);
  }
}

// Unnormalized Sylvester Walsh-Hadamard transform of one row spread over `lpr`
// consecutive lanes, each holding 8 consecutive elements (element 8*c + i in lane c).
// Butterflies (a, b) -> (a + b, a - b) over every bit of the element index; the
// three low bits are inside a lane, the others pair lane c with lane c ^ m.  All the
// row's lanes must be active.
template <int LPR>
__device__ __forceinline__ void wht_row(float v[8], int c) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  // the lane with bit M of c set keeps p - v, its partner v + p: both are fma(+-1, v, p),
  // which rounds the exact sum once, as the add / subtract does
  auto stage = [&](auto mtag) {
    constexpr int M = decltype(mtag)::value;
    const float sgn = (c & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sgn, v[i], xor_lane<M>(v[i], c));
  };
  if constexpr (LPR > 1) stage(std::integral_constant<int, 1>{});
  if constexpr (LPR > 2) stage(std::integral_constant<int, 2>{});
  if constexpr (LPR > 4) stage(std::integral_constant<int, 4>{});
  if constexpr (LPR > 8) stage(std::integral_constant<int, 8>{});
  if constexpr (LPR > 16) stage(std::integral_constant<int, 16>{});
}

// The codec's 15 decision thresholds as wave-uniform values, read at the point of the
// call (a kernel reads them at its start, so that their load is not on the critical path
// of the coder: the empty asm pins each value to a scalar register there).
struct Thresholds {
  float t[15];
};
__device__ __forceinline__ Thresholds load_thresholds(const float* thr) {
  Thresholds r;
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    float x = thr[k];
    asm volatile("" : "+s"(x));
    r.t[k] = x;
  }
  return r;
}

// The number of the 15 ascending thresholds strictly below u, by binary search: "t[k] < u"
// holds for a prefix of k, whose length is found bit by bit (8, 4, 2, 1), each step
// comparing u with the one threshold that splits what is left.  Equal to counting all
// 15 comparisons (u = NaN: 0) at about half the instructions.  The selects are bit
// selects in assembly: as plain selects of array elements the compiler turns them into
// a per-lane indexed load from a stack copy of the array.
__device__ __forceinline__ float bit_select(bool b, float x, float y) {   // b ? x : y
  const int m = b ? -1 : 0;
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ int count_below15(const Thresholds& th, float u) {
  const float* t = th.t;
  const bool b3 = t[7] < u;
  const bool b2 = bit_select(b3, t[11], t[3]) < u;
  const float t1a = bit_select(b2, t[13], t[9]), t1b = bit_select(b2, t[5], t[1]);
  const bool b1 = bit_select(b3, t1a, t1b) < u;
  const float q3 = bit_select(b1, t[14], t[12]), q2 = bit_select(b1, t[10], t[8]);
  const float q1 = bit_select(b1, t[6], t[4]), q0 = bit_select(b1, t[2], t[0]);
  const float t0 = bit_select(b3, bit_select(b2, q3, q2), bit_select(b2, q1, q0));
  return 8 * b3 + 4 * b2 + 2 * b1 + (t0 < u ? 1 : 0);
}

// Sum over the LPR lanes of a row, by the same xor pairings as wht_row (so every path
// that reduces a row this way gets the same bits).
template <int LPR>
__device__ __forceinline__ float row_xor_sum(float x, int c) {
  if constexpr (LPR > 1) x += xor_lane<1>(x, c);
  if constexpr (LPR > 2) x += xor_lane<2>(x, c);
  if constexpr (LPR > 4) x += xor_lane<4>(x, c);
  if constexpr (LPR > 8) x += xor_lane<8>(x, c);
  if constexpr (LPR > 16) x += xor_lane<16>(x, c);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Codec encode of one row spread over LPR = D/8 lanes (8 elements in lane c) for the
// WHT + Lloyd-Max codec ("长上下文内存大瘦身：LARQL 四大 KV 缓存引擎原理与横向对比",
// engine three): s = ||x||_2 / sqrt(D); the index of element i is the number of the
// 15 decision thresholds strictly below (H x / sqrt(D))_i / s (a zero row: / 1).  Every
// kernel that codes a row calls this, so all paths write the same codes.  x is
// overwritten (rotated); w gets the lane's 8 indices (element 8c + i in bits 4i..4i+3).
template <int LPR>
__device__ __forceinline__ void codec_encode_row(float x[8], int c, const Thresholds& thr,
                                                 uint32_t& w, float& s) {
  constexpr int D = LPR * 8;
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(x[j], x[j], ss);
  ss = row_xor_sum<LPR>(ss, c);
  wht_row<LPR>(x, c);
  s = sqrtf(ss / (float)D);
  const float inv = (1.0f / sqrtf((float)D)) / (s == 0.0f ? 1.0f : s);  // u = (H x / sqrt(D)) / s
  w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= (uint32_t)count_below15(thr, x[j] * inv) << (4 * j);
}

// 3-bit codec rows: the D indices packed back to back, index i in bits 3i .. 3i + 2 of
// the row read as a little-endian bit string (3D/8 bytes).  Lane c owns indices
// 8c .. 8c + 7, i.e. the 24 bits of bytes 3c .. 3c + 2.  The encoder, the dequantizer
// and the fused append convert between those 24 bits and the 4-bit codec's nibble word
// (index j in nibble j, values 0..7), so the coder and the level lookups are shared.
__device__ __forceinline__ uint32_t packed3_of_nibbles(uint32_t w) {   // nibble j -> bits 3j
  w &= 0x77777777u;
  w = (w & 0x07070707u) | ((w >> 1) & 0x38383838u);   // byte k: indices 2k, 2k+1 in 6 bits
  w = (w & 0x003F003Fu) | ((w >> 2) & 0x0FC00FC0u);   // half h: indices 4h .. 4h+3 in 12 bits
  return (w & 0x00000FFFu) | ((w >> 4) & 0x00FFF000u);
}
__device__ __forceinline__ uint32_t nibbles_of_packed3(uint32_t t) {   // bits 3j -> nibble j
  t = (t & 0x00000FFFu) | ((t & 0x00FFF000u) << 4);
  t = (t & 0x003F003Fu) | ((t & 0x0FC00FC0u) << 2);
  return (t & 0x07070707u) | ((t & 0x38383838u) << 1);
}
// lane c's 24 bits by byte accesses (encode, dequant, append: off the decode loop)
template <int LPR>
__device__ __forceinline__ void store_packed3(uint8_t* row, int c, uint32_t w) {
  const uint32_t t = packed3_of_nibbles(w);
  row[3 * c] = (uint8_t)t;
  row[3 * c + 1] = (uint8_t)(t >> 8);
  row[3 * c + 2] = (uint8_t)(t >> 16);
}
template <int LPR>
__device__ __forceinline__ uint32_t load_packed3(const uint8_t* row, int c) {
  return nibbles_of_packed3((uint32_t)row[3 * c] | ((uint32_t)row[3 * c + 1] << 8) |
                            ((uint32_t)row[3 * c + 2] << 16));
}
// The decode loop fetches a row with one aligned dword per lane: lane 4m + i loads
// dword 3m + min(i, 2) of the row (its quad's 12 bytes; lanes 4m + 2 and 4m + 3 load the
// same dword), and packed3_bits later assembles its 24 bits from its own dword and the
// one of lane 4m + i - 1 (a quad DPP): i = 0: bytes 0-2 of its own; 1: the last byte of
// lane 4m's and the first two of its own; 2: the last two of lane 4m + 1's and the first
// of its own; 3: bytes 1-3 of its own.  Every lane of the quad must be active.
__device__ __forceinline__ int packed3_dword(int c) { return 3 * (c >> 2) + min(c & 3, 2); }
__device__ __forceinline__ uint32_t packed3_bits(uint32_t own, int i) {
  const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0x90, 0xF, 0xF, false);   // quad_perm [0, 0, 1, 2]
  const uint32_t lo = (i == 1 || i == 2) ? prev : own;
  return __builtin_amdgcn_alignbyte(own, lo, (uint32_t)((4 - i) & 3));
}

// Sum over aligned groups of LANES (2, 4, 8, 16 or 32) lanes, left in every lane of the
// group, without an LDS round trip: quad swaps for partners 1 and 2, the half-row and
// row mirrors (each pairs a lane with one in the other half of its group of 8 / 16)
// and, for 32 lanes, the gfx950 row-pair swap (v_permlane16_swap of a register with a
// copy of itself leaves row r in one and row r ^ 1 in the other; written in assembly,
// with the s_nop covering the VALU-write -> permlane-read hazard).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int LANES>
__device__ __forceinline__ float lane_group_sum(float x) {
  if (LANES >= 2) x = dpp_add<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  if (LANES >= 4) x = dpp_add<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  if (LANES >= 8) x = dpp_add<0x141>(x);   // row_half_mirror
  if (LANES >= 16) x = dpp_add<0x140>(x);  // row_mirror
  if (LANES >= 32) {
    uint32_t p = __builtin_bit_cast(uint32_t, x), q = p;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(p), "+v"(q));
    x = __builtin_bit_cast(float, p) + __builtin_bit_cast(float, q);
  }
  return x;
}

// The value of lane L (a constant) in every lane.
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Maximum over aligned groups of LANES lanes, by the same lane pairings: one
// v_max_f32_dpp per stage, in asm (fmaxf would first quiet signalling NaNs with a max of
// each operand with itself, and the builtin DPP move is not folded into the max; the
// values reduced here are never NaN).  Each stage starts with the two wait states a DPP
// read needs after a VALU write.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  float r;
  if constexpr (CTRL == 0xB1)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else if constexpr (CTRL == 0x4E)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else if constexpr (CTRL == 0x141)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else {
    static_assert(CTRL == 0x140, "lane pairing");
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  }
  return r;
}
template <int LANES>
__device__ __forceinline__ float lane_group_max(float x) {
  if (LANES >= 2) x = dpp_max<0xB1>(x);
  if (LANES >= 4) x = dpp_max<0x4E>(x);
  if (LANES >= 8) x = dpp_max<0x141>(x);
  if (LANES >= 16) x = dpp_max<0x140>(x);
  if (LANES >= 32) {
    uint32_t p = __builtin_bit_cast(uint32_t, x), q = p;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(p), "+v"(q));
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(p), "v"(q));
    x = r;
  }
  return x;
}
// max(|x[0]|, ..., |x[7]|): four v_max3_f32 with absolute-value source modifiers.
__device__ __forceinline__ float abs_max8(const float (&x)[8]) {
  float m;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m) : "v"(x[0]), "v"(x[1]), "v"(x[2]));
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(m) : "v"(m), "v"(x[3]), "v"(x[4]));
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(m) : "v"(m), "v"(x[5]), "v"(x[6]));
  asm("v_max_f32 %0, %1, |%2|" : "=v"(m) : "v"(m), "v"(x[7]));
  return m;
}

// Enqueue `kernel(args)` and return the runtime's status for this launch only (the
// thread's last-error slot may hold an unrelated earlier status, e.g. a not-ready
// query made by the caller, so it is never consulted).
template <typename Args>
inline hipError_t launch_kernel(void (*kernel)(Args), dim3 grid, dim3 block, const Args& a,
                                hipStream_t s) {
  void* params[] = {const_cast<Args*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0, s);
}

}  // namespace kvq

#endif  // KVQ_DEVICE_H
