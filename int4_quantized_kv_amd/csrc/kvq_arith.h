// kvq_arith.h -- scalar arithmetic of the quantizers, shared by the gfx950 kernels and
// by a host-compiled exhaustive check of the same instruction sequence.
//
// The INT4 rule (lpnh.cn/news/2042373, section 2.1) and the INT8 rule
// (bxzpzcl.cn/news/2871434, section 3.1) both need q = round_half_even(fl32(x / s)).
// A correctly rounded IEEE divide costs ~10 VALU instructions on gfx950.  Here the
// quotient is formed from one reciprocal per group instead:
//   r  = fl32(1 / s)                 (one IEEE divide per group)
//   y0 = fl32(x * r)
//   e  = fma(-y0, s, x)              (exact residual x - y0 * s)
//   y1 = fma(e, r, y0)               (Markstein-style correction)
// For every fp16 x and every scale s the quantizers can produce from an fp16 amax
// with |x| <= amax (s = fl32(amax/7), and s = max(fl32(amax/127), 1e-8)), y1 equals
// fl32(x / s) bit for bit; the host test enumerates all ~1e9 such pairs per rule.
#ifndef KVQ_ARITH_H
#define KVQ_ARITH_H

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define KVQ_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define KVQ_HD static inline
#endif

// fl32(x / s) given r = fl32(1 / s), for the (x, s) domain described above.
KVQ_HD float kvq_div_exact(float x, float s, float r) {
  float y0 = x * r;
  float e = __builtin_fmaf(-y0, s, x);
  return __builtin_fmaf(e, r, y0);
}

// INT4 group scale from the group's amax: fl32(amax / 7), 1 for an all-zero group.
// The quotient by the constant is the corrected product above with r = fl32(1/7)
// (constant-folded); for every fp16 amax it equals the IEEE quotient (checked
// exhaustively on the host), at 3 instructions instead of a full divide.
KVQ_HD float kvq_int4_scale(float amax) {
  float s = kvq_div_exact(amax, 7.0f, 1.0f / 7.0f);
  return s == 0.0f ? 1.0f : s;
}

// INT8 per-token scale: max(fl32(amax / 127), 1e-8f), the quotient formed as above.
KVQ_HD float kvq_int8_scale(float amax) {
  float s = kvq_div_exact(amax, 127.0f, 1.0f / 127.0f);
  return s < 1e-8f ? 1e-8f : s;
}

// rint(q) (half to even) as the low bits of a word, for |q| <= 128: the fp32 sum
// q + 1.5 * 2^23 lies in [2^23, 2^24), where the spacing is 1, so the addition rounds q
// to an integer (to nearest, ties to even) and leaves 0x400000 + rint(q) in the
// mantissa; 0x400000 is a multiple of 256, so the low 4 (8) bits are the two's
// complement nibble (byte) of rint(q).  One add in place of round, convert and mask.
KVQ_HD uint32_t kvq_round_bits(float q) {
  union {
    float f;
    uint32_t u;
  } v;
  v.f = q + 12582912.0f;
  return v.u;
}

#endif  // KVQ_ARITH_H
