/* Exhaustive host check of the quantizers' scalar arithmetic (kvq_arith.h): for every
 * positive fp16 amax a, every fp16 x with |x| <= a, the reciprocal + FMA-corrected
 * quotient must equal the IEEE fp32 quotient fl32(x / s) bit for bit, the INT4 /
 * INT8 scale helpers must equal the IEEE quotients a/7 and max(a/127, 1e-8), and the
 * code the kernels form (clamp, then round by one add) must equal the rule's
 * clamp(rint(x / s)) as a two's complement nibble / byte.
 * Usage: arith_exhaustive int4|int8.  Prints the number of mismatches; exit 0 iff none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq_arith.h"

static float fp16_to_f32(uint16_t h) {
  const uint32_t e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
  return (h >> 15) ? -v : v;
}

int main(int argc, char** argv) {
  const int int8 = argc > 1 && strcmp(argv[1], "int8") == 0;
  long long pairs = 0, bad = 0, bad_scale = 0, bad_code = 0;
  const float lo = int8 ? -128.0f : -7.0f, hi = int8 ? 127.0f : 7.0f;
  const uint32_t mask = int8 ? 255u : 15u;
  for (uint32_t ha = 1; ha < 0x7c00; ++ha) {
    const float a = fp16_to_f32((uint16_t)ha);
    const float s = int8 ? kvq_int8_scale(a) : kvq_int4_scale(a);
    volatile float ref_s = int8 ? a / 127.0f : a / 7.0f;
    const float want_s = int8 ? (ref_s < 1e-8f ? 1e-8f : ref_s) : ref_s;
    if (s != want_s) ++bad_scale;
    const float r = 1.0f / s;
    for (uint32_t hx = 0; hx <= ha; ++hx) {
      const float xp = fp16_to_f32((uint16_t)hx);
      for (int sg = 0; sg < 2; ++sg) {
        const float x = sg ? -xp : xp;
        volatile float ref = x / s;
        ++pairs;
        const float q = kvq_div_exact(x, s, r);
        if (q != ref) ++bad;
        const uint32_t code = kvq_round_bits(fminf(fmaxf(q, lo), hi)) & mask;
        const uint32_t want = (uint32_t)(int)fminf(fmaxf(rintf(ref), lo), hi) & mask;
        if (code != want) ++bad_code;
      }
    }
  }
  printf("%s pairs=%lld quotient_mismatches=%lld scale_mismatches=%lld code_mismatches=%lld\n",
         int8 ? "int8" : "int4", pairs, bad, bad_scale, bad_code);
  return (bad || bad_scale || bad_code) ? 1 : 0;
}
