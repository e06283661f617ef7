// quant.hip -- INT4 group / INT8 per-token quantize (prefill + append) and dequantize.
//
// INT4 rule: lpnh.cn/news/2042373 section 2.1 (per group of g head_dim elements:
// s = amax/7, 1 for an all-zero group, q = clamp(round(x/s), -7, 7)); K groups of 64
// and V groups of 128 from its section 2.2.  INT8 rule: bxzpzcl.cn/news/2871434
// section 3.1 (per token and head: s = max(amax/127, 1e-8), q = clamp(round(x/s),
// -128, 127)).  Scales are fp32; x/s is rounded to fp32 and then half-to-even.
//
// Mapping: one lane owns 8 consecutive fp16 of a row (one 16-byte load); a row of
// D elements spans D/8 consecutive lanes, a group of g elements g/8 lanes, so the
// group amax is an xor-shuffle reduction inside the wave.  Each lane writes its 8
// codes as one 32-bit word (INT4) or one 64-bit word (INT8).  K and V are the two
// grid rows (blockIdx.y) of one launch.  Streaming kernel: HBM bound.
#include "kvq_arith.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ int slot_of(const SlotMap& m, int b, int t) {
  const int p = m.append ? m.pos[b] : m.start + t;
  return p % m.cap;
}

__global__ void __launch_bounds__(256) quant_int4_kernel(QuantArgs a) {
  const int isv = blockIdx.y;
  const uint16_t* src = isv ? a.v : a.k;
  uint32_t* codes = reinterpret_cast<uint32_t*>(isv ? a.v_codes : a.k_codes);
  float* scales = isv ? a.v_scales : a.k_scales;
  const int g = isv ? a.gv : a.gk;
  const int lpg = g >> 3, lpr = a.D >> 3, gpr = a.D / g;
  const uint32_t total = (uint32_t)a.rows * (uint32_t)lpr;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / lpr;
    const int c = (int)(i - row * lpr);
    float x[8];
    load8_f16(src + (size_t)i * 8, x);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
    // groups are lpg aligned consecutive lanes, entirely inside or outside the loop
    for (int m = 1; m < lpg; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
    const float s = kvq_int4_scale(am);
    const float r = 1.0f / s;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = kvq_div_exact(x[j], s, r);
      const float q = fminf(fmaxf(rintf(y), -7.0f), 7.0f);
      w |= ((uint32_t)(int)q & 15u) << (4 * j);
    }
    const uint32_t bh = row / (uint32_t)a.map.n;
    const int t = (int)(row - bh * a.map.n);
    const int b = (int)(bh / (uint32_t)a.Hkv);
    const size_t drow = (size_t)bh * a.map.cap + slot_of(a.map, b, t);
    codes[drow * lpr + c] = w;
    if ((c & (lpg - 1)) == 0) scales[drow * gpr + c / lpg] = s;
  }
}

__global__ void __launch_bounds__(256) quant_int8_kernel(QuantArgs a) {
  const int isv = blockIdx.y;
  const uint16_t* src = isv ? a.v : a.k;
  uint2* codes = reinterpret_cast<uint2*>(isv ? a.v_codes : a.k_codes);
  float* scales = isv ? a.v_scales : a.k_scales;
  const int lpr = a.D >> 3;
  const uint32_t total = (uint32_t)a.rows * (uint32_t)lpr;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / lpr;
    const int c = (int)(i - row * lpr);
    float x[8];
    load8_f16(src + (size_t)i * 8, x);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
    for (int m = 1; m < lpr; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
    const float s = kvq_int8_scale(am);
    const float r = 1.0f / s;
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = kvq_div_exact(x[j], s, r);
      const float q = fminf(fmaxf(rintf(y), -128.0f), 127.0f);
      const uint32_t byte = (uint32_t)(int)q & 255u;
      if (j < 4) w0 |= byte << (8 * j); else w1 |= byte << (8 * (j - 4));
    }
    const uint32_t bh = row / (uint32_t)a.map.n;
    const int t = (int)(row - bh * a.map.n);
    const int b = (int)(bh / (uint32_t)a.Hkv);
    const size_t drow = (size_t)bh * a.map.cap + slot_of(a.map, b, t);
    codes[drow * lpr + c] = make_uint2(w0, w1);
    if (c == 0) scales[drow] = s;
  }
}

// out[b, h, t, :] = fl32(code * scale) for positions start + t, t < n.
__global__ void __launch_bounds__(256) dequant_int4_kernel(DequantArgs a) {
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(a.codes);
  const int lpr = a.D >> 3, lpg = a.g >> 3, gpr = a.D / a.g;
  const uint32_t total = (uint32_t)a.B * a.Hkv * a.n * lpr;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / lpr;
    const int c = (int)(i - row * lpr);
    const uint32_t bh = row / (uint32_t)a.n;
    const int t = (int)(row - bh * a.n);
    const size_t drow = (size_t)bh * a.cap + (a.start + t) % a.cap;
    const uint32_t w = codes[drow * lpr + c];
    const float s = a.scales[drow * gpr + c / lpg];
    float4 o0, o1;
    o0.x = (float)nib_s(w, 0) * s; o0.y = (float)nib_s(w, 1) * s;
    o0.z = (float)nib_s(w, 2) * s; o0.w = (float)nib_s(w, 3) * s;
    o1.x = (float)nib_s(w, 4) * s; o1.y = (float)nib_s(w, 5) * s;
    o1.z = (float)nib_s(w, 6) * s; o1.w = (float)nib_s(w, 7) * s;
    float4* out = reinterpret_cast<float4*>(a.out + (size_t)i * 8);
    out[0] = o0;
    out[1] = o1;
  }
}

__global__ void __launch_bounds__(256) dequant_int8_kernel(DequantArgs a) {
  const uint2* codes = reinterpret_cast<const uint2*>(a.codes);
  const int lpr = a.D >> 3;
  const uint32_t total = (uint32_t)a.B * a.Hkv * a.n * lpr;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / lpr;
    const int c = (int)(i - row * lpr);
    const uint32_t bh = row / (uint32_t)a.n;
    const int t = (int)(row - bh * a.n);
    const size_t drow = (size_t)bh * a.cap + (a.start + t) % a.cap;
    const uint2 w = codes[drow * lpr + c];
    const float s = a.scales[drow];
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (float)(int8_t)((w.x >> (8 * j)) & 255u) * s;
      v[j + 4] = (float)(int8_t)((w.y >> (8 * j)) & 255u) * s;
    }
    float4* out = reinterpret_cast<float4*>(a.out + (size_t)i * 8);
    out[0] = make_float4(v[0], v[1], v[2], v[3]);
    out[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

inline int grid_for(uint64_t lanes) {
  uint64_t blocks = (lanes + 255) / 256;
  const uint64_t cap = 256ull * 16;  // enough resident waves to cover HBM latency
  return (int)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_quant_intq(int32_t format, const QuantArgs& a, hipStream_t s) {
  const uint64_t lanes = (uint64_t)a.rows * (a.D / 8);
  dim3 grid(grid_for(lanes), 2);
  return launch_kernel(format == KVQ_INT4_G ? quant_int4_kernel : quant_int8_kernel, grid,
                       dim3(256), a, s);
}

hipError_t launch_dequant_intq(int32_t format, const DequantArgs& a, hipStream_t s) {
  const uint64_t lanes = (uint64_t)a.B * a.Hkv * a.n * (a.D / 8);
  return launch_kernel(format == KVQ_INT4_G ? dequant_int4_kernel : dequant_int8_kernel,
                       dim3(grid_for(lanes)), dim3(256), a, s);
}

}  // namespace kvq
