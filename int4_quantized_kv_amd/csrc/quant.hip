// quant.hip -- INT4 group / INT8 per-token quantize (prefill + append) and dequantize.
//
// INT4 rule: lpnh.cn/news/2042373 section 2.1 (per group of g head_dim elements:
// s = amax/7, 1 for an all-zero group, q = clamp(round(x/s), -7, 7)); K groups of 64
// and V groups of 128 from its section 2.2.  INT8 rule: bxzpzcl.cn/news/2871434
// section 3.1 (per token and head: s = max(amax/127, 1e-8), q = clamp(round(x/s),
// -128, 127)).  Scales are fp32; x/s is rounded to fp32, clamped and then rounded
// half-to-even (clamping first is the same for integer bounds).  INT4 with fp16 scales
// runs the INT4 rule in fp16, as the page's code does on fp16 tensors: s = fl16(amax/7)
// (1 if 0), code = rne(fl16(x/s)); each quotient is the correctly rounded fp32 division
// rounded once more to fp16, which equals the correctly rounded fp16 quotient (fp32
// carries more than 2 * 11 + 2 significand bits).
//
// Mapping: one lane owns 8 consecutive fp16 of a row (one 16-byte load); a row of
// D elements spans D/8 consecutive lanes, a group of g elements g/8 lanes, so the
// group amax is a DPP reduction inside the wave.  Each lane writes its 8
// codes as one 32-bit word (INT4) or one 64-bit word (INT8).  K and V are the two
// grid rows (blockIdx.y) of one launch.  Streaming kernel: HBM bound.  Each lane takes
// U chunks of the grid-stride sequence per iteration and issues their loads before
// using any, so that enough bytes are in flight to cover the memory latency (a row's
// lanes are consecutive and the stride is a multiple of 256, so the lanes of a row or
// group are all in or all out of an iteration's chunk u).
constexpr int U = 4;
#include "kvq_arith.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// Grid: (chunks of a (b, h) pair, K or V (quantizers), pairs bh = blockIdx.z + k *
// gridDim.z; gridDim.z is capped at 65535).  A pair's
// rows are n consecutive source rows of D/8 16-byte chunks; chunk ci is row ci / lpr,
// lane-chunk ci % lpr (lpr a power of two: shifts).  The cache slot of row t is
// (base + t) mod cap with base < cap and t < n <= cap: one conditional subtract
// (cache_slot when the cache keeps sink slots ahead of its ring).
__device__ __forceinline__ int log2i(int x) { return 31 - __builtin_clz(x); }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));


template <bool INT8, bool H16 = false>
__device__ __forceinline__ void quant_pair(const QuantArgs& a, int bh) {
  const int isv = blockIdx.y;
  const int b = bh / a.Hkv;
  const uint16_t* src = (isv ? a.v : a.k);
  float* scales = isv ? a.v_scales : a.k_scales;
  const int g = INT8 ? a.D : (isv ? a.gv : a.gk);
  // lpr, lpg and gpr are powers of two (D in {64, 128, 256}, g a power of two >= 32)
  const int lpr = a.D >> 3, lsh = log2i(lpr), lpg = g >> 3, gsh = log2i(lpg);
  const int gprsh = log2i(a.D / g);
  const int cap = a.map.cap, sinks = a.map.sinks;
  const int p0 = a.map.append ? a.map.pos[b] : a.map.start;
  const int base = p0 % cap;
  const uint32_t npair = (uint32_t)a.map.n * (uint32_t)lpr;
  const uint4* srcp = reinterpret_cast<const uint4*>(src) + (size_t)bh * npair;
  const size_t row0 = (size_t)bh * cap;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i0 = blockIdx.x * blockDim.x + threadIdx.x; i0 < npair; i0 += U * stride) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = i0 + u * stride;
      if (i < npair) {   // non-temporal: every source byte is read once (+6% on a 3.4 GB layer)
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(srcp) + i);
        raw[u] = make_uint4(t.x, t.y, t.z, t.w);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = i0 + u * stride;
      if (i >= npair) break;
      const int t = (int)(i >> lsh), c = (int)(i & (lpr - 1));
      float x[8];
      f16x8_unpack(raw[u], x);
      float am = abs_max8(x);
      // a group is lpg aligned consecutive lanes, all of which take this chunk
      switch (lpg) {   // (uniform)
        case 4: am = lane_group_max<4>(am); break;
        case 8: am = lane_group_max<8>(am); break;
        case 16: am = lane_group_max<16>(am); break;
        default: am = lane_group_max<32>(am); break;
      }
      float sc;
      if (H16) {
        const float s16 = (float)(_Float16)(am / 7.0f);
        sc = s16 == 0.0f ? 1.0f : s16;
      } else {
        sc = INT8 ? kvq_int8_scale(am) : kvq_int4_scale(am);
      }
      const float r = 1.0f / sc;
      size_t drow;
      if (a.pages.size) {   // (uniform) paged layout: the page of position p0 + t
        drow = paged_row(a.pages, a.Hkv, b, bh - b * a.Hkv, p0 + t);
      } else {
        int slot;
        if (sinks) {   // (uniform) sink slots ahead of the ring
          slot = cache_slot(p0 + t, cap, sinks);
        } else {
          slot = base + t;
          if (slot >= cap) slot -= cap;
        }
        drow = row0 + slot;
      }
      if (!INT8 && a.recent) {   // (uniform) the call's last `recent` positions also
        const int p = p0 + t;    // go to the fp16 ring, row p mod recent, unchanged
        if (p >= p0 + a.map.n - a.recent) {
          uint4* ring = reinterpret_cast<uint4*>(isv ? a.v_recent : a.k_recent);
          ring[(((size_t)bh * a.recent + p % a.recent) << lsh) + c] = raw[u];
        }
      }
      if (INT8) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t byte = kvq_round_bits(fminf(fmaxf(kvq_div_exact(x[j], sc, r), -128.0f), 127.0f)) & 255u;
          if (j < 4) w0 |= byte << (8 * j); else w1 |= byte << (8 * (j - 4));
        }
        reinterpret_cast<uint2*>(isv ? a.v_codes : a.k_codes)[(drow << lsh) + c] = make_uint2(w0, w1);
        if (c == 0) scales[drow] = sc;
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float y = H16 ? (float)(_Float16)(x[j] / sc) : kvq_div_exact(x[j], sc, r);
          w |= (kvq_round_bits(fminf(fmaxf(y, -7.0f), 7.0f)) & 15u) << (4 * j);
        }
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(isv ? a.v_codes : a.k_codes) + (drow << lsh) + c);
        if ((c & (lpg - 1)) == 0) {
          if (H16) reinterpret_cast<_Float16*>(scales)[(drow << gprsh) + (c >> gsh)] = (_Float16)sc;
          else scales[(drow << gprsh) + (c >> gsh)] = sc;
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) quant_int4_kernel(QuantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) quant_pair<false>(a, bh);
}
__global__ void __launch_bounds__(256) quant_int8_kernel(QuantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) quant_pair<true>(a, bh);
}
__global__ void __launch_bounds__(256) quant_int4h_kernel(QuantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) quant_pair<false, true>(a, bh);
}

// out[b, h, t, :] = fl32(code * scale) for positions start + t, t < n; one (b, h) pair
// per blockIdx.z, mapped as the quantizers except that a lane owns half of a code
// word's chunk (4 values, 16 output bytes): the two lanes of a chunk read the same
// word, and each store instruction of a wave writes 1 KiB of consecutive output
// (owning whole chunks, a lane's two 16-byte stores leave every other 16 bytes of a
// 2 KiB span to the other store).
constexpr int UD = 1;   // half-chunks per lane per iteration (more gave less: see the launch)
template <bool INT8, bool H16 = false>
__device__ __forceinline__ void dequant_pair(const DequantArgs& a, int bh) {
  const int g = INT8 ? a.D : a.g;
  const int lpr = a.D >> 3, lsh = log2i(lpr), gsh = log2i(g >> 3), gprsh = log2i(a.D / g);
  const int cap = a.cap, sinks = a.sinks;
  const int base = a.start % cap;
  const uint32_t nhalf = 2u * (uint32_t)a.n * (uint32_t)lpr;
  const size_t row0 = (size_t)bh * cap;
  float4* outp = reinterpret_cast<float4*>(a.out) + (size_t)bh * nhalf;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t k0 = blockIdx.x * blockDim.x + threadIdx.x; k0 < nhalf; k0 += UD * stride) {
    uint32_t wr[UD];
    float sr[UD];
#pragma unroll
    for (int u = 0; u < UD; ++u) {
      const uint32_t k = k0 + u * stride;
      if (k < nhalf) {
        const uint32_t i = k >> 1;
        const int t = (int)(i >> lsh), c = (int)(i & (lpr - 1));
        size_t drow;
        if (a.pages.size) {   // (uniform) paged layout
          const int b = bh / a.Hkv;
          drow = paged_row(a.pages, a.Hkv, b, bh - b * a.Hkv, a.start + t);
        } else {
          int slot;
          if (sinks) {   // (uniform) sink slots ahead of the ring
            slot = cache_slot(a.start + t, cap, sinks);
          } else {
            slot = base + t;
            if (slot >= cap) slot -= cap;
          }
          drow = row0 + slot;
        }
        if (INT8) {   // the half's 4 bytes
          wr[u] = reinterpret_cast<const uint32_t*>(a.codes)[2 * ((drow << lsh) + c) + (k & 1)];
          sr[u] = a.scales[drow];
        } else {
          wr[u] = reinterpret_cast<const uint32_t*>(a.codes)[(drow << lsh) + c] >> (16 * (k & 1));
          sr[u] = H16 ? (float)reinterpret_cast<const _Float16*>(a.scales)[(drow << gprsh) + (c >> gsh)]
                      : a.scales[(drow << gprsh) + (c >> gsh)];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UD; ++u) {
      const uint32_t k = k0 + u * stride;
      if (k >= nhalf) break;
      const float s = sr[u];
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (INT8 ? (float)(int8_t)((wr[u] >> (8 * j)) & 255u) : (float)nib_s(wr[u], j)) * s;
      __builtin_nontemporal_store((floatx4){v[0], v[1], v[2], v[3]}, reinterpret_cast<floatx4*>(outp) + k);
    }
  }
}

__global__ void __launch_bounds__(256) dequant_int4_kernel(DequantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) dequant_pair<false>(a, bh);
}
__global__ void __launch_bounds__(256) dequant_int8_kernel(DequantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) dequant_pair<true>(a, bh);
}
__global__ void __launch_bounds__(256) dequant_int4h_kernel(DequantArgs a) {
  for (int bh = blockIdx.z; bh < a.B * a.Hkv; bh += gridDim.z) dequant_pair<false, true>(a, bh);
}

// Chunk blocks per (b, h) pair: about `target` workgroups in all, at least one per
// pair, no more than a pair's chunks need.
inline int blocks_per_pair(uint64_t pairs, uint64_t chunks_per_pair, uint64_t target) {
  const uint64_t want = (target + pairs - 1) / pairs;
  const uint64_t need = (chunks_per_pair + 255) / 256;
  const uint64_t n = want < need ? want : need;
  return (int)(n ? n : 1);
}

}  // namespace

hipError_t launch_quant_intq(int32_t format, const QuantArgs& a, hipStream_t s) {
  const uint64_t pairs = (uint64_t)a.B * a.Hkv;
  // about 4096 workgroups (16 per CU)
  const dim3 grid(blocks_per_pair(2 * pairs, (uint64_t)a.map.n * (a.D / 8), 4096), 2,
                  (uint32_t)(pairs < 65535 ? pairs : 65535));
  return launch_kernel(format == KVQ_INT4_G     ? quant_int4_kernel
                       : format == KVQ_INT4_G16 ? quant_int4h_kernel
                                                : quant_int8_kernel,
                       grid, dim3(256), a, s);
}

hipError_t launch_dequant_intq(int32_t format, const DequantArgs& a, hipStream_t s) {
  const uint64_t pairs = (uint64_t)a.B * a.Hkv;
  // about 16384 workgroups (64 per CU) of one half-chunk per lane and iteration: on
  // the 8-layer Llama-3-8B 8K dequantization this measured faster than 2048 - 65536
  // workgroups with 2 - 16 half-chunks per iteration
  const dim3 grid(blocks_per_pair(pairs, (uint64_t)a.n * (a.D / 4), 16384), 1,
                  (uint32_t)(pairs < 65535 ? pairs : 65535));
  return launch_kernel(format == KVQ_INT4_G     ? dequant_int4_kernel
                       : format == KVQ_INT4_G16 ? dequant_int4h_kernel
                                                : dequant_int8_kernel,
                       grid, dim3(256), a, s);
}

}  // namespace kvq
