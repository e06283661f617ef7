// codec.hip -- Walsh-Hadamard rotation + 4-bit or 3-bit Lloyd-Max KV codec: encode
// (prefill and append), dequantize, and the library's own codebooks.
//
// Page: "长上下文内存大瘦身：LARQL 四大 KV 缓存引擎原理与横向对比" (pwwt.cn/news/5725003),
// engine three (codec): every K/V row is coded per head by a Walsh-Hadamard rotation
// followed by Lloyd-Max quantization at 3 or 4 bits; head_dim must be a power of two.
// The page gives no further detail; this library takes the plainest algorithm that
// fits it: y = H x / sqrt(D) (Sylvester order, orthonormal, no sign flips),
// s = ||x||_2 / sqrt(D), index = number of Lloyd-Max decision thresholds of N(0,1)
// strictly below y / s (a zero row is coded as y / 1), decode x = s * H c[index] / sqrt(D).
//
// Mapping: as for INT4, a row of D elements spans D/8 lanes of 8 elements; three
// butterfly stages run inside a lane, log2(D/8) across lanes with xor shuffles.  4-bit
// rows are D/2 bytes of nibbles; 3-bit rows the indices packed back to back in 3D/8
// bytes (see store_packed3).  The 3-bit coder is the 4-bit one with thresholds 7 .. 14
// set to +inf.
#include <cmath>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D, int BITS>
__global__ void __launch_bounds__(256) codec_encode_kernel(QuantArgs a) {
  constexpr int LPR = D / 8;
  const int isv = blockIdx.y;
  const uint16_t* src = isv ? a.v : a.k;
  void* codes = isv ? a.v_codes : a.k_codes;
  float* scales = isv ? a.v_scales : a.k_scales;
  const uint32_t total = (uint32_t)a.rows * LPR;
  const uint32_t stride = gridDim.x * blockDim.x;
  const Thresholds thr = load_thresholds(a.thr);
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / LPR;
    const int c = (int)(i - row * LPR);
    float x[8];
    load8_f16(src + (size_t)i * 8, x);
    uint32_t w;
    float s;
    codec_encode_row<LPR>(x, c, thr, w, s);
    const uint32_t bh = row / (uint32_t)a.map.n;
    const int t = (int)(row - bh * a.map.n);
    const int b = (int)(bh / (uint32_t)a.Hkv);
    const int p = a.map.append ? a.map.pos[b] : a.map.start + t;
    const size_t drow = a.pages.size ? paged_row(a.pages, a.Hkv, b, (int)(bh - b * a.Hkv), p)
                                     : (size_t)bh * a.map.cap + cache_slot(p, a.map.cap, a.map.sinks);
    if (BITS == 4) static_cast<uint32_t*>(codes)[drow * LPR + c] = w;
    else store_packed3<LPR>(static_cast<uint8_t*>(codes) + drow * 3 * LPR, c, w);
    if (c == 0) scales[drow] = s;
  }
}

template <int D, int BITS>
__global__ void __launch_bounds__(256) codec_dequant_kernel(DequantArgs a) {
  constexpr int LPR = D / 8;
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = a.levels[threadIdx.x];
  __syncthreads();
  const uint32_t total = (uint32_t)a.B * a.Hkv * a.n * LPR;
  const uint32_t stride = gridDim.x * blockDim.x;
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  // a row's LPR lanes are aligned and consecutive, so they enter and leave the loop
  // together and the butterfly shuffles never read a lane outside the row
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / LPR;
    const int c = (int)(i - row * LPR);
    const uint32_t bh = row / (uint32_t)a.n;
    const int t = (int)(row - bh * a.n);
    const int b = (int)(bh / (uint32_t)a.Hkv);
    const size_t drow = a.pages.size ? paged_row(a.pages, a.Hkv, b, (int)(bh - b * a.Hkv), a.start + t)
                                     : (size_t)bh * a.cap + cache_slot(a.start + t, a.cap, a.sinks);
    const uint32_t w = BITS == 4 ? static_cast<const uint32_t*>(a.codes)[drow * LPR + c]
                                 : load_packed3<LPR>(static_cast<const uint8_t*>(a.codes) + drow * 3 * LPR, c);
    const float s = a.scales[drow];
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = lv[nib_u(w, j)];
    wht_row<LPR>(v, c);
    const float f = s * inv_sqrt_d;
    float4* out = reinterpret_cast<float4*>(a.out + (size_t)i * 8);
    out[0] = make_float4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
    out[1] = make_float4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
  }
}

inline int grid_for(uint64_t lanes) {
  uint64_t blocks = (lanes + 255) / 256;
  const uint64_t cap = 256ull * 16;
  return (int)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

struct Book {
  float levels[16];        // 2^bits used
  float thresholds[15];    // 2^bits - 1 used
};

double phi(double t) { return std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI); }
double Phi(double t) { return 0.5 * std::erfc(-t / std::sqrt(2.0)); }

// Lloyd's two optimality conditions for N(0,1), iterated to a fixed point in double:
// thresholds are midpoints of adjacent levels; each level is the mean of its cell,
// (phi(lo) - phi(hi)) / (Phi(hi) - Phi(lo)).
Book compute_book(int n) {   // n = 2^bits levels
  double c[16];
  for (int i = 0; i < n; ++i) c[i] = -2.5 + 5.0 * i / (n - 1);
  for (int it = 0; it < 200000; ++it) {
    double t[15];
    for (int j = 0; j < n - 1; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
    double delta = 0.0;
    for (int j = 0; j < n; ++j) {
      const double plo = j == 0 ? 0.0 : phi(t[j - 1]);
      const double phi_hi = j == n - 1 ? 0.0 : phi(t[j]);
      const double Plo = j == 0 ? 0.0 : Phi(t[j - 1]);
      const double Phi_hi = j == n - 1 ? 1.0 : Phi(t[j]);
      const double cn = (plo - phi_hi) / (Phi_hi - Plo);
      delta = std::fmax(delta, std::fabs(cn - c[j]));
      c[j] = cn;
    }
    if (delta < 1e-14) break;
  }
  // N(0,1) is symmetric, so is its optimal quantizer: make the levels exactly odd so
  // that the middle threshold is exactly 0
  double cs[16];
  for (int j = 0; j < n; ++j) cs[j] = 0.5 * (c[j] - c[n - 1 - j]);
  Book b;
  for (int j = 0; j < 16; ++j) b.levels[j] = j < n ? (float)cs[j] : 0.0f;
  for (int j = 0; j < 15; ++j)
    b.thresholds[j] = j < n - 1 ? (float)(0.5 * (cs[j] + cs[j + 1])) : __builtin_huge_valf();
  return b;
}

}  // namespace

void codec_codebook(int32_t bits, float levels[16], float thresholds[15]) {
  static const Book book4 = compute_book(16), book3 = compute_book(8);   // computed once
  const Book& book = bits == 3 ? book3 : book4;
  for (int j = 0; j < 16; ++j) levels[j] = book.levels[j];
  for (int j = 0; j < 15; ++j) thresholds[j] = book.thresholds[j];
}

template <int BITS>
hipError_t encode_bits(const QuantArgs& a, dim3 grid, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_kernel(codec_encode_kernel<64, BITS>, grid, dim3(256), a, s);
    case 128: return launch_kernel(codec_encode_kernel<128, BITS>, grid, dim3(256), a, s);
    case 256: return launch_kernel(codec_encode_kernel<256, BITS>, grid, dim3(256), a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t dequant_bits(const DequantArgs& a, dim3 grid, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_kernel(codec_dequant_kernel<64, BITS>, grid, dim3(256), a, s);
    case 128: return launch_kernel(codec_dequant_kernel<128, BITS>, grid, dim3(256), a, s);
    case 256: return launch_kernel(codec_dequant_kernel<256, BITS>, grid, dim3(256), a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_codec_encode(int32_t bits, const QuantArgs& a, hipStream_t s) {
  const uint64_t lanes = (uint64_t)a.rows * (a.D / 8);
  const dim3 grid(grid_for(lanes), 2);
  return bits == 3 ? encode_bits<3>(a, grid, s) : encode_bits<4>(a, grid, s);
}

hipError_t launch_codec_dequant(int32_t bits, const DequantArgs& a, hipStream_t s) {
  const uint64_t lanes = (uint64_t)a.B * a.Hkv * a.n * (a.D / 8);
  const dim3 grid(grid_for(lanes));
  return bits == 3 ? dequant_bits<3>(a, grid, s) : dequant_bits<4>(a, grid, s);
}

}  // namespace kvq
