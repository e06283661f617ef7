// stream_read.hip -- attainable HBM read rate of the machine, for the roofline figures of
// the benchmark.  Not part of the KV-cache library: it is built into its own shared
// object (libkvq_bench.so) and exported under a separate prefix.
//
// The kernel reads a buffer once, as fast as plain loads allow: every lane issues U
// independent 16-byte loads (global_load_dwordx4) per iteration before it uses any of
// them, iterations stride over the whole grid, and the loaded words are folded with
// xor into one word per lane so that nothing is written but one word per workgroup.
// The decode kernels' own streams are read-only in the same way, so this rate (not the
// copy rate, which also writes) is the ceiling their loops are held against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  // whole iterations: U loads per lane in flight
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {   // the tail
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup (lane 0's fold; the others' loads still had to complete)
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < (int)blockDim.x; ++t) r ^= s[t];
    sink[blockIdx.x] = r;
  }
}

template <int U, bool NT>
hipError_t launch(const void* buf, size_t bytes, int grid, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL((stream_read_kernel<U, NT>), dim3(grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// The decode step's own access pattern with no arithmetic: the attainable rate of exactly
// the transfers the matrix-core INT4 decode issues.  Each (b, kv head) unit's rows are
// cut into nsplit ranges of 32-row tiles; a workgroup of 8 waves takes one range, wave w
// tiles w, w + 8, ..., each tile four 1 KB pieces of K and V codes plus the tile's K and
// V scales moved global -> LDS, one tile in flight behind the one being waited for (the
// decode kernel's 2-slot ring).  The tiles are never read: only the transfers are timed.
constexpr int PT_WAVES = 8, PT_SLOT = 4608, PT_TILE = 32;
typedef __attribute__((address_space(3))) void* pt_lds_ptr;
typedef __attribute__((address_space(1))) void* pt_gbl_ptr;

template <int N>
__device__ __forceinline__ void pt_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int SIZE>
__device__ __forceinline__ void pt_dma(const uint8_t* g, uint8_t* l) {
  // non-temporal, as the decode kernel's transfers
  if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds((pt_gbl_ptr)g, (pt_lds_ptr)l, 16, 0, 2);
  else __builtin_amdgcn_global_load_lds((pt_gbl_ptr)g, (pt_lds_ptr)l, 4, 0, 2);
}

// k_codes / v_codes: [units][cap][64] bytes; k_scales: [units][cap][ksb]; v_scales:
// [units][cap][4]; tiles per split `nt`, rows per split nt * 32 from row 0.
__global__ void __launch_bounds__(PT_WAVES * 64) tile_pattern_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const uint8_t* __restrict__ vs, int cap, int ksb, int nt) {
  constexpr int DMA = 6;   // transfers per tile
  __shared__ __attribute__((aligned(16))) uint8_t ring[PT_WAVES * 2 * PT_SLOT];
  const int sp = blockIdx.x, unit = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* wr = ring + wave * 2 * PT_SLOT;
  const size_t row0 = (size_t)unit * cap + (size_t)sp * nt * PT_TILE;
  auto issue = [&](int t, int slot) {
    const size_t r = row0 + (size_t)t * PT_TILE;
    uint8_t* lb = wr + slot * PT_SLOT;
    pt_dma<16>(kc + r * 64 + 16 * lane, lb);
    pt_dma<16>(kc + r * 64 + 1024 + 16 * lane, lb + 1024);
    pt_dma<16>(vc + r * 64 + 16 * lane, lb + 2048);
    pt_dma<16>(vc + r * 64 + 1024 + 16 * lane, lb + 3072);
    pt_dma<4>(ks + r * ksb + (4 * lane) % (PT_TILE * ksb), lb + 4096);   // the tile's K scales
    pt_dma<4>(vs + r * 4 + 4 * (lane & 31), lb + 4352);                  // and its V scales
  };
  int t0 = wave;
  if (t0 < nt) issue(t0, 0);
  for (int k = 0; t0 < nt; ++k) {
    const int t1 = t0 + PT_WAVES;
    if (t1 < nt) {
      issue(t1, (k + 1) & 1);
      pt_wait<DMA>();   // tile t0 in LDS; t1 in flight
    } else {
      pt_wait<0>();
    }
    t0 = t1;
  }
  pt_wait<0>();
}

}  // namespace

extern "C" {

// The decode access pattern over one layer's INT4 cache: `units` (b, kv head) units of
// `cap` rows, K codes / V codes 64 bytes per row (head_dim 128), K scales `kscale_bytes`
// (4 to 64, a multiple of 4) and V scales 4 bytes per row, each unit's first
// nsplit * tiles_per_split * 32 rows (<= cap) read as nsplit workgroups of 8 waves.
// Returns 0, -1 for invalid arguments, -5 for a launch error.  Asynchronous on `stream`.
int32_t kvqb_tile_pattern(const void* k_codes, const void* k_scales, const void* v_codes,
                          const void* v_scales, int32_t units, int32_t cap, int32_t kscale_bytes,
                          int32_t nsplit, int32_t tiles_per_split, void* stream) {
  if (!k_codes || !k_scales || !v_codes || !v_scales || units < 1 || nsplit < 1 ||
      tiles_per_split < 1 || kscale_bytes < 4 || kscale_bytes > 64 || kscale_bytes % 4 ||
      (int64_t)nsplit * tiles_per_split * PT_TILE > cap || units > 65535)
    return -1;
  hipLaunchKernelGGL(tile_pattern_kernel, dim3(nsplit, units), dim3(PT_WAVES * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(k_codes),
                     static_cast<const uint8_t*>(k_scales), static_cast<const uint8_t*>(v_codes),
                     static_cast<const uint8_t*>(v_scales), cap, kscale_bytes, tiles_per_split);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Read `bytes` (a multiple of 16; buffer 16-byte aligned) of device memory at `buf`
// once with `grid` workgroups of 256 lanes, `unroll` (1, 2, 4, 8 or 16) 16-byte loads
// in flight per lane, plain or non-temporal (`nontemporal` != 0) loads; `sink` is a
// device buffer of at least `grid` words that receives one fold per workgroup.
// Returns 0, -1 for invalid arguments, -5 for a launch error.  Asynchronous on `stream`.
int32_t kvqb_stream_read(const void* buf, size_t bytes, int32_t grid, int32_t unroll,
                         int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!buf || !sink || grid < 1 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool nt = nontemporal != 0;
  switch (unroll) {
    case 1: e = nt ? launch<1, true>(buf, bytes, grid, sink, s) : launch<1, false>(buf, bytes, grid, sink, s); break;
    case 2: e = nt ? launch<2, true>(buf, bytes, grid, sink, s) : launch<2, false>(buf, bytes, grid, sink, s); break;
    case 4: e = nt ? launch<4, true>(buf, bytes, grid, sink, s) : launch<4, false>(buf, bytes, grid, sink, s); break;
    case 8: e = nt ? launch<8, true>(buf, bytes, grid, sink, s) : launch<8, false>(buf, bytes, grid, sink, s); break;
    case 16: e = nt ? launch<16, true>(buf, bytes, grid, sink, s) : launch<16, false>(buf, bytes, grid, sink, s); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -5;
}

}  // extern "C"
