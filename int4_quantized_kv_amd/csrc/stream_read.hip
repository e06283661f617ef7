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

}  // namespace

extern "C" {

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
