// A plain streaming read of device memory: the ceiling that bench.py sets
// beside the HBM-bound kernels of liblbq (same byte counts, same launch
// pattern).  Not part of liblbq's interface; bench.py loads it with ctypes.
//
// Each lane reads 16-byte chunks with non-temporal buffer loads, UNROLL loads
// in flight, grid-stride; the words are folded with xor and the result is
// stored only if it equals a value no input here produces, so the loads
// cannot be removed and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ p, int64_t nchunks,
                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; c + (UNROLL - 1) * stride < nchunks; c += UNROLL * stride) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + c + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; c < nchunks; c += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + c);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) at `p` on `stream` with
// `grid` workgroups of 256 lanes and `unroll` (1, 2, 4 or 8) loads in flight
// per lane.  `sink` must hold `grid` uint32 (never written in practice).
// Returns the hipError_t of the launch.
extern "C" int bench_stream_read(const void* p, int64_t bytes, int grid, int unroll, void* sink, void* stream) {
  const int64_t nchunks = bytes / 16;
  const u32x4_t* src = static_cast<const u32x4_t*>(p);
  uint32_t* out = static_cast<uint32_t*>(sink);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((k_stream_read<1>), dim3(grid), dim3(256), 0, s, src, nchunks, out); break;
    case 2: hipLaunchKernelGGL((k_stream_read<2>), dim3(grid), dim3(256), 0, s, src, nchunks, out); break;
    case 4: hipLaunchKernelGGL((k_stream_read<4>), dim3(grid), dim3(256), 0, s, src, nchunks, out); break;
    default: hipLaunchKernelGGL((k_stream_read<8>), dim3(grid), dim3(256), 0, s, src, nchunks, out); break;
  }
  return (int)hipGetLastError();
}
