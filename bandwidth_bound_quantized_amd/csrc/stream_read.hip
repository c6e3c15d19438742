// Streaming-read kernel: reads a device buffer once with 16-byte loads.
//
// Its best rate over large buffers is the measured HBM read peak that the
// GEMV's bandwidth is reported against, as the infer page does with a
// streaming-read kernel of its own rather than the spec sheet. Grid size
// and loads in flight per thread are parameters so a sweep can find the
// best configuration; loads are non-temporal, as in the GEMV.
#include "qgemv_internal.h"

namespace qgemv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int UNROLL>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                               size_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads / 64];
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) a ^= red[w];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, int unroll,
                              hipStream_t stream) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  switch (unroll) {
    case 1: stream_read_kernel<1><<<grid, kThreads, 0, stream>>>(p, n16, sink); break;
    case 2: stream_read_kernel<2><<<grid, kThreads, 0, stream>>>(p, n16, sink); break;
    case 4: stream_read_kernel<4><<<grid, kThreads, 0, stream>>>(p, n16, sink); break;
    case 8: stream_read_kernel<8><<<grid, kThreads, 0, stream>>>(p, n16, sink); break;
    default: stream_read_kernel<16><<<grid, kThreads, 0, stream>>>(p, n16, sink); break;
  }
  return hipGetLastError();
}

}  // namespace qgemv
