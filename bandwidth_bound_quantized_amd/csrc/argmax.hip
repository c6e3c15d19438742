// Greedy-token argmax over LM-head logits on CDNA4 (gfx950).
//
// The decode step ends by picking the largest logit ("infer", decode
// pipeline figure; its per-kernel table has the argmax over a 128256-word
// vocabulary as a separate bandwidth-bound kernel). One launch: each
// workgroup reduces one slice (about 1024 logits, one load per thread) of
// one batch row to a 64-bit key whose high word orders the value and whose
// low word is ~index (so the larger key is the larger value and, on equal
// values, the lower index), and folds it into the row's running maximum in
// the caller's workspace with a 64-bit atomic max. The last workgroup of a
// row to finish (found with an agent-scope counter next to the maximum)
// writes the index and returns both words to zero.
//
// Order of values: NaN above everything (every NaN equal, so the first NaN
// wins), then the IEEE order with -0.0 == +0.0.
#include "qgemv_internal.h"
#include "qgemv.h"

namespace qgemv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t make_key(float v, uint32_t i) {
  uint32_t u = __float_as_uint(v);
  uint32_t ord;
  if (v != v) {
    ord = 0xFFFFFFFFu;
  } else {
    if (v == 0.0f) u = 0u;                           // -0.0 ties +0.0
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - i);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t block_max(uint64_t k, uint64_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) k = umax64(k, __shfl_xor(k, o));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = k;
  __syncthreads();
  k = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) k = umax64(k, red[w]);
  return k;
}

__global__ __launch_bounds__(kThreads) void argmax_kernel(const float* __restrict__ logits,
                                                          int64_t V, int slices,
                                                          uint64_t* __restrict__ ws,
                                                          int32_t* __restrict__ idx) {
  __shared__ uint64_t red[kThreads / 64];
  const int b = blockIdx.y;
  const int s = blockIdx.x;
  const int64_t per = (V + slices - 1) / slices;
  const int64_t beg = static_cast<int64_t>(s) * per;
  const int64_t end = beg + per < V ? beg + per : V;
  const float* row = logits + static_cast<int64_t>(b) * V;

  // all of this thread's loads are issued before any is used (addresses
  // clamped into the slice; elements past its end do not count)
  uint64_t key = 0;
  constexpr int kU = 4;
  for (int64_t i0 = beg + threadIdx.x; i0 < end; i0 += kU * kThreads) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + u * kThreads;
      v[u] = __builtin_nontemporal_load(row + (i < end ? i : end - 1));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < end) key = umax64(key, make_key(v[u], static_cast<uint32_t>(i)));
    }
  }
  key = block_max(key, red);

  // ws row: word 0 = running max key, word 1 = count of finished workgroups
  uint64_t* slot = ws + static_cast<int64_t>(b) * QGEMV_ARGMAX_WS_WORDS_PER_ROW;
  uint32_t* counter = reinterpret_cast<uint32_t*>(slot + 1);
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_max(slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == static_cast<uint32_t>(slices - 1)) {
      // every other workgroup's max happened before its counter increment
      const uint64_t k = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      idx[b] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFu));
      __hip_atomic_store(slot, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_argmax(const float* logits, int64_t V, int batch, uint64_t* ws, int32_t* idx,
                         hipStream_t stream) {
  int64_t slices = (V + 1023) / 1024;                // one load per thread per slice
  if (slices < 1) slices = 1;
  if (slices > kArgmaxSlices) slices = kArgmaxSlices;
  dim3 grid(static_cast<unsigned>(slices), static_cast<unsigned>(batch));
  argmax_kernel<<<grid, kThreads, 0, stream>>>(logits, V, static_cast<int>(slices), ws, idx);
  return hipGetLastError();
}

}  // namespace qgemv
