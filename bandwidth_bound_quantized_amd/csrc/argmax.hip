// Greedy-token argmax over LM-head logits on CDNA4 (gfx950).
//
// The decode step ends by picking the largest logit ("infer", decode
// pipeline figure; its per-kernel table has the argmax over a 128256-word
// vocabulary as a separate bandwidth-bound kernel). One launch of
// 256-thread workgroups: each reduces a slice (1-16 Ki logits) of one batch
// row to a 64-bit key whose high word orders the value and whose low word is
// ~index (so the larger key is the larger value and, on equal values, the
// lower index). A row that fits one slice is one workgroup, which writes the
// index itself; otherwise the slices of a row meet through a 64-bit atomic
// max and a counter in the caller's workspace (the last slice writes the
// index and zeroes both words).
//
// Order of values (argmax_key.h): NaN above everything (every NaN equal, so
// the first NaN wins), then the IEEE order with -0.0 == +0.0.
#include <mutex>

#include "argmax_key.h"
#include "qgemv_internal.h"
#include "qgemv.h"

namespace qgemv {
namespace {

#ifndef QGEMV_ARGMAX_THREADS
#define QGEMV_ARGMAX_THREADS 256
#endif
#ifndef QGEMV_ARGMAX_TARGET_WGS
#define QGEMV_ARGMAX_TARGET_WGS 32    // workgroups per launch (all rows together)
#endif
#ifndef QGEMV_ARGMAX_MAX_SLICE
#define QGEMV_ARGMAX_MAX_SLICE 16384
#endif
constexpr int kThreads = QGEMV_ARGMAX_THREADS;
constexpr int64_t kMinSlice = 1024;   // logits per workgroup, bounds of the adaptive slice
constexpr int64_t kMaxSlice = QGEMV_ARGMAX_MAX_SLICE;

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

// grid = (slices, batch). slices == 1: the workgroup writes idx directly. Otherwise
// each slice folds its key into ws[row][0] with a 64-bit atomic max and counts itself
// in ws[row][1]; the last slice of the row writes idx and zeroes both words.
// Device-scope atomics on one address serialize (tens of ns each on MI355X), so the
// number of slices per row is kept small.
template <bool VEC4>
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

  uint64_t key = 0;
  if constexpr (VEC4) {
    // rows start 16-byte aligned and per is a multiple of 4: float4 loads,
    // all of a thread's loads issued before any is used
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kU = 8;
    const int64_t n4 = (end - beg) / 4;
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row + beg);
    for (int64_t j0 = threadIdx.x; j0 < n4; j0 += kU * kThreads) {
      f32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t j = j0 + u * kThreads;
        v[u] = __builtin_nontemporal_load(r4 + (j < n4 ? j : n4 - 1));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t j = j0 + u * kThreads;
        if (j < n4) {
          const uint32_t i = static_cast<uint32_t>(beg + 4 * j);
          key = umax64(key, argmax_key(v[u].x, i));
          key = umax64(key, argmax_key(v[u].y, i + 1));
          key = umax64(key, argmax_key(v[u].z, i + 2));
          key = umax64(key, argmax_key(v[u].w, i + 3));
        }
      }
    }
  } else {
    constexpr int kU = 8;
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
        if (i < end) key = umax64(key, argmax_key(v[u], static_cast<uint32_t>(i)));
      }
    }
  }
  key = block_max(key, red);
  if (threadIdx.x != 0) return;
  if (slices == 1) {
    idx[b] = argmax_index(key);
    return;
  }
  uint64_t* slot = ws + static_cast<int64_t>(b) * QGEMV_ARGMAX_WS_WORDS_PER_ROW;
  uint32_t* counter = reinterpret_cast<uint32_t*>(slot + 1);
  __hip_atomic_fetch_max(slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (prev == static_cast<uint32_t>(slices - 1)) {
    // every other slice's max happened before its counter increment
    const uint64_t k = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    idx[b] = argmax_index(k);
    __hip_atomic_store(slot, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_argmax(const float* logits, int64_t V, int batch, uint64_t* ws, int32_t* idx,
                         hipStream_t stream) {
  // Slices of 1-16 Ki logits, aiming at ~32 workgroups per launch: fewer
  // leave the load latency of each workgroup exposed, more make the
  // same-address atomics that join the slices of a row queue up (measured on
  // MI355X: V=32000 B=1 best with 32 slices, V=128256 B=8 with 8 per row).
  int64_t slice = (V * batch + QGEMV_ARGMAX_TARGET_WGS - 1) / QGEMV_ARGMAX_TARGET_WGS;
  slice = (slice + kMinSlice - 1) / kMinSlice * kMinSlice;
  if (slice < kMinSlice) slice = kMinSlice;
  if (slice > kMaxSlice) slice = kMaxSlice;
  int64_t slices = (V + slice - 1) / slice;
  if (slices > kArgmaxSlices) slices = kArgmaxSlices;
  const int64_t per = (V + slices - 1) / slices;
  const bool vec4 = (V % 4 == 0) && (per % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  dim3 grid(static_cast<unsigned>(slices), static_cast<unsigned>(batch));
  if (vec4)
    argmax_kernel<true><<<grid, kThreads, 0, stream>>>(logits, V, static_cast<int>(slices), ws, idx);
  else
    argmax_kernel<false><<<grid, kThreads, 0, stream>>>(logits, V, static_cast<int>(slices), ws, idx);
  return hipGetLastError();
}

// ------------------------------------------------- argmax without allocation
// The workspace of launch_argmax_noalloc: one copy per GPU for the life of the
// process (a code-object global). In host code `scratch` names a host-side
// stand-in, not device memory: the kernels get the device address that
// hipGetSymbolAddress returns for the current device, kept per device below.
constexpr int kScratchWords = QGEMV_ARGMAX_NOALLOC_MAX_BATCH * QGEMV_ARGMAX_WS_WORDS_PER_ROW;
static __device__ __align__(256) uint64_t scratch[kScratchWords];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(uint64_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// The current device's copy of `scratch`. The first call on a device looks up
// its address and clears it with a kernel on `stream` (ahead of the caller's
// argmax in stream order; a kernel rather than a memset so that a first call
// made under graph capture records an ordinary kernel node).
hipError_t device_scratch(hipStream_t stream, uint64_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    uint64_t* ptr = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    zero_words_kernel<<<1, 64, 0, stream>>>(ptr, kScratchWords);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_argmax_noalloc(const float* logits, int64_t V, int batch, int32_t* idx,
                                 hipStream_t stream) {
  if (batch < 1 || batch > QGEMV_ARGMAX_NOALLOC_MAX_BATCH) return hipErrorInvalidValue;
  uint64_t* ws = nullptr;
  const hipError_t e = device_scratch(stream, &ws);
  if (e != hipSuccess) return e;
  // the kernel leaves every word it uses zero again (the last slice of a row
  // resets the row's two words), so the scratch is zero at every call's start
  return launch_argmax(logits, V, batch, ws, idx, stream);
}

}  // namespace qgemv
