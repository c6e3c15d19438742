// The 64-bit argmax key shared by the argmax kernel and the GEMV launch that
// folds the argmax of its LM-head output in (device code, gfx950).
//
// High word: the value mapped to an unsigned order (NaN above everything,
// every NaN equal, -0.0 equal to +0.0, then the IEEE order); low word:
// 0xFFFFFFFF - index. So the larger key is the larger value and, between
// equal values, the lower index: the first index of the maximum, with the
// first NaN winning if there is one (NumPy's argmax). Every key of a real
// value has a high word >= 0x007FFFFF (that of -inf), so keys 0 and 1 never
// win against one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemv {

__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t i) {
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

__device__ __forceinline__ int32_t argmax_index(uint64_t key) {
  return static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFu));
}

}  // namespace qgemv
