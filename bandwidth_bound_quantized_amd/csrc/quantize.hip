// Weight quantizer on the device (gfx950): bf16 weights -> Q4_0-g32,
// int4-g128, int4-g64, int8-g32 or int8-row codes and binary16 scales,
// bit-identical to the host quantizer of qgemv_pack (SRC_BF16).
//
// Rule (the Rust page, "Is the 4-bit model still good?", and "infer", design
// notes: the group's element of largest magnitude, with its sign, maps to
// code 0, i.e. to -8 * d; int8 is symmetric with d = max|w| / 127), with the
// readings the host packer and the oracle share: the first element wins a
// tie in |w|; d is rounded to binary16 (nearest, ties to even) before the
// codes are computed; code = round-half-even(w / d) (+8 for 4-bit), clamped
// to [0, 15] or [-127, 127], with the division in float64; a scale that
// rounds to zero is stored as +0 with codes 8 (4-bit) or 0 (int8); a
// non-finite weight or a scale past binary16's range is an error.
//
// One thread per group (offline work; every thread reads its group's
// contiguous bf16 weights with 16-byte loads); int8-row: one wave per row. float64 arithmetic: every
// bf16 and binary16 value is exact in it, and the divisions are IEEE
// (correctly rounded) divisions.
#include "qgemv_internal.h"
#include "qgemv.h"

namespace qgemv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_double(uint16_t b) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(b) << 16));
}

__device__ __forceinline__ double half_bits_to_double(uint16_t h) {
  return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, h)));
}

// float64 -> binary16, one rounding (nearest, ties to even), overflow to inf:
// on the bit pattern, shifting the 53-bit significand down to binary16's
// quantum (2^-24 for subnormal results, 2^(e-10) otherwise). A conversion
// through float32 would round twice.
__device__ __forceinline__ uint16_t double_to_half_rne(double v) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000);
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag > 0x7FF0000000000000ull) return 0x7E00;
  if (mag == 0x7FF0000000000000ull) return sign | 0x7C00;
  const int biased = static_cast<int>(mag >> 52);
  if (biased == 0) return sign;
  int e = biased - 1023;
  const uint64_t m = (mag & ((uint64_t(1) << 52) - 1)) | (uint64_t(1) << 52);
  const int shift = (e < -14) ? 28 - e : 42;
  uint64_t n = 0;
  if (shift < 64) {
    n = m >> shift;
    const uint64_t rem = m & ((uint64_t(1) << shift) - 1);
    const uint64_t half = uint64_t(1) << (shift - 1);
    if (rem > half || (rem == half && (n & 1))) ++n;
  }
  if (e < -14) return sign | static_cast<uint16_t>(n);
  if (n == 2048) { n = 1024; ++e; }
  if (e > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (n - 1024));
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                       int32_t* __restrict__ err) {
  constexpr int G = FMT == QGEMV_INT4_G128 ? 128 : FMT == QGEMV_INT4_G64 ? 64 : 32;
  const int64_t ng = K / G;
  const int64_t grp = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (grp >= M * ng) return;
  const int64_t m = grp / ng, g = grp - m * ng;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + m * K + g * G);
  uint32_t v[G / 2];                                   // bf16 pairs
#pragma unroll
  for (int t = 0; t < G / 8; ++t) {
    const u32x4 u = src[t];
    v[4 * t] = u.x; v[4 * t + 1] = u.y; v[4 * t + 2] = u.z; v[4 * t + 3] = u.w;
  }
  auto elem = [&](int j) -> uint16_t {
    return static_cast<uint16_t>((j & 1) ? (v[j >> 1] >> 16) : (v[j >> 1] & 0xFFFFu));
  };
  bool bad = false;
  // largest |w| (first in index order), on the bit pattern: |bf16| orders as
  // its magnitude bits
  uint16_t best = 0, best_signed = 0;                  // |w| and w of the first maximum
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint16_t e = elem(j);
    const uint16_t a = e & 0x7FFF;
    bad |= a >= 0x7F80;                                // inf or NaN
    if (a > best) { best = a; best_signed = e; }
  }
  double d_exact;
  if constexpr (FMT == QGEMV_INT8_G32) d_exact = bf16_to_double(best) / 127.0;
  else d_exact = bf16_to_double(best_signed) / -8.0;
  uint16_t dh = double_to_half_rne(d_exact);
  if ((dh & 0x7FFF) == 0) dh = 0;                      // a zero scale is +0
  bad |= (dh & 0x7C00) == 0x7C00;                      // past binary16's range
  const double d = half_bits_to_double(dh);
  scales[grp] = dh;
  // codes: the group's weights are read again (from cache) word by word
  // rather than indexed out of registers
  const uint32_t* wr = reinterpret_cast<const uint32_t*>(w + m * K + g * G);
  auto code = [&](uint32_t pair, int hi) -> double {
    const uint16_t b = static_cast<uint16_t>(hi ? (pair >> 16) : (pair & 0xFFFFu));
    return d == 0.0 ? 0.0 : __builtin_rint(bf16_to_double(b) / d);
  };
  if constexpr (FMT == QGEMV_INT8_G32) {
    uint32_t* out = reinterpret_cast<uint32_t*>(codes + m * K + g * G);
#pragma unroll 2
    for (int t = 0; t < G / 4; ++t) {
      const uint32_t p0 = wr[2 * t], p1 = wr[2 * t + 1];
      const double qd[4] = {code(p0, 0), code(p0, 1), code(p1, 0), code(p1, 1)};
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double q = qd[u] < -127.0 ? -127.0 : (qd[u] > 127.0 ? 127.0 : qd[u]);
        word |= (static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu) << (8 * u);
      }
      out[t] = word;
    }
  } else {
    uint32_t* out = reinterpret_cast<uint32_t*>(codes + grp * (G / 2));
#pragma unroll 2
    for (int t = 0; t < G / 8; ++t) {                  // output bytes 4t..4t+3
      // byte j: element j (low nibble) and element j + G/2 (high nibble)
      const uint32_t lo0 = wr[2 * t], lo1 = wr[2 * t + 1];
      const uint32_t hi0 = wr[G / 4 + 2 * t], hi1 = wr[G / 4 + 2 * t + 1];
      const double ql[4] = {code(lo0, 0), code(lo0, 1), code(lo1, 0), code(lo1, 1)};
      const double qh[4] = {code(hi0, 0), code(hi0, 1), code(hi1, 0), code(hi1, 1)};
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        double a = (d == 0.0) ? 8.0 : ql[u] + 8.0;
        double b = (d == 0.0) ? 8.0 : qh[u] + 8.0;
        a = a < 0.0 ? 0.0 : (a > 15.0 ? 15.0 : a);
        b = b < 0.0 ? 0.0 : (b > 15.0 ? 15.0 : b);
        word |= static_cast<uint32_t>(static_cast<int>(a) | (static_cast<int>(b) << 4)) << (8 * u);
      }
      out[t] = word;
    }
  }
  if (bad && err) atomicExch(err, QGEMV_ERANGE);
}

// int8 with one scale per row: one wave per row (4 per workgroup). The
// row's largest |w| (on the magnitude bits, an exact max in any order), the
// scale, then the codes, 8 weights per lane and step.
__global__ __launch_bounds__(256) void quantize_int8_row_kernel(const uint16_t* __restrict__ w, int64_t M,
                                                                int64_t K, int8_t* __restrict__ codes,
                                                                uint16_t* __restrict__ scales,
                                                                int32_t* __restrict__ err) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;                                // the whole wave
  const uint16_t* wr = w + row * K;
  uint32_t best = 0;
  bool bad = false;
  for (int64_t k = 8 * lane; k < K; k += 512) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(wr + k);
    const uint32_t d4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a0 = d4[i] & 0x7FFFu, a1 = (d4[i] >> 16) & 0x7FFFu;
      bad |= a0 >= 0x7F80u || a1 >= 0x7F80u;
      best = a0 > best ? a0 : best;
      best = a1 > best ? a1 : best;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t t = static_cast<uint32_t>(__shfl_xor(static_cast<int>(best), o));
    best = t > best ? t : best;
  }
  bad = __any(bad);
  uint16_t dh = double_to_half_rne(bf16_to_double(static_cast<uint16_t>(best)) / 127.0);
  if ((dh & 0x7FFF) == 0) dh = 0;                      // a zero scale is +0
  bad |= (dh & 0x7C00) == 0x7C00;
  const double d = half_bits_to_double(dh);
  if (lane == 0) scales[row] = dh;
  for (int64_t k = 8 * lane; k < K; k += 512) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(wr + k);
    const uint32_t d4[4] = {u.x, u.y, u.z, u.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t b = static_cast<uint16_t>((i & 1) ? (d4[i >> 1] >> 16) : (d4[i >> 1] & 0xFFFFu));
      double q = d == 0.0 ? 0.0 : __builtin_rint(bf16_to_double(b) / d);
      q = q < -127.0 ? -127.0 : (q > 127.0 ? 127.0 : q);
      out[i >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(codes + row * K + k) = make_uint2(out[0], out[1]);
  }
  if (bad && err && lane == 0) atomicExch(err, QGEMV_ERANGE);
}

}  // namespace

hipError_t launch_quantize(int fmt, const uint16_t* w, int64_t M, int64_t K, void* codes, uint16_t* scales,
                           int32_t* err, hipStream_t stream) {
  uint8_t* c = static_cast<uint8_t*>(codes);
  if (fmt == QGEMV_INT8_ROW) {
    const unsigned grid = static_cast<unsigned>((M + 3) / 4);
    quantize_int8_row_kernel<<<grid, 256, 0, stream>>>(w, M, K, reinterpret_cast<int8_t*>(c), scales, err);
    return hipGetLastError();
  }
  const int G = fmt == QGEMV_INT4_G128 ? 128 : fmt == QGEMV_INT4_G64 ? 64 : 32;
  const int64_t groups = M * (K / G);
  const unsigned grid = static_cast<unsigned>((groups + 255) / 256);
  switch (fmt) {
    case QGEMV_INT8_G32: quantize_kernel<QGEMV_INT8_G32><<<grid, 256, 0, stream>>>(w, M, K, c, scales, err); break;
    case QGEMV_Q4_0_G32: quantize_kernel<QGEMV_Q4_0_G32><<<grid, 256, 0, stream>>>(w, M, K, c, scales, err); break;
    case QGEMV_INT4_G128: quantize_kernel<QGEMV_INT4_G128><<<grid, 256, 0, stream>>>(w, M, K, c, scales, err); break;
    case QGEMV_INT4_G64: quantize_kernel<QGEMV_INT4_G64><<<grid, 256, 0, stream>>>(w, M, K, c, scales, err); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qgemv
