// Fused-dequantization decode GEMV for CDNA4 (gfx950): y[b][m] = sum_k w(m,k) x[b][k].
//
// The decode step reads every weight once and does one multiply-add per
// weight and batch row, so this kernel is bound by HBM bandwidth ("infer",
// the roofline discussion; "Writing an LLM inference engine from scratch in
// Rust", Lesson 1). Everything here serves one goal: stream each weight byte
// from HBM exactly once, with wide coalesced loads and enough bytes in
// flight, while keeping the per-byte instruction count well under what the
// vector ALUs can issue at that rate.
//
// Work decomposition
//   * A row of the weight matrix is a sequence of 16-byte "units" (8 bf16
//     weights, 16 int8 weights, or 32 4-bit weights). Lane l of a wavefront
//     loads units l, l+64, l+128, ... of each row it works on, so every
//     16-byte load instruction of a wave covers 1 KiB of contiguous bytes.
//   * A wave works on R rows at a time (a "row group") and walks all of K;
//     waves take row groups in a grid-stride loop, with the next step's
//     weight loads issued before the current step is computed (register
//     double buffering), so a wave always has loads in flight.
//   * x (all batch rows) is staged once per workgroup in LDS as bf16; the
//     same LDS read feeds the R rows of a group.
//   * Dequantization happens in registers and is never written back
//     ("infer", design notes; Rust page, Lesson 2): codes are turned into
//     packed bf16 pairs and multiplied with packed bf16 activations by
//     v_dot2_f32_bf16 (two exact products and a float32 add per instruction).
//     Each group's scale multiplies the group's partial sum once.
//   * 4-bit codes: each nibble is masked into its own byte and converted to
//     bf16 exactly by the fp8 -> bf16 conversion instruction (a byte q in
//     0..15 is the e4m3 number q * 2^-9; the conversion's scale 2^9 undoes
//     that), two codes per instruction. The stored offset 8 is removed with
//     the per-unit sum of x folded into the dot chain's start value:
//     sum(q x) - 8 sum(x) = sum((q - 8) x) (the Rust page's bias-removal
//     identity, Lesson 6).
//   * int8 codes: sign-extended to float32 (exact) and packed to bf16 pairs
//     by taking the high halves (exact: at most 8 significant bits).
//   * The per-row reduction over the 64 lanes reduces all R*batch partial
//     sums together by repeatedly exchanging half of them with the partner
//     lane (each step halves the number of live values per lane).
// No MFMA: at batch <= 8 this is a matrix-vector product, not a dense
// contraction.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "argmax_key.h"
#include "qgemv_internal.h"
#include "qgemv.h"

// Launch-shape defaults (build-time overrides; the values were chosen by
// sweeping each one on MI355X with graph-timed, rotated launches).
#ifndef QGEMV_XREG_MAX_R
#define QGEMV_XREG_MAX_R 4        // rows per wave step, register-x kernel
#endif
#ifndef QGEMV_MIN_WAVES_PER_CU
#define QGEMV_MIN_WAVES_PER_CU 8  // shrink R until this many waves per CU have work
#endif
#ifndef QGEMV_MAX_WG_PER_CU
#define QGEMV_MAX_WG_PER_CU 8     // cap on resident workgroups per CU (persistent grid)
#endif
#ifndef QGEMV_GROUP_MAX_WG_PER_CU
#define QGEMV_GROUP_MAX_WG_PER_CU QGEMV_MAX_WG_PER_CU   // grouped launch: workgroups per CU cap
#endif
#ifndef QGEMV_GROUP_R2
#define QGEMV_GROUP_R2 2          // grouped launch: rows per wave step at 2 units per lane-column
#endif
#ifndef QGEMV_GROUP_RLONG
#define QGEMV_GROUP_RLONG 2       // ... and at 3 or 4 units per lane-column
#endif
#ifndef QGEMV_NT_LOADS
#define QGEMV_NT_LOADS 1          // stream weights with non-temporal loads
#endif
#ifndef QGEMV_GROUP_CONTIG_MIN
#define QGEMV_GROUP_CONTIG_MIN 8  // grouped launch: row groups per wave from which waves take contiguous ranges
#endif

namespace qgemv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// f(std::integral_constant<int, FMT>{}) for the runtime format (validated by
// the caller)
template <typename F>
auto with_fmt(int fmt, F&& f) {
  switch (fmt) {
    case QGEMV_BF16: return f(std::integral_constant<int, QGEMV_BF16>{});
    case QGEMV_INT8_G32: return f(std::integral_constant<int, QGEMV_INT8_G32>{});
    case QGEMV_Q4_0_G32: return f(std::integral_constant<int, QGEMV_Q4_0_G32>{});
    case QGEMV_INT4_G128: return f(std::integral_constant<int, QGEMV_INT4_G128>{});
    case QGEMV_INT8_ROW: return f(std::integral_constant<int, QGEMV_INT8_ROW>{});
    default: return f(std::integral_constant<int, QGEMV_INT4_G64>{});
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// One 16-byte weight load; weights are read exactly once, so by default they
// are fetched with the non-temporal hint and do not displace x in the caches.
__device__ __forceinline__ u32x4 load_weights(const u32x4* p) {
#if QGEMV_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// float32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}
// the two bf16 values of a packed pair, as float32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// SwiGLU's gate activation t * sigmoid(t) (for t -> -inf, t / inf = -0)
__device__ __forceinline__ float silu(float t) { return t / (1.f + expf(-t)); }

// Epilogue of one output y[b][m] = v (see Fusion): a plain store, a residual
// add, or, on the even row of each gate/up pair, the SwiGLU activation of
// the pair (partner = the odd row's value). Returns the value stored in y.
__device__ __forceinline__ float epi_store(const Fusion& f, float* __restrict__ Y, int M, int b, int m,
                                           float v, float partner) {
  const size_t o = static_cast<size_t>(b) * M + m;
  if (f.epi == kEpiSwiglu) {
    if ((m & 1) == 0) f.act[static_cast<size_t>(b) * (M >> 1) + (m >> 1)] = to_bf16(silu(v) * partner);
    return v;
  }
  if (f.epi == kEpiResidual) v = f.res[o] + v;
  Y[o] = v;
  return v;
}

template <int FMT> struct Traits;
template <> struct Traits<QGEMV_BF16> {
  static constexpr int kElems = 8;      // weights per 16-byte unit
  static constexpr int kPairs = 4;      // bf16 pairs per unit (= x dwords per unit)
  static constexpr int kUnitsPerScale = 0;  // no scales (-1: one per row; else units per group)
  static constexpr int kUC = 4;         // units per lane per step
  static constexpr bool kBias = false;
};
template <> struct Traits<QGEMV_INT8_G32> {
  static constexpr int kElems = 16;
  static constexpr int kPairs = 8;
  static constexpr int kUnitsPerScale = 2;
  static constexpr int kUC = 2;
  static constexpr bool kBias = false;
};
template <> struct Traits<QGEMV_Q4_0_G32> {
  static constexpr int kElems = 32;
  static constexpr int kPairs = 16;
  static constexpr int kUnitsPerScale = 1;
  static constexpr int kUC = 1;
  static constexpr bool kBias = true;
};
template <> struct Traits<QGEMV_INT4_G128> {
  static constexpr int kElems = 32;
  static constexpr int kPairs = 16;
  static constexpr int kUnitsPerScale = 4;
  static constexpr int kUC = 1;
  static constexpr bool kBias = true;
};
template <> struct Traits<QGEMV_INT8_ROW> {
  static constexpr int kElems = 16;
  static constexpr int kPairs = 8;
  static constexpr int kUnitsPerScale = -1;  // one scale per row
  static constexpr int kUC = 2;
  static constexpr bool kBias = false;
};
template <> struct Traits<QGEMV_INT4_G64> {
  static constexpr int kElems = 32;
  static constexpr int kPairs = 16;
  static constexpr int kUnitsPerScale = 2;
  static constexpr int kUC = 1;
  static constexpr bool kBias = true;
};

constexpr bool is_int8_fmt(int f) { return f == QGEMV_INT8_G32 || f == QGEMV_INT8_ROW; }

// Scales of one row of U units, and the scale of unit t (kUnitsPerScale:
// 0 none, -1 one per row, else units per scale group).
template <int FMT>
__device__ __forceinline__ int scales_per_row(int U) {
  constexpr int k = Traits<FMT>::kUnitsPerScale;
  return k > 0 ? U / k : (k < 0 ? 1 : 0);
}
template <int FMT>
__device__ __forceinline__ int scale_index(int t) {
  constexpr int k = Traits<FMT>::kUnitsPerScale;
  return k > 0 ? t / k : 0;
}

// Dword offset (within one batch row of x, stored as bf16 pairs) of the x
// values that pair with the first and the second half of unit t's pairs.
template <int FMT>
__device__ __forceinline__ void x_offsets(int t, int& lo, int& hi) {
  if constexpr (FMT == QGEMV_BF16) {
    lo = 4 * t; hi = lo;
  } else if constexpr (is_int8_fmt(FMT)) {
    lo = 8 * t; hi = lo + 4;
  } else if constexpr (FMT == QGEMV_Q4_0_G32) {
    // block t: low nibbles are elements 32t..32t+15, high nibbles 32t+16..32t+31
    lo = 16 * t; hi = lo + 8;
  } else if constexpr (FMT == QGEMV_INT4_G64) {
    // block t>>1, half c = t&1: low nibbles are elements 64(t>>1)+16c..+15,
    // high nibbles the same positions + 32
    lo = 32 * (t >> 1) + 8 * (t & 1); hi = lo + 16;
  } else {
    // block t>>2, quarter c = t&3: low nibbles are elements 128(t>>2)+16c..+15,
    // high nibbles the same positions + 64
    lo = 64 * (t >> 2) + 8 * (t & 3); hi = lo + 32;
  }
}

// Read the x dwords that pair with unit t from LDS (one batch row).
template <int FMT>
__device__ __forceinline__ void read_x(const uint32_t* xb, int t, uint32_t (&xv)[Traits<FMT>::kPairs]) {
  int lo, hi;
  x_offsets<FMT>(t, lo, hi);
  if constexpr (FMT == QGEMV_BF16) {
    u32x4 a = *reinterpret_cast<const u32x4*>(xb + lo);
    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
  } else if constexpr (is_int8_fmt(FMT)) {
    u32x4 a = *reinterpret_cast<const u32x4*>(xb + lo);
    u32x4 b = *reinterpret_cast<const u32x4*>(xb + hi);
    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
    xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
  } else {
    u32x4 a0 = *reinterpret_cast<const u32x4*>(xb + lo);
    u32x4 a1 = *reinterpret_cast<const u32x4*>(xb + lo + 4);
    u32x4 b0 = *reinterpret_cast<const u32x4*>(xb + hi);
    u32x4 b1 = *reinterpret_cast<const u32x4*>(xb + hi + 4);
    xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
    xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
    xv[8] = b0.x; xv[9] = b0.y; xv[10] = b0.z; xv[11] = b0.w;
    xv[12] = b1.x; xv[13] = b1.y; xv[14] = b1.z; xv[15] = b1.w;
  }
}

// Turn one 16-byte unit of codes into packed bf16 pairs, in the order of the
// x dwords read_x returns.
template <int FMT>
__device__ __forceinline__ void unpack(const u32x4& w, uint32_t (&p)[Traits<FMT>::kPairs]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  if constexpr (FMT == QGEMV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = wd[i];
  } else if constexpr (is_int8_fmt(FMT)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // sign-extended bytes -> float32 (exact); a float32 holding an integer of
      // at most 8 significant bits is exactly its own high half as bf16
      const float f0 = static_cast<float>(static_cast<int32_t>(wd[i] << 24) >> 24);
      const float f1 = static_cast<float>(static_cast<int32_t>(wd[i] << 16) >> 24);
      const float f2 = static_cast<float>(static_cast<int32_t>(wd[i] << 8) >> 24);
      const float f3 = static_cast<float>(static_cast<int32_t>(wd[i]) >> 24);
      p[2 * i] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                       __builtin_bit_cast(uint32_t, f0), 0x07060302u);
      p[2 * i + 1] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                           __builtin_bit_cast(uint32_t, f2), 0x07060302u);
    }
  } else {
    // byte j of the unit: low nibble -> element j of the low run, high nibble
    // -> element j of the high run. A byte holding a value 0..15 read as an
    // fp8 e4m3 number is value * 2^-9 (subnormals for 0..7, exponent 1 for
    // 8..15), so the fp8 -> bf16 conversion with scale 2^9 gives the code
    // exactly, two bytes per instruction.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = wd[i] & 0x0F0F0F0Fu;
      const uint32_t hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
      p[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));
      p[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));
      p[8 + 2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));
      p[8 + 2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));
    }
  }
}

// Reduce N values per lane over the 64 lanes of a wave. Each step exchanges
// half of the live values with lane ^ O and keeps the other half, so after
// log2(N) steps every lane holds one value (index = lane >> (6 - log2 N)),
// summed over 2^log2(N) lanes; plain butterflies finish the remaining lanes.
template <int N, int O>
__device__ __forceinline__ void halve(float* v, int lane) {
  if constexpr (N > 1) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = upper ? v[i + N / 2] : v[i];
      const float send = upper ? v[i] : v[i + N / 2];
      v[i] = keep + __shfl_xor(send, O);
    }
    halve<N / 2, O / 2>(v, lane);
  }
}

template <int O>
__device__ __forceinline__ float butterfly(float x) {
  if constexpr (O >= 1) {
    x += __shfl_xor(x, O);
    return butterfly<O / 2>(x);
  } else {
    return x;
  }
}

template <int N>
__device__ __forceinline__ float reduce_wave(float* v, int lane) {
  halve<N, 32>(v, lane);
  return butterfly<32 / N>(v[0]);
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Accumulate one unit of R rows against one batch row of x:
// acc[r] += scale_r * sum_p dot2(pair_rp, x_p) (+ the 4-bit bias start value).
template <int FMT, int R>
__device__ __forceinline__ void accumulate_unit(const uint32_t (&pr)[R][Traits<FMT>::kPairs],
                                                const float (&dsc)[R],
                                                const uint32_t (&xv)[Traits<FMT>::kPairs],
                                                float init, float* acc, int stride) {
  constexpr int P = Traits<FMT>::kPairs;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (FMT == QGEMV_BF16) {
      float a = acc[r * stride];
#pragma unroll
      for (int p = 0; p < P; ++p) a = dot2(pr[r][p], xv[p], a);
      acc[r * stride] = a;
    } else {
      float a = init;
#pragma unroll
      for (int p = 0; p < P; ++p) a = dot2(pr[r][p], xv[p], a);
      acc[r * stride] = __builtin_fmaf(dsc[r], a, acc[r * stride]);
    }
  }
}

// Scale factor applied to a unit's dot chain: the binary16 scale of the
// unit's group (1 for bf16).
template <int FMT>
__device__ __forceinline__ float unit_scale(uint32_t sbits) {
  if constexpr (FMT == QGEMV_BF16) return 1.f;
  else return half_to_float(static_cast<uint16_t>(sbits));
}

// Sum of the x values that pair with one unit, times -8: the start value of a
// 4-bit unit's dot chain, which turns sum(q x) into sum((q - 8) x).
template <int FMT>
__device__ __forceinline__ float bias_start(const uint32_t (&xv)[Traits<FMT>::kPairs]) {
  constexpr uint32_t kOnes = 0x3f803f80u;              // bf16 pair (1.0, 1.0)
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < Traits<FMT>::kPairs; ++p) s = dot2(xv[p], kOnes, s);
  return -8.f * s;
}

// ---------------------------------------------------------------------------
// Wave reduction without LDS round trips (for R * NB <= 8 partial sums).
// v_permlane32_swap / v_permlane16_swap exchange whole 16-lane rows between
// two registers: swap(X, Y) followed by one add leaves X's sum in the rows
// whose lane bit 5 (or 4) is 0 and Y's sum in the others, which halves the
// number of live values per lane in two instructions. The rest of a 16-lane
// row is reduced with DPP lane permutations folded into the adds.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowShr4 = 0x114;    // row_shr:4 (bound_ctrl: lanes 0-3 read 0)
constexpr int kDppRowShr8 = 0x118;    // row_shr:8
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// (the two results are copied out of the returned vector before the bit
// casts: a bit cast applied to a vector element directly read element 0 twice)
__device__ __forceinline__ float halve32(float x, float y) {   // x to bit5=0 lanes, y to bit5=1
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __uint_as_float(r0) + __uint_as_float(r1);
}
__device__ __forceinline__ float halve16(float x, float y) {   // x to bit4=0 lanes, y to bit4=1
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __uint_as_float(r0) + __uint_as_float(r1);
}
__device__ __forceinline__ float row_allreduce(float x) {      // every lane: sum over its 16-lane row
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return x;
}

// Reduce v[0..V) over the 64 lanes. Returns this lane's result; *idx is the
// value index it holds and *owner whether this lane stores it (one lane per
// index).
template <int V>
__device__ __forceinline__ float reduce_wave_rows(float* v, int lane, int* idx, bool* owner) {
  static_assert(V == 1 || V == 2 || V == 4 || V == 8, "V");
  const int b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1, b0 = lane & 1;
  // (the swaps write both operands, so a swap of a register with itself is
  // not a butterfly; the final cross-row steps pair the value with zero and
  // leave the complete sum in the rows whose bit is 0)
  if constexpr (V == 1) {
    float x = row_allreduce(v[0]);
    x = halve32(x, 0.f);
    x = halve16(x, 0.f);
    *idx = 0;
    *owner = lane == 0;
    return x;
  } else if constexpr (V == 2) {
    float x = halve32(v[0], v[1]);
    x = row_allreduce(x);
    x = halve16(x, 0.f);
    *idx = b5;
    *owner = (lane & 31) == 0;
    return x;
  } else if constexpr (V == 4) {
    const float a = halve32(v[0], v[2]);
    const float b = halve32(v[1], v[3]);
    float x = halve16(a, b);
    x = row_allreduce(x);
    *idx = 2 * b5 + b4;
    *owner = (lane & 15) == 0;
    return x;
  } else {
    const float a0 = halve32(v[0], v[4]), a1 = halve32(v[1], v[5]);
    const float a2 = halve32(v[2], v[6]), a3 = halve32(v[3], v[7]);
    const float c0 = halve16(a0, a2), c1 = halve16(a1, a3);
    // bit 0: lanes with bit0 = 0 keep c0, the others c1
    const float keep = b0 ? c1 : c0;
    const float send = b0 ? c0 : c1;
    float x = keep + dpp_f<kDppXor1>(send);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppRowShr4>(x);
    x += dpp_f<kDppRowShr8>(x);          // lanes 12..15 of each row hold the row sums
    *idx = 4 * b5 + 2 * b4 + b0;
    *owner = (lane & 14) == 12;          // lanes 12 and 13 of each row
    return x;
  }
}

// Buffer resource over `bytes` bytes at `base` (raw buffer: out-of-range
// loads return 0). Built from wave-uniform values, so it lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
#if QGEMV_NT_LOADS
constexpr int kWeightAux = 2;         // non-temporal
#else
constexpr int kWeightAux = 0;
#endif

// Sum over the 64 lanes, the same value in every lane, in a fixed order.
__device__ __forceinline__ float wave_sum(float x) {
  x = row_allreduce(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float rms_factor(float sumsq, int K, float eps) {
  return 1.f / sqrtf(sumsq / static_cast<float>(K) + eps);
}

// The lane that holds the value of index idx + NB after reduce_wave_rows<V>
// (the next row of a gate/up pair, same batch row) is lane ^ pair_xor: index
// bit log2(NB) lives in lane bit 5 (V = 2); 4, 5 (V = 4); 0, 4, 5 (V = 8).
template <int V, int NB>
constexpr int pair_xor() {
  return V == 2 ? 32 : V == 4 ? (NB == 1 ? 16 : 32) : (NB == 1 ? 1 : NB == 2 ? 16 : 32);
}

// One GEMV of a table walked by the register-x kernel. `start` is the index of
// the GEMV's first row group in the concatenation of all the table's groups.
struct TableEntry {
  const uint8_t* W;
  const uint16_t* S;
  const uint16_t* X;
  float* Y;
  int M;
  int K;
  int start;
  int shape;    // xreg_shape(R, NCH) of the entry
};

// (rows per wave step, 16-byte units per lane-column of a row) as one code
constexpr int xreg_shape(int R, int NCH) { return R * 16 + NCH; }

// Up to N independent GEMVs of one format and batch, passed by value (they
// live in the kernel-argument segment and are read with scalar loads).
template <int N>
struct GemvTable {
  int n;        // entries
  int total;    // row groups over all entries
  int am;       // entry whose outputs the fused argmax reads (grouped launch with argmax)
  int contig;   // nonzero: each wave takes one contiguous range of row groups (grouped launch)
  TableEntry e[N];
};

// The entry of a table whose entries' first row groups (or workgroups), read
// by key, ascend: the last entry e with key(e) <= v. Lane l reads entry l and
// a ballot counts the entries at or below v: one load, where walking the
// table costs one dependent scalar load per entry passed (a workgroup of the
// fifth entry waited for four of them before its first weight load). All 64
// lanes must be active; n <= 64.
template <typename Tab, typename Key>
__device__ __forceinline__ int find_entry(const Tab& tab, int v, Key key) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  bool le = false;
  if (lane < tab.n) le = key(tab.e[lane]) <= v;
  return __popcll(__builtin_amdgcn_ballot_w64(le)) - 1;
}

// Small-batch variant: x never goes through LDS. Lane l always works on the
// same NCH units (l, l+64, ...) of every row of a GEMV, so it loads the x
// values those units pair with once, straight into registers (with the 4-bit
// bias start values), and then only streams weights: no LDS, no barrier, and
// the first weight loads are in flight while x arrives.
//
// The kernel walks a table of GEMVs (one entry for qgemv_run, up to N for a
// grouped launch of independent GEMVs): the row groups of all entries are
// numbered consecutively and waves take them in a grid-stride loop (or, in
// a grouped launch with many row groups per wave, one contiguous range
// each), so one launch streams every entry's weights and pays the launch
// and ramp-up cost once. A wave reloads its x registers when its next row
// group belongs to another entry, and issues that group's loads before
// reducing the current one unless the entry's (R, NCH) differs.
// Fused-argmax state of a lane (see gemv_xreg_group_kernel): its running key
// over the LM-head outputs it stored, their batch row, and whether its wave
// has already published its keys.
struct AmLane {
  uint64_t key = 0;
  int b = 0;
  bool left = false;
};

// Workspace word of this wave's argmax key (per batch row): waves of
// workgroups 1.. in order (workgroup 0 collects).
__device__ __forceinline__ int am_slot() {
  return (static_cast<int>(blockIdx.x) - 1) * kWaves + static_cast<int>(threadIdx.x >> 6);
}

// Largest 64-bit key over the wave, in every lane: DPP inside 16-lane rows
// (quad swaps, rotations by 4 and 8), then permlane butterflies across rows
// (a swap of a register with itself returns rows (0,1,0,1) and (2,3,2,3)
// for 32 lanes, (0,0,2,2) and (1,1,3,3) for 16).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x >> 32), CTRL, 0xF, 0xF, false));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_umax64(uint64_t x) {
  x = umax64(x, dpp_u64<0xB1>(x));             // quad_perm [1,0,3,2]
  x = umax64(x, dpp_u64<0x4E>(x));             // quad_perm [2,3,0,1]
  x = umax64(x, dpp_u64<0x124>(x));            // row_ror:4
  x = umax64(x, dpp_u64<0x128>(x));            // row_ror:8
  {
    const auto l = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x >> 32), static_cast<uint32_t>(x >> 32), false, false);
    const uint32_t l0 = l[0], l1 = l[1], h0 = h[0], h1 = h[1];
    x = umax64((static_cast<uint64_t>(h0) << 32) | l0, (static_cast<uint64_t>(h1) << 32) | l1);
  }
  {
    const auto l = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x >> 32), static_cast<uint32_t>(x >> 32), false, false);
    const uint32_t l0 = l[0], l1 = l[1], h0 = h[0], h1 = h[1];
    x = umax64((static_cast<uint64_t>(h0) << 32) | l0, (static_cast<uint64_t>(h1) << 32) | l1);
  }
  return x;
}

// A wave is done with the LM-head entry: one wave-wide max per batch row,
// and lane b publishes row b's key in the wave's own workspace word (a
// relaxed device-scope store; key 1, which never wins, if the wave stored no
// output of the entry). No LDS and no counting among the workgroup's waves.
template <int NB>
__device__ __forceinline__ void am_leave(AmLane& am, uint64_t* __restrict__ slots, int batch, int lane) {
  uint64_t mine = 1;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint64_t k = wave_umax64(am.b == b ? am.key : uint64_t{0});
    if (lane == b) mine = umax64(k, 1);
  }
  if (lane < batch)
    __hip_atomic_store(slots + static_cast<size_t>(lane) * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + am_slot(),
                       mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  am.left = true;
}

// With AM, every output of entry tab.am a lane stores also goes into the
// lane's running argmax key, and after the wave's last row group of that
// entry the wave hands its keys over (am_leave).
// FUSED: the RMSNorm prologue (into xn, when given) and the epilogue of fu
// (one-entry tables).
template <int NB>
__device__ __forceinline__ void stage_norm_rows(const Fusion& fu, int K, int batch, uint32_t* xs, float* scr);

// first (with has_first): entry j's fields, already read by the caller, so
// that the first loads need no further table read.
template <int FMT, int NB, int R, int NCH, int N, bool AM = false, bool FUSED = false>
__device__ __forceinline__ int xreg_run(const GemvTable<N>& tab, int& j, int item, int stride,
                                        int batch, int lane, AmLane& am,
                                        uint64_t* am_slots, const Fusion& fu,
                                        uint32_t* xn = nullptr, int end = -1,
                                        const TableEntry& first = TableEntry{}, bool has_first = false,
                                        int first_next_start = 0) {
  if (end < 0) end = tab.total;                  // row groups item, item + stride, ... below end
  using T = Traits<FMT>;
  static_assert(!FUSED || R % 2 == 0, "gate/up pairs must share a row group");
  constexpr int P = T::kPairs;
  constexpr int kShape = xreg_shape(R, NCH);
  const uint8_t* W;
  const uint16_t* S;
  float* Y;
  int M, U, nsc, start, next_start, row_bytes;
  uint32_t xr[NB][NCH][P];
  float sx[NB][NCH];
  // per lane: byte offset of its unit in a row and of its unit's scale in a scale row
  int woff[NCH], soff[NCH];

  // make entry j current: its geometry (enter_geom), then this lane's x
  // registers (enter_x); use_first: the caller's copy of entry j (used once;
  // taken by value, never through a pointer that may point at either copy,
  // which would put the table in scratch memory)
  bool use_first = has_first;
  auto entry = [&](int jj) -> TableEntry {
    if (use_first) return first;
    return tab.e[jj];
  };
  auto enter_geom = [&](int jj) {
    const TableEntry e = entry(jj);
    W = e.W; S = e.S; Y = e.Y; M = e.M; start = e.start;
    next_start = use_first ? first_next_start : (N > 1 && jj + 1 < tab.n) ? tab.e[jj + 1].start : tab.total;
    U = e.K / T::kElems;
    row_bytes = U * 16;
    nsc = scales_per_row<FMT>(U);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int t = min(c * 64 + lane, U - 1);
      woff[c] = t * 16;
      soff[c] = scale_index<FMT>(t) * 2;
    }
  };
  auto enter_x = [&](int jj) {
    const TableEntry e = entry(jj);
    // (fused prologue: x was normalized into LDS by the workgroup, xn)
    const uint32_t* xsrc = reinterpret_cast<const uint32_t*>(e.X);
    if constexpr (FUSED) {
      if (xn != nullptr) xsrc = xn;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t* xb = xsrc + static_cast<size_t>(min(b, batch - 1)) * (e.K >> 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) read_x<FMT>(xb, min(c * 64 + lane, U - 1), xr[b][c]);
    }
  };
  auto enter = [&](int jj) {
    enter_geom(jj);
    enter_x(jj);
  };

  u32x4 wv[R][NCH];
  uint32_t sv[R][NCH];
  // loads of one row group through buffer resources whose base is the group's
  // first row (scalar address math); rows past M read as zero and are not stored
  auto load_step = [&](int grp) {
    const int row0 = grp * R;
    const int rows = min(R, M - row0);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(W + static_cast<size_t>(row0) * row_bytes, static_cast<uint32_t>(rows * row_bytes));
    // the row offset goes into the VGPR offset: the hardware range check
    // covers the VGPR and instruction offsets, not the SGPR offset
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        wv[r][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[c] + r * row_bytes, 0, kWeightAux));
    if constexpr (T::kUnitsPerScale != 0) {
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(S + static_cast<size_t>(row0) * nsc, static_cast<uint32_t>(rows * nsc * 2));
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          sv[r][c] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[c] + r * nsc * 2, 0, 0);
    }
  };
  auto bias_sums = [&]() {
    if constexpr (T::kBias) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < NCH; ++c) sx[b][c] = bias_start<FMT>(xr[b][c]);
    }
  };

  if constexpr (FUSED) {
    // The first row group's weight loads go out first: before the workgroup
    // normalizes x into LDS (every wave of the workgroup takes part in that,
    // with or without a row group of its own) and before this lane's x
    // loads, so their latency overlaps the prologue's. (In the unfused
    // kernels x is loaded first: issuing the weights first measured slower
    // on the grouped launch with the argmax.)
    const bool active = item < end;
    if (active) {
      enter_geom(j);
      load_step(item - start);
    }
    if (xn != nullptr) {
      const int K0 = tab.e[0].K;
      stage_norm_rows<NB>(fu, K0, batch, xn, reinterpret_cast<float*>(xn + NB * (K0 >> 1)));
    }
    if (!active) return item;
    enter_x(j);
  } else {
    enter(j);
    load_step(item - start);
  }
  use_first = false;
  bias_sums();

  float acc[R][NB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  while (true) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c * 64 + lane < U) {
        uint32_t pr[R][P];
        float dsc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          unpack<FMT>(wv[r][c], pr[r]);
          dsc[r] = unit_scale<FMT>(sv[r][c]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
          accumulate_unit<FMT, R>(pr, dsc, xr[b][c], T::kBias ? sx[b][c] : 0.f, &acc[0][b], NB);
      }
    }
    // issue the next row group's loads before reducing this one
    const int grp = item - start;
    const int cur_M = M;
    const int cur_j = j;
    float* cur_Y = Y;
    item += stride;
    bool more = item < end;
    bool switched = false;
    if (more) {
      if constexpr (N > 1) {
        if (item >= next_start) {
          while (j + 1 < tab.n && item >= tab.e[j + 1].start) ++j;
          if (tab.e[j].shape != kShape) {
            more = false;                // another shape: the caller dispatches it
          } else {
            enter(j);
            switched = true;
          }
        }
      }
      if (more) load_step(item - start);
    }
    {
      constexpr int V = R * NB;
      float v[V];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) { v[r * NB + b] = acc[r][b]; acc[r][b] = 0.f; }
      int idx;
      bool owner;
      const float res = reduce_wave_rows<V>(v, lane, &idx, &owner);
      const int r = idx / NB, b = idx % NB;
      const int row = grp * R + r;
      float partner = 0.f;
      if constexpr (FUSED) {
        if (fu.epi == kEpiSwiglu) partner = __shfl_xor(res, pair_xor<V, NB>());
      }
      if (owner && row < cur_M && b < batch) {
        float out = res;
        if constexpr (FUSED) out = epi_store(fu, cur_Y, cur_M, b, row, res, partner);
        else cur_Y[static_cast<size_t>(b) * cur_M + row] = res;
        if constexpr (AM) {
          if (cur_j == tab.am) {
            am.key = umax64(am.key, argmax_key(out, static_cast<uint32_t>(row)));
            am.b = b;
          }
        }
      }
    }
    if constexpr (AM) {
      // the entry's row groups are one contiguous range of items
      const int am_end = tab.am + 1 < tab.n ? tab.e[tab.am + 1].start : tab.total;
      if (cur_j == tab.am && !am.left && (item >= am_end || item >= end))
        am_leave<NB>(am, am_slots, batch, lane);
    }
    if (!more) break;
    if (switched) bias_sums();
  }
  return item;
}

// Row groups of a wave: item, item + stride, ... (grid-stride over the table).
// (with AM, workgroup 0 collects the argmax keys and the others work:
// first = 1)
template <int first = 0>
__device__ __forceinline__ int first_item(int& stride) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  stride = (gridDim.x - first) * kWaves;
  return (blockIdx.x - first) * kWaves + wave;
}

// One GEMV (or a table of GEMVs of one shape) with a fixed (R, NCH).
template <int FMT, int NB, int R, int NCH>
__global__ __launch_bounds__(kThreads) void gemv_xreg_kernel(const GemvTable<1> tab, int batch) {
  int stride;
  const int item = first_item(stride);
  if (item >= tab.total) return;                 // no barriers in this kernel
  int j = 0;
  AmLane am;
  xreg_run<FMT, NB, R, NCH, 1>(tab, j, item, stride, batch, threadIdx.x & 63, am, nullptr, Fusion{});
}

constexpr int kFusedSlots = QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW;   // most worker waves per launch
constexpr int kFusedMaxWorkers = kFusedSlots / kWaves;              // ... workgroups
constexpr int kFusedPerThread = kFusedSlots / kThreads;
constexpr int kFusedSpinLimit = 1 << 20;

// The fused argmax's last step, run by workgroup 0 of the launch, which does
// no GEMV work: wait until every wave of the other workgroups has published
// its key for each batch row (slots[b][am_slot()], nonzero once written),
// take the largest, write the index, and clear the slots for the next call.
// The argmax entry's row groups are the launch's first, so its keys are in
// while the other entries still stream, and this wait overlaps them. All of
// a thread's slot loads are in flight together; the wait is bounded (a key
// never published - which needs a workgroup that never runs - gives idx -1
// instead of a hang).
//
// kFusedChunk: a thread's words are taken that many at a time (their loads
// in flight together). All at once (kFusedPerThread) is fastest when the
// keys arrive early and the workers need more registers than the collector
// anyway (the grouped launch); 4 keeps the collector's registers, which set
// the whole kernel's budget, below a small worker's (the fused single GEMV).
template <int kFusedChunk>
__device__ __forceinline__ void fused_argmax_tail(uint64_t* __restrict__ slots, int batch,
                                                  int32_t* __restrict__ idx, uint64_t* red) {
  static_assert(kFusedPerThread % kFusedChunk == 0, "collector chunks");
  const int tid = threadIdx.x;
  const int grid = (gridDim.x - 1) * kWaves;            // worker waves (workgroups 1..)
  for (int b = 0; b < batch; ++b) {
    uint64_t* row = slots + static_cast<size_t>(b) * kFusedSlots;
    uint64_t key = 1;
    bool gave_up = false;          // a bounded wait ran out: the rest is read once, not waited for
    for (int k0 = 0; k0 < kFusedPerThread && k0 * kThreads < grid; k0 += kFusedChunk) {
      uint64_t v[kFusedChunk];
#pragma unroll
      for (int k = 0; k < kFusedChunk; ++k) v[k] = 0;
      bool pending = true;
      for (int spin = 0; pending && spin < (gave_up ? 1 : kFusedSpinLimit); ++spin) {
#pragma unroll
        for (int k = 0; k < kFusedChunk; ++k) {
          const int w = tid + (k0 + k) * kThreads;
          if (w < grid && v[k] == 0) v[k] = __hip_atomic_load(row + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        pending = false;
#pragma unroll
        for (int k = 0; k < kFusedChunk; ++k) pending |= (tid + (k0 + k) * kThreads < grid) && v[k] == 0;
        if (pending) __builtin_amdgcn_s_sleep(2);
      }
#pragma unroll
      for (int k = 0; k < kFusedChunk; ++k) {
        const int w = tid + (k0 + k) * kThreads;
        if (w < grid) {
          key = umax64(key, v[k]);
          __hip_atomic_store(row + w, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // (every slot of every chunk is cleared, arrived or not; after a
      // timeout, idx is -1, and a wave that publishes later still leaves its
      // word behind: the caller zeroes ws again, as the header says)
      gave_up |= pending;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) key = umax64(key, __shfl_xor(key, o));
    if ((tid & 63) == 0) red[tid >> 6] = key;
    const int all_arrived = __syncthreads_and(gave_up ? 0 : 1);
    if (tid == 0) {
      uint64_t m = red[0];
      for (int w = 1; w < kWaves; ++w) m = umax64(m, red[w]);
      idx[b] = (all_arrived && m > 1) ? argmax_index(m) : -1;
    }
    __syncthreads();
  }
}

// A table of GEMVs of one format whose entries may differ in (R, NCH): a
// wave runs the specialization of the entry its row group belongs to and
// moves to another specialization when its next row group does.
//
// AM: also idx[b] = argmax of row b of entry tab.am's output (the LM-head
// logits), in the same launch. The host puts that entry first, so its row
// groups are taken in the first rounds. Every lane folds the outputs it
// stores into a key; when a wave is done with the entry it publishes one key
// per batch row (a wave-wide max) into its own word of the caller's
// workspace with a relaxed device-scope store (no two waves touch one
// address: same-address atomics from thousands of waves would queue up).
// Workgroup 0 does no GEMV work and collects the words (fused_argmax_tail),
// most of them while the other entries still stream. A wave that stored no
// output of the entry publishes key 1, which never wins.
template <int FMT, int NB, int N, bool AM>
__global__ __launch_bounds__(kThreads) void gemv_xreg_group_kernel(const GemvTable<N> tab, int batch,
                                                                   uint64_t* __restrict__ slots,
                                                                   int32_t* __restrict__ idx) {
  __shared__ uint64_t red[kWaves];
  if constexpr (AM) {
    if (blockIdx.x == 0) {                      // the collector
      fused_argmax_tail<kFusedPerThread>(slots, batch, idx, red);
      return;
    }
  }
  // With the argmax: the table's header, entry 0 (the argmax entry) and
  // where entry 1 starts, at fixed offsets of the argument table, are read
  // together at the start with one wait (the empty asm needs every value
  // there). A wave whose first row group is in entry 0 (with strided row
  // groups, every wave) then issues its first loads one table round trip
  // after it starts instead of three (the walk or ballot, then the entry's
  // shape, then its fields, each waiting for the one before): the TinyLlama
  // set at batch 1 14.98 -> 14.60 us. (Without the argmax the first entry
  // holds fewer waves' first row groups, and the early wait measured
  // slower: the int8 set 13.94 -> 14.36 us.)
  const TableEntry e0 = AM ? tab.e[0] : TableEntry{};
  const int e1_start = AM && N > 1 ? tab.e[1].start : tab.total;   // (entries past n start at INT_MAX)
  const int t_total = tab.total, t_contig = tab.contig;
  if constexpr (AM) {
    asm volatile("" ::"s"(e0.W), "s"(e0.S), "s"(e0.X), "s"(e0.Y), "s"(e0.M), "s"(e0.K), "s"(e0.start),
                 "s"(e0.shape), "s"(e1_start), "s"(t_total), "s"(t_contig));
  }
  int stride;
  int item = first_item<AM ? 1 : 0>(stride);
  int end = t_total;
  if (t_contig) {
    // one contiguous range of row groups per wave (waves in order), so a
    // wave stays in one entry for many steps instead of reloading x at
    // almost every step
    const int nw = stride, wid = item;
    const int per = t_total / nw, rem = t_total % nw;
    item = wid * per + min(wid, rem);
    end = item + per + (wid < rem ? 1 : 0);
    stride = 1;
  }
  const int lane = threadIdx.x & 63;
  AmLane am;
  if (item < end) {
    int j = 0;
    if constexpr (N > 1) {
      if (!AM || item >= e1_start) j = find_entry(tab, item, [](const TableEntry& e) { return e.start; });
    }
    bool has_first = AM && j == 0;
    while (item < end) {
      if constexpr (AM) {
        if (j > tab.am && !am.left) am_leave<NB>(am, slots, batch, lane);   // past the entry
      }
      switch (has_first ? e0.shape : tab.e[j].shape) {
#define QG_SHAPE(R_, C_) \
        case xreg_shape(R_, C_): \
          item = xreg_run<FMT, NB, R_, C_, N, AM>(tab, j, item, stride, batch, lane, am, slots, Fusion{}, nullptr, end, \
                                                  e0, has_first, e1_start); break;
        // the shapes launch_gemv_group produces (the kernel's register budget,
        // and with it its occupancy, is the largest of theirs)
        QG_SHAPE(4, 1) QG_SHAPE(2, 1)
        case xreg_shape(8, 1):                   // batch 1, contiguous ranges only
          if constexpr (NB == 1)
            item = xreg_run<FMT, NB, 8, 1, N, AM>(tab, j, item, stride, batch, lane, am, slots, Fusion{}, nullptr, end,
                                                  e0, has_first, e1_start);
          else
            item = end;
          break;
        QG_SHAPE(QGEMV_GROUP_R2, 2)
        QG_SHAPE(QGEMV_GROUP_RLONG, 3) QG_SHAPE(QGEMV_GROUP_RLONG, 4)
        case xreg_shape(1, 8):                   // int8 at batch 1 only
          if constexpr (is_int8_fmt(FMT) && NB == 1)
            item = xreg_run<FMT, NB, 1, 8, N, AM>(tab, j, item, stride, batch, lane, am, slots, Fusion{}, nullptr, end,
                                                  e0, has_first, e1_start);
          else
            item = tab.total;
          break;
#undef QG_SHAPE
        default: item = tab.total;               // not produced by the host
      }
      has_first = false;
    }
  }
  if constexpr (AM) {
    if (!am.left) am_leave<NB>(am, slots, batch, lane);
  }
}


// ---------------------------------------------------------------------------
// Batch 3..8: matrix cores.
//
// From batch 3 on, the dot-product kernels above spend one dot2 instruction
// per weight pair and batch row and become bound by the vector ALUs instead
// of HBM. The matrix-core kernel below hands the products to
// v_mfma_f32_4x4x4bf16_1k; the vector ALUs only unpack codes (exactly, as
// above) and apply each unit's scale.
//
// Work split: a workgroup takes a contiguous range of 8- or 16-row tiles of
// one GEMV (in a grouped launch, the workgroups are shared out among the
// GEMVs of one format, whatever their K); its waves split the range's
// (tile, step) pairs evenly (see mfma_tiles).

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four int8 codes -> two bf16 pairs (in byte order).
__device__ __forceinline__ void int8x4_to_bf16(uint32_t d, uint32_t& p0, uint32_t& p1) {
  const float f0 = static_cast<float>(static_cast<int32_t>(d << 24) >> 24);
  const float f1 = static_cast<float>(static_cast<int32_t>(d << 16) >> 24);
  const float f2 = static_cast<float>(static_cast<int32_t>(d << 8) >> 24);
  const float f3 = static_cast<float>(static_cast<int32_t>(d) >> 24);
  p0 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  p1 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

constexpr int kMfmaMaxThreads = 1024;
typedef short v4i16 __attribute__((ext_vector_type(4)));
// rows per matrix-core tile: 2 (batch 5..8) or 4 (batch 3..4) groups of 4
template <int NB> constexpr int kMfmaTileRows = NB == 8 ? 8 : 16;

// One GEMV of a matrix-core launch: workgroups wg0 .. wg0 + nwg - 1 of the
// launch take contiguous, balanced ranges of its 16-row tiles.
struct MfmaEntry {
  const uint8_t* W;
  const uint16_t* S;
  const uint16_t* X;
  float* Y;
  int M;
  int K;
  int wg0;
  int nwg;
};

// Up to N GEMVs of one format and batch, any K (by value: kernel arguments).
template <int N>
struct MfmaTable {
  int n;
  int am;       // entry whose output's argmax the launch computes (-1: none)
  int pad[2];
  MfmaEntry e[N];
};

// Where the matrix-core launch's argmax meets: row b's key of the entry's
// workgroup w in slots[b * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + w].
struct MfmaArgmax {
  uint64_t* slots = nullptr;   // nullptr: this workgroup's entry has no argmax
  int wg = 0;                  // this workgroup within the entry
};

// The argmax of a matrix-core launch, run by its workgroup 0 (which does no
// GEMV work) while the others stream: wait until each of the argmax entry's
// nwords workgroups has published its key for every batch row
// (slots[b * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + w], nonzero once
// written), take the largest, write idx[b], and clear the words again. A
// thread takes words tid, tid + blockDim.x, ..., all batch rows' loads in
// flight together. The wait is bounded: a key never published (which needs
// a workgroup that never runs) gives idx -1 instead of a hang. red: LDS for
// NB + 1 words per wave (the kernel's dynamic LDS: a reduction through
// static LDS, as __syncthreads_and uses, would leave the dynamic LDS short
// of the 160 KiB a workgroup may take). (Before, a one-workgroup kernel
// launched after the matrix-core launch took the keys: 4.5 us plus its
// launch gap, at batch 8.)
constexpr int kMaxArgmaxKeyWords = 8 * 64;     // argmax workgroups per launch (<= a collector's threads)
template <int NB>
__device__ __forceinline__ void mfma_argmax_collect(uint64_t* __restrict__ slots, int nwords, int batch,
                                                    int32_t* __restrict__ idx, uint64_t* red) {
  const int tid = static_cast<int>(threadIdx.x), nt = static_cast<int>(blockDim.x);
  const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  uint64_t key[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) key[b] = 1;
  bool gave_up = false;
  for (int w = tid; w < nwords; w += nt) {
    uint64_t v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] = b < batch ? 0 : 1;
    bool pending = true;
    for (int spin = 0; pending && spin < (gave_up ? 1 : kFusedSpinLimit); ++spin) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (v[b] == 0)
          v[b] = __hip_atomic_load(slots + static_cast<size_t>(b) * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + w,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pending = false;
#pragma unroll
      for (int b = 0; b < NB; ++b) pending |= v[b] == 0;
      if (pending) __builtin_amdgcn_s_sleep(2);
    }
    gave_up |= pending;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < batch) {
        key[b] = umax64(key[b], v[b]);
        __hip_atomic_store(slots + static_cast<size_t>(b) * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + w, uint64_t{0},
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  const bool wave_gave_up = __builtin_amdgcn_ballot_w64(gave_up) != 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint64_t k = wave_umax64(key[b]);
    if (lane == 0) red[wave * (NB + 1) + b] = k;
  }
  if (lane == 0) red[wave * (NB + 1) + NB] = wave_gave_up ? 1 : 0;
  __syncthreads();
  if (tid < batch) {
    uint64_t m = 1;
    bool all_arrived = true;
    for (int w = 0; w < nw; ++w) {
      m = umax64(m, red[w * (NB + 1) + tid]);
      all_arrived &= red[w * (NB + 1) + NB] == 0;
    }
    idx[tid] = (all_arrived && m > 1) ? argmax_index(m) : -1;
  }
}
constexpr int kNormFactorOff = (kMfmaMaxThreads / 64) * QGEMV_MAX_BATCH;   // floats
static_assert((kNormFactorOff + QGEMV_MAX_BATCH) * 4 <= static_cast<int>(kNormScratchBytes), "norm scratch");

// Block-wide RMSNorm factors of the fused prologue: scr[kNormFactorOff + b]
// = 1 / sqrt(mean of h[b][:]^2 + eps) for b < batch (scr: kNormScratchBytes
// of LDS). Thread t sums k = 4t, 4t + 4 * threads, ... of every batch row
// (the loads of all rows issued together), the waves' sums are added in
// wave order. Ends with a barrier; every thread must call it.
template <int NB>
__device__ __forceinline__ void block_rms_factors(const Fusion& fu, int K, int batch, float* scr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = static_cast<int>(blockDim.x >> 6);
  float s[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) s[b] = 0.f;
  for (int k = 4 * tid; k < K; k += 4 * static_cast<int>(blockDim.x)) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // rows past the batch re-read the last row (in bounds; not used)
      const f32x4 v = *reinterpret_cast<const f32x4*>(fu.h + static_cast<size_t>(min(b, batch - 1)) * K + k);
      s[b] = __builtin_fmaf(v.x, v.x, s[b]);
      s[b] = __builtin_fmaf(v.y, v.y, s[b]);
      s[b] = __builtin_fmaf(v.z, v.z, s[b]);
      s[b] = __builtin_fmaf(v.w, v.w, s[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float t = wave_sum(s[b]);
    if (lane == 0) scr[wave * QGEMV_MAX_BATCH + b] = t;
  }
  __syncthreads();
  if (tid < batch) {
    float t = 0.f;
    for (int w = 0; w < nw; ++w) t += scr[w * QGEMV_MAX_BATCH + tid];
    scr[kNormFactorOff + tid] = rms_factor(t, K, fu.eps);
  }
  __syncthreads();
}

// The fused prologue for kernels that keep x rows contiguous: LDS
// xs[b][0..K) = bf16(h[b][k] * r_b * g[k]) for b < NB (rows past the batch
// zero), 8 elements per 16-byte chunk. Barriers inside; every thread must
// call it.
//
// One pass at batch <= 2 with at most two chunks of a row per thread (K <=
// 16 * threads): thread t loads chunks t and t + threads of every row and
// the matching g once, sums its squares (chunk t's eight elements, then
// chunk t + threads'), the waves' sums go through LDS, and every thread adds
// them in wave order for the factors of its rows, then scales the values it
// holds. Otherwise h is read twice (block_rms_factors, then the scaling).
// Either way a row's sum of squares is taken in an order set by K and the
// workgroup size alone, not by the batch.
template <int NB>
__device__ __forceinline__ void stage_norm_rows(const Fusion& fu, int K, int batch, uint32_t* xs, float* scr) {
  const int row_chunks = K / 8, nxc = NB * row_chunks;
  const int nt = static_cast<int>(blockDim.x);
  if constexpr (NB <= 2) {
    if (row_chunks <= 2 * nt) {
      const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
      f32x4 h0[NB][2], h1[NB][2];
      u32x4 gg[2];
      bool have[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = tid + u * nt;
        have[u] = c < row_chunks;
        gg[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < NB; ++b) { h0[b][u] = f32x4{0.f, 0.f, 0.f, 0.f}; h1[b][u] = h0[b][u]; }
        if (have[u]) {
          gg[u] = *reinterpret_cast<const u32x4*>(fu.g + 8 * c);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            // rows past the batch re-read the last row (in bounds; stored as zero)
            const float* hr = fu.h + static_cast<size_t>(min(b, batch - 1)) * K + 8 * c;
            h0[b][u] = *reinterpret_cast<const f32x4*>(hr);
            h1[b][u] = *reinterpret_cast<const f32x4*>(hr + 4);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float sq = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sq = __builtin_fmaf(h0[b][u][e], h0[b][u][e], sq);
#pragma unroll
          for (int e = 0; e < 4; ++e) sq = __builtin_fmaf(h1[b][u][e], h1[b][u][e], sq);
        }
        const float t = wave_sum(sq);
        if (lane == 0) scr[wave * QGEMV_MAX_BATCH + b] = t;
      }
      __syncthreads();
      const int nw = nt >> 6;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float t = 0.f;
        for (int w = 0; w < nw; ++w) t += scr[w * QGEMV_MAX_BATCH + b];
        const float r = b < batch ? rms_factor(t, K, fu.eps) : 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (!have[u]) continue;
          const u32x4 g = gg[u];
          const f32x4 a = h0[b][u], c = h1[b][u];
          u32x4 v = {pack_bf16(a.x * r * bf16_lo(g.x), a.y * r * bf16_hi(g.x)),
                     pack_bf16(a.z * r * bf16_lo(g.y), a.w * r * bf16_hi(g.y)),
                     pack_bf16(c.x * r * bf16_lo(g.z), c.y * r * bf16_hi(g.z)),
                     pack_bf16(c.z * r * bf16_lo(g.w), c.w * r * bf16_hi(g.w))};
          if (b >= batch) v = u32x4{0u, 0u, 0u, 0u};
          reinterpret_cast<u32x4*>(xs)[b * row_chunks + tid + u * nt] = v;
        }
      }
      __syncthreads();
      return;
    }
  }
  block_rms_factors<NB>(fu, K, batch, scr);
  // rounds of four chunks per thread (their loads issued together) while
  // all four exist, then one chunk per round
  int base = threadIdx.x;
  auto round = [&](auto width) {
    constexpr int kW = decltype(width)::value;
    f32x4 h0[kW], h1[kW];
    u32x4 gg[kW];
    float r[kW];
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      const int i = base + u * nt;
      const int b = i / row_chunks, c = i - b * row_chunks;
      const float* hr = fu.h + static_cast<size_t>(min(b, batch - 1)) * K + 8 * c;
      h0[u] = *reinterpret_cast<const f32x4*>(hr);
      h1[u] = *reinterpret_cast<const f32x4*>(hr + 4);
      gg[u] = *reinterpret_cast<const u32x4*>(fu.g + 8 * c);
      r[u] = b < batch ? scr[kNormFactorOff + b] : -1.f;      // -1: a row past the batch
    }
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      const int i = base + u * nt;
      {
        u32x4 v = {pack_bf16(h0[u].x * r[u] * bf16_lo(gg[u].x), h0[u].y * r[u] * bf16_hi(gg[u].x)),
                         pack_bf16(h0[u].z * r[u] * bf16_lo(gg[u].y), h0[u].w * r[u] * bf16_hi(gg[u].y)),
                         pack_bf16(h1[u].x * r[u] * bf16_lo(gg[u].z), h1[u].y * r[u] * bf16_hi(gg[u].z)),
                         pack_bf16(h1[u].z * r[u] * bf16_lo(gg[u].w), h1[u].w * r[u] * bf16_hi(gg[u].w))};
        if (r[u] < 0.f) v = u32x4{0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4*>(xs)[i] = v;
      }
    }
    base += kW * nt;
  };
  while (base + 3 * nt < nxc) round(std::integral_constant<int, 4>{});
  while (base < nxc) round(std::integral_constant<int, 1>{});
  __syncthreads();
}

// Units [g0, g1) of one entry (the body of the matrix-core kernel).
// FUSED: the operations of fu fused in (prologue in the x staging, epilogue
// in the store); the LDS then ends with kNormScratchBytes of scratch.
// ---- matrix-core kernel (batch 3..8) -------------------------------------
// The products go to v_mfma_f32_4x4x4bf16_1k: 16 independent 4 x 4 x 4
// blocks per instruction. Block b (lanes 4b .. 4b + 3) takes its own stretch
// of K, so a lane group needs only four weight rows at one position of K:
//   A (x):       lane 4b + i holds 4 consecutive x values of batch row i
//   B (weights): lane 4b + j holds the same 4 positions of weight row j
//   D:           lane 4b + j, register r: sum over the 4 positions, batch
//                row r, weight row j
// A load instruction reads 4 rows x 256 bytes (lane 4b + j: row j, 16-byte
// unit b), and the unit's codes feed the B operand in place: no lane
// exchange. A unit is one scale group or a part of one (4-bit: 32 weights,
// int8: 16, bf16: 8), so each lane applies one scale per unit to its D
// registers; the 4-bit offset (codes stored as w + 8) is removed by starting
// each unit's chain at -8 * (sum of the unit's x), the bias identity of the
// Rust page's Lesson 6. At the end of a tile each lane's running sums are
// added across the 16 lane groups (permlane swaps, then DPP row rotations).
// Batch rows come in halves of 4 (batch 5..8: two A operands per position,
// each B operand used twice).
template <int FMT> struct M4 {
  static constexpr int kUnitElems = Traits<FMT>::kElems;    // weights per 16-byte unit
  static constexpr int kSub = kUnitElems / 4;               // MFMA positions of 4 per unit
  static constexpr int kStepElems = 16 * kUnitElems;        // a step: 16 units of each row
  static constexpr bool kBias = Traits<FMT>::kBias;         // 4-bit: the -8 offset
  // scales: 0 none, -1 one per row, else units per scale group
  static constexpr int kUnitsPerScale = Traits<FMT>::kUnitsPerScale;
};

// K element of the first of the 4 positions of MFMA step s of unit u
// (nibble order: Q4_0 element j / j + 16, g64 j / j + 32, g128 j / j + 64 in
// the low / high nibble of byte j; a 4-bit unit is a 16-byte quarter (g128),
// half (g64) or all (Q4_0) of its group's codes)
template <int FMT>
__device__ __forceinline__ int m4_elem(int u, int s) {
  if constexpr (FMT == QGEMV_BF16) return 8 * u + 4 * s;
  else if constexpr (is_int8_fmt(FMT)) return 16 * u + 4 * s;
  else {
    const int d = s >> 1, h = s & 1;               // dword d, low (0) or high (1) nibbles
    if constexpr (FMT == QGEMV_Q4_0_G32) return 32 * u + 16 * h + 4 * d;
    else if constexpr (FMT == QGEMV_INT4_G64) return 64 * (u >> 1) + 16 * (u & 1) + 32 * h + 4 * d;
    else return 128 * (u >> 2) + 16 * (u & 3) + 64 * h + 4 * d;
  }
}

// B operand (4 bf16) of MFMA step s of a unit's 16 code bytes
template <int FMT>
__device__ __forceinline__ v4i16 m4_b(const u32x4& w, int s) {
  uint32_t lo, hi;
  if constexpr (FMT == QGEMV_BF16) {
    lo = s ? w.z : w.x;
    hi = s ? w.w : w.y;
  } else if constexpr (is_int8_fmt(FMT)) {
    const uint32_t d = s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
    int8x4_to_bf16(d, lo, hi);
  } else {
    const int di = s >> 1;
    const uint32_t d = di == 0 ? w.x : di == 1 ? w.y : di == 2 ? w.z : w.w;
    const uint32_t n = (s & 1) ? ((d >> 4) & 0x0F0F0F0Fu) : (d & 0x0F0F0F0Fu);
    // a byte q in 0..15 read as e4m3 is q * 2^-9: the conversion's scale 2^9 makes it exact
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(n, 512.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(n, 512.0f, true));
  }
  const u32x2 v = {lo, hi};
  return __builtin_bit_cast(v4i16, v);
}

// x in LDS: batch row r, element e at byte r * m4_xrow(K) + 136 * (e / 64) +
// 2 * (e % 64): 64-element runs padded by 8 bytes and a row stride of 8 * c
// bytes past a multiple of 128, so that the 16 lanes an A read serves
// together fall on distinct bank pairs (c from the format's unit pattern).
template <int FMT>
__host__ __device__ constexpr int m4_bank_shift() {
  return (FMT == QGEMV_INT8_G32 || FMT == QGEMV_INT8_ROW || FMT == QGEMV_INT4_G128) ? 1 : 2;
}
template <int FMT>
__host__ __device__ __forceinline__ uint32_t m4_xrow(int K) {
  const uint32_t run = 136u * static_cast<uint32_t>((K + 63) / 64);
  return (run + 127u) / 128u * 128u + 8u * m4_bank_shift<FMT>();
}
__device__ __forceinline__ uint32_t m4_xoff(int e) {
  return 136u * static_cast<uint32_t>(e >> 6) + 2u * static_cast<uint32_t>(e & 63);
}

template <int CTRL>
__device__ __forceinline__ f32x4 dpp4(const f32x4& v) {
  f32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = dpp_f<CTRL>(v[k]);
  return o;
}
constexpr int kDppRowRor8 = 0x128;    // row_ror:8
constexpr int kDppRowRor4 = 0x124;    // row_ror:4

// Tiles t0 .. t1 - 1 (kTR rows each) of one GEMV by one workgroup. The
// workgroup's (tile, step) pairs are laid end to end and every wave takes an
// equal contiguous share, so all waves stream the same number of steps
// whatever the tile count, and no barrier stands between tiles. A wave
// stores a tile it holds whole; a tile split between waves leaves one
// partial result per wave in LDS, and after the workgroup's last barrier the
// wave holding the tile's last step adds them in wave order (a fixed order:
// results are deterministic, and a row's arithmetic does not depend on the
// batch or on the other rows).
template <int FMT, int NB, bool FUSED = false, bool AM = false>
__device__ __forceinline__ void mfma_tiles(const MfmaEntry& ent, int t0, int t1, int batch,
                                           u32x4* lds_v4, const Fusion& fu, const MfmaArgmax& amx = MfmaArgmax{}) {
  using F = M4<FMT>;
  constexpr int NBh = NB / 4;                          // batch halves of 4 rows
  constexpr int R = NB == 8 ? 2 : 4;                   // row groups of 4 rows per tile
  constexpr int kTR = 4 * R;                           // rows per tile
  constexpr int kV = R * NBh * 4;                      // running sums per lane (16)
  static_assert(kV == 16, "sums per lane");
  constexpr bool kScaled = F::kUnitsPerScale > 0;      // a scale per group inside the row
  const uint8_t* __restrict__ W = ent.W;
  const uint16_t* __restrict__ S = ent.S;
  const uint16_t* __restrict__ X = ent.X;
  float* __restrict__ Y = ent.Y;
  const int M = ent.M, K = ent.K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int lb = lane >> 2, lj = lane & 3;             // MFMA block (unit of the step), row / batch index
  const int nst = K / F::kStepElems;                   // steps per tile
  const int nflat = (t1 - t0) * nst;                   // the workgroup's (tile, step) pairs
  const int va = static_cast<int>(static_cast<long>(wave) * nflat / nw);
  const int vb = static_cast<int>(static_cast<long>(wave + 1) * nflat / nw);
  const uint32_t row_bytes = static_cast<uint32_t>(
      FMT == QGEMV_BF16 ? 2 * K : is_int8_fmt(FMT) ? K : K / 2);
  const int spr = F::kUnitsPerScale > 0 ? (K / F::kUnitElems) / F::kUnitsPerScale : 0;   // scales per row
  const int nunits = K / F::kUnitElems;
  const uint32_t xrow = m4_xrow<FMT>(K);
  // LDS: partial tiles [waves][2][16 lanes] f32x4 | RMSNorm scratch (fused) |
  //      x [NB][xrow bytes] | -8 * unit sums [nunits][NB] (4-bit)
  f32x4* part = reinterpret_cast<f32x4*>(lds_v4);
  float* scr = reinterpret_cast<float*>(part + nw * 2 * 16);
  char* xs = reinterpret_cast<char*>(scr) + (FUSED ? kNormScratchBytes : 0);
  float* sneg = reinterpret_cast<float*>(xs + static_cast<size_t>(NB) * xrow);

  // Loads of one step: the tile's buffer resources are rebuilt when the tile
  // changes; a step past the wave's share uses resources of zero range, so
  // its loads read zero and move no data.
  int rkey = -1;
  __amdgpu_buffer_rsrc_t rw = make_rsrc(W, 0), rs = make_rsrc(S, 0);
  const uint32_t woff = lj * row_bytes + 16 * lb;
  auto load = [&](u32x4 (&w)[R], uint32_t (&s)[R], int tile, int st, bool live) {
    const int key = live ? tile : -2;
    if (key != rkey) {
      rkey = key;
      const int row0 = tile * kTR;
      // (a select and a min rather than a clamp: see the register-x kernel)
      const int rows = (live && row0 < M) ? min(kTR, M - row0) : 0;
      rw = make_rsrc(W + (rows ? static_cast<size_t>(row0) * row_bytes : 0), static_cast<uint32_t>(rows) * row_bytes);
      if constexpr (kScaled)
        rs = make_rsrc(S + (rows ? static_cast<size_t>(row0) * spr : 0), static_cast<uint32_t>(rows * spr * 2));
    }
    // row lj of each row group, unit lb of the step: the VGPR offset (range
    // checked: rows past M read as zero); the step's offset in the SGPR offset
    const int so = st * (16 * 16);
#pragma unroll
    for (int g = 0; g < R; ++g)
      w[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff + 4 * g * row_bytes, so, kWeightAux));
    if constexpr (kScaled) {
      const int sidx = (st * 16 + lb) / F::kUnitsPerScale;
#pragma unroll
      for (int g = 0; g < R; ++g)
        s[g] = __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<uint32_t>(((4 * g + lj) * spr + sidx) * 2), 0, 0);
    }
  };

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 tot[R][NBh];                                   // running sums of this tile
#pragma unroll
  for (int g = 0; g < R; ++g)
#pragma unroll
    for (int h = 0; h < NBh; ++h) tot[g][h] = zero;

  auto compute = [&](const u32x4 (&w)[R], const uint32_t (&s)[R], int st) {
    const int u = st * 16 + lb;                        // this lane group's unit
    f32x4 d[R][NBh];
    f32x4 c0[NBh];
#pragma unroll
    for (int h = 0; h < NBh; ++h) {
      if constexpr (F::kBias) c0[h] = *reinterpret_cast<const f32x4*>(sneg + u * NB + 4 * h);
      else c0[h] = zero;
    }
#pragma unroll
    for (int g = 0; g < R; ++g)
#pragma unroll
      for (int h = 0; h < NBh; ++h) d[g][h] = kScaled ? c0[h] : tot[g][h];
#pragma unroll
    for (int sub = 0; sub < F::kSub; ++sub) {
      const uint32_t xo = m4_xoff(m4_elem<FMT>(u, sub));
      v4i16 a[NBh];
#pragma unroll
      for (int h = 0; h < NBh; ++h)
        a[h] = __builtin_bit_cast(v4i16, *reinterpret_cast<const u32x2*>(xs + (4 * h + lj) * xrow + xo));
#pragma unroll
      for (int g = 0; g < R; ++g) {
        const v4i16 bv = m4_b<FMT>(w[g], sub);
#pragma unroll
        for (int h = 0; h < NBh; ++h) d[g][h] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a[h], bv, d[g][h], 0, 0, 0);
      }
    }
#pragma unroll
    for (int g = 0; g < R; ++g) {
      if constexpr (kScaled) {
        const float sc = half_to_float(static_cast<uint16_t>(s[g]));
#pragma unroll
        for (int h = 0; h < NBh; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) tot[g][h][r] = __builtin_fmaf(sc, d[g][h][r], tot[g][h][r]);
      } else {
#pragma unroll
        for (int h = 0; h < NBh; ++h) tot[g][h] = d[g][h];
      }
    }
  };

  // The tile's sums added over the 16 lane groups: value v = 4 (g * NBh + h)
  // + r goes through two halvings (v bit 0 <-> lane bit 5, v bit 1 <-> lane
  // bit 4), then rotations by 8 and 4 inside each 16-lane row; afterwards
  // register n of every lane holds the total of v = 4n + 2 (lane bit 4) +
  // (lane bit 5), for weight row 4 (v >> 2) / NBh + (lane & 3).
  auto reduce = [&]() {
    float t[kV];
#pragma unroll
    for (int g = 0; g < R; ++g)
#pragma unroll
      for (int h = 0; h < NBh; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[(g * NBh + h) * 4 + r] = tot[g][h][r];
    float u8[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) u8[m] = halve32(t[2 * m], t[2 * m + 1]);
    f32x4 q;
#pragma unroll
    for (int n = 0; n < 4; ++n) q[n] = halve16(u8[2 * n], u8[2 * n + 1]);
    const f32x4 q8 = dpp4<kDppRowRor8>(q);
#pragma unroll
    for (int n = 0; n < 4; ++n) q[n] += q8[n];
    const f32x4 q4 = dpp4<kDppRowRor4>(q);
#pragma unroll
    for (int n = 0; n < 4; ++n) q[n] += q4[n];
#pragma unroll
    for (int g = 0; g < R; ++g)
#pragma unroll
      for (int h = 0; h < NBh; ++h) tot[g][h] = zero;
    return q;
  };

  // results -> y (lanes whose bits 3, 2 are 0 store; the row paired with row
  // 2i of a gate/up pair is in the lane next to it)
  const int vlo = 2 * ((lane >> 4) & 1) + ((lane >> 5) & 1);
  // argmax keys of the outputs this lane stores: batch rows vlo (+ 4)
  uint64_t amk[NBh];
#pragma unroll
  for (int h = 0; h < NBh; ++h) amk[h] = 0;
  const bool am_on = AM && amx.slots != nullptr;
  auto store = [&](const f32x4& q_in, int tile) {
    f32x4 q = q_in;
    if constexpr (FMT == QGEMV_INT8_ROW) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int v = 4 * n + vlo;
        const int row = tile * kTR + 4 * ((v >> 2) / NBh) + lj;
        q[n] *= half_to_float(S[min(row, M - 1)]);     // the row's scale, once per dot product
      }
    }
    f32x4 pq = q;
    if constexpr (FUSED) {
      if (fu.epi == kEpiSwiglu) pq = dpp4<kDppXor1>(q);
    }
    if (((lane >> 2) & 3) == 0) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int v = 4 * n + vlo;
        const int b = 4 * ((v >> 2) % NBh) + (v & 3);
        const int row = tile * kTR + 4 * ((v >> 2) / NBh) + lj;
        if (row < M && b < batch) {
          float out = q[n];
          if constexpr (FUSED) out = epi_store(fu, Y, M, b, row, q[n], pq[n]);
          else Y[static_cast<size_t>(b) * M + row] = q[n];
          if constexpr (AM) {
            if (am_on) amk[n % NBh] = umax64(amk[n % NBh], argmax_key(out, static_cast<uint32_t>(row)));
          }
        }
      }
    }
  };
  const int pslot = ((lane >> 4) << 2) | lj;           // lanes with bits 3, 2 = 0 -> 0..15

  // the wave's share [va, vb) of the (tile, step) sequence
  const int tfirst = t0 + va / nst;
  int lt = tfirst, ls = va - (va / nst) * nst, lv = va;
  int ct = lt, cs = ls, cv = va;
  auto issue = [&](u32x4 (&w)[R], uint32_t (&s)[R]) {
    load(w, s, lt, ls, lv < vb);
    if (++ls == nst) { ls = 0; ++lt; }
    ++lv;
  };
  auto step = [&](const u32x4 (&w)[R], const uint32_t (&s)[R]) {
    compute(w, s, cs);
    if (cs == nst - 1 || cv == vb - 1) {
      const f32x4 q = reduce();
      const int fstart = (ct - t0) * nst;              // the tile's first flattened step
      if (fstart >= va && fstart + nst <= vb) {
        store(q, ct);                                  // the whole tile is this wave's
      } else if (((lane >> 2) & 3) == 0) {
        part[(wave * 2 + (ct == tfirst ? 0 : 1)) * 16 + pslot] = q;
      }
    }
    if (++cs == nst) { cs = 0; ++ct; }
    ++cv;
  };

  // steps of weights in flight: three of 2 KiB per wave (8-row tiles) or two
  // of 4 KiB (16-row tiles); all but one issued before x is staged
  constexpr int kDepth = R == 2 ? 3 : 2;
  u32x4 w0[R], w1[R], w2[R];
  uint32_t s0[R], s1[R], s2[R];

  // ---- stage x (all K, NB rows; rows >= batch as zero): 8 elements per
  // thread per round, two 8-byte LDS stores. The first round's x loads go
  // out before the first weight steps (loads complete in order: x issued
  // behind the weights waits for them, 3.3 us in the TinyLlama set at batch
  // 4; the step time is the same either way, since the first weight steps'
  // round trip bounds a wave's start). The RMSNorm prologue keeps the
  // weights first.
  const int per_row = K / 8;
  const int nslots = NB * per_row;
  const int nt = static_cast<int>(blockDim.x);
  bool early = true;
  if constexpr (FUSED) early = fu.h == nullptr;
  u32x4 xv[4];
  auto x_round = [&](int base) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = base + k * nt;
      const int r = p / per_row, e = 8 * (p - r * per_row);
      xv[k] = u32x4{0u, 0u, 0u, 0u};
      if (p < nslots && r < batch) xv[k] = *reinterpret_cast<const u32x4*>(X + static_cast<size_t>(r) * K + e);
    }
  };
  auto x_store = [&](int base) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = base + k * nt;
      if (p < nslots) {
        const int r = p / per_row, e = 8 * (p - r * per_row);
        char* dst = xs + r * xrow + m4_xoff(e);
        *reinterpret_cast<u32x2*>(dst) = u32x2{xv[k].x, xv[k].y};
        *reinterpret_cast<u32x2*>(dst + 8) = u32x2{xv[k].z, xv[k].w};
      }
    }
  };
  if (early) x_round(tid);
  issue(w0, s0);
  if constexpr (kDepth == 3) issue(w1, s1);
  {
    bool staged = false;
    if constexpr (FUSED) {
      if (fu.h != nullptr) {
        // RMSNorm prologue: x = bf16(h * rms factor * g)
        block_rms_factors<NB>(fu, K, batch, scr);
        for (int p = tid; p < nslots; p += nt) {
          const int r = p / per_row, e = 8 * (p - r * per_row);
          u32x4 v = {0u, 0u, 0u, 0u};
          if (r < batch) {
            const float* hr = fu.h + static_cast<size_t>(r) * K + e;
            const f32x4 h0 = *reinterpret_cast<const f32x4*>(hr);
            const f32x4 h1 = *reinterpret_cast<const f32x4*>(hr + 4);
            const u32x4 gg = *reinterpret_cast<const u32x4*>(fu.g + e);
            const float f = scr[kNormFactorOff + r];
            v = u32x4{pack_bf16(h0.x * f * bf16_lo(gg.x), h0.y * f * bf16_hi(gg.x)),
                      pack_bf16(h0.z * f * bf16_lo(gg.y), h0.w * f * bf16_hi(gg.y)),
                      pack_bf16(h1.x * f * bf16_lo(gg.z), h1.y * f * bf16_hi(gg.z)),
                      pack_bf16(h1.z * f * bf16_lo(gg.w), h1.w * f * bf16_hi(gg.w))};
          }
          char* dst = xs + r * xrow + m4_xoff(e);
          *reinterpret_cast<u32x2*>(dst) = u32x2{v.x, v.y};
          *reinterpret_cast<u32x2*>(dst + 8) = u32x2{v.z, v.w};
        }
        staged = true;
      }
    }
    if (!staged) {
      x_store(tid);
      for (int base = tid + 4 * nt; base < nslots; base += 4 * nt) {
        x_round(base);
        x_store(base);
      }
    }
  }
  __syncthreads();
  if constexpr (F::kBias) {
    // -8 * (sum of x over each unit), per batch row
    constexpr uint32_t kOnes = 0x3f803f80u;
    for (int e = tid; e < nunits * NB; e += blockDim.x) {
      const int u = e / NB, r = e - u * NB;
      float sum = 0.f;
#pragma unroll
      for (int sub = 0; sub < F::kSub; ++sub) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(xs + r * xrow + m4_xoff(m4_elem<FMT>(u, sub)));
        sum = dot2(v.x, kOnes, sum);
        sum = dot2(v.y, kOnes, sum);
      }
      sneg[e] = -8.f * sum;
    }
    __syncthreads();
  }

  if constexpr (kDepth == 3) {
    for (int v = va; v < vb; v += 3) {
      issue(w2, s2);
      step(w0, s0);
      if (v + 1 >= vb) break;
      issue(w0, s0);
      step(w1, s1);
      if (v + 2 >= vb) break;
      issue(w1, s1);
      step(w2, s2);
    }
  } else {
    for (int v = va; v < vb; v += 2) {
      issue(w1, s1);
      step(w0, s0);
      if (v + 1 >= vb) break;
      issue(w0, s0);
      step(w1, s1);
    }
  }

  // ---- tiles split between waves: the wave holding a tile's last step adds
  // the partial results of every wave holding part of it, in wave order
  __syncthreads();
  const int rel = va / nst;                            // the wave's first tile, relative to t0
  if (va < vb && va != rel * nst && (rel + 1) * nst <= vb) {
    int wf = wave - 1;                                 // the wave holding the tile's first step
    while (static_cast<int>(static_cast<long>(wf) * nflat / nw) > rel * nst) --wf;
    f32x4 sum = zero;
    if (((lane >> 2) & 3) == 0) {
      for (int w = wf; w <= wave; ++w) {
        const int a2 = static_cast<int>(static_cast<long>(w) * nflat / nw);
        const int b2 = static_cast<int>(static_cast<long>(w + 1) * nflat / nw);
        if (a2 == b2) continue;                        // a wave with no steps
        const f32x4 o = part[(w * 2 + (a2 / nst == rel ? 0 : 1)) * 16 + pslot];
#pragma unroll
        for (int n = 0; n < 4; ++n) sum[n] += o[n];
      }
    }
    store(sum, t0 + rel);
  }

  if constexpr (AM) {
    // ---- argmax of the entry's output: the workgroup's largest key per
    // batch row (waves, then through LDS) goes to its own word of the
    // caller's workspace (a relaxed device-scope store; key 1 never wins);
    // workgroup 0 of the launch takes the largest of the words
    // (mfma_argmax_collect). (A counter that let the last workgroup finish
    // the argmax made every workgroup queue on one address at the end.)
    if (!am_on) return;                                // (uniform over the workgroup)
    uint64_t* wk = reinterpret_cast<uint64_t*>(xs);    // x is no longer read
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint64_t k = wave_umax64(vlo == (b & 3) ? amk[b >> 2] : uint64_t{0});
      if (lane == 0) wk[wave * NB + b] = k;
    }
    __syncthreads();
    if (tid < NB && tid < batch) {
      uint64_t k = 0;
      for (int w = 0; w < nw; ++w) k = umax64(k, wk[w * NB + tid]);
      __hip_atomic_store(amx.slots + static_cast<size_t>(tid) * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW + amx.wg,
                         umax64(k, 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// qgemv_run_fused at batch <= 2 with short rows: one GEMV of one (R, NCH)
// with the RMSNorm prologue and the epilogue of fu, and with AM the argmax
// of its output fused in as in the grouped launch (one kernel per shape, so
// each shape gets its own register budget). With the prologue, the
// workgroup first normalizes x once into LDS (dynamic LDS: NB * K bf16 +
// kNormScratchBytes) and its waves read their x registers from there: done
// per wave, every wave would read all of h and g again.
template <int FMT, int NB, int R, int NCH, bool AM>
__global__ __launch_bounds__(kThreads) void gemv_xreg_fused_kernel(const GemvTable<1> tab, int batch,
                                                                   uint64_t* __restrict__ slots,
                                                                   int32_t* __restrict__ idx,
                                                                   const Fusion fu) {
  extern __shared__ u32x4 lds_v4[];
  __shared__ uint64_t red[kWaves];
  if constexpr (AM) {
    if (blockIdx.x == 0) {                      // the collector (see fused_argmax_tail)
      fused_argmax_tail<4>(slots, batch, idx, red);
      return;
    }
  }
  // (with the prologue, every wave runs xreg_run, which normalizes x into
  // LDS with the whole workgroup after issuing its first weight loads)
  uint32_t* xn = fu.h != nullptr ? reinterpret_cast<uint32_t*>(lds_v4) : nullptr;
  int stride;
  int item = first_item<AM ? 1 : 0>(stride);
  const int lane = threadIdx.x & 63;
  AmLane am;
  if (xn != nullptr || item < tab.total) {
    int j = 0;
    xreg_run<FMT, NB, R, NCH, 1, AM, true>(tab, j, item, stride, batch, lane, am, slots, fu, xn);
  }
  if constexpr (AM) {
    if (!am.left) am_leave<NB>(am, slots, batch, lane);
  }
}


// The LDS dot2 kernel: x for all batch rows staged once per workgroup in
// LDS, then the dot2 streaming loop over row groups of R rows. FUSED: the
// operations of fu fused in (prologue in the staging, epilogue in the
// store); the LDS then ends with kNormScratchBytes of scratch.
template <int FMT, int NB, int R, bool FUSED = false>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ S,
    const uint16_t* __restrict__ X, float* __restrict__ Y, int M, int K, int batch, const Fusion fu) {
  static_assert(!FUSED || R % 2 == 0, "gate/up pairs must share a row group");
  using T = Traits<FMT>;
  constexpr int UC = T::kUC;
  constexpr int P = T::kPairs;
  extern __shared__ u32x4 lds_v4[];
  uint32_t* lds = reinterpret_cast<uint32_t*>(lds_v4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int KD = K >> 1;                              // x dwords per batch row
  const int U = K / T::kElems;                        // 16-byte units per row
  const size_t row_bytes = static_cast<size_t>(U) * 16;
  const int nsc = scales_per_row<FMT>(U);
  const int groups = (M + R - 1) / R;
  const int waves_total = gridDim.x * kWaves;
  const int nchunk = (U + 64 * UC - 1) / (64 * UC);

  uint32_t* xs = lds;                                        // [NB][KD]
  float* sxs = reinterpret_cast<float*>(lds + NB * KD);      // [NB][U] (4-bit only)

  u32x4 wv[R][UC];
  uint32_t sv[R][UC];   // binary16 scale bits, one per 32-bit register

  // Issue the loads of one step (R rows x UC units per lane), branch-free:
  // lanes past the end of a ragged row re-load the row's last unit (an
  // in-bounds address on a line the wave reads anyway) and skip it when
  // computing; rows past M re-load row M-1 and are not stored.
  auto load_step = [&](int grp, int ch) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(grp * R + r, M - 1);
      const u32x4* wrow = reinterpret_cast<const u32x4*>(W + static_cast<size_t>(row) * row_bytes);
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int t = min(ch * 64 * UC + u * 64 + lane, U - 1);
        wv[r][u] = load_weights(wrow + t);
        if constexpr (T::kUnitsPerScale != 0)
          sv[r][u] = S[static_cast<size_t>(row) * nsc + scale_index<FMT>(t)];
      }
    }
  };

  // ---- stage x. The first chunks are loaded before this wave's first
  // weight loads are issued, so waiting for them does not wait for weights.
  constexpr int kXPre = 4;
  const int row_chunks = K / 8;                      // 16-byte chunks per x row
  const int nxc = NB * row_chunks;                   // chunks staged (NB rows)
  const int valid_xc = batch * row_chunks;           // chunks that exist in X
  bool norm = false;
  if constexpr (FUSED) norm = fu.h != nullptr;
  u32x4 xpre[kXPre];
  if (!norm) {
#pragma unroll
    for (int j = 0; j < kXPre; ++j) {
      const int i = tid + j * kThreads;
      xpre[j] = reinterpret_cast<const u32x4*>(X)[min(i, valid_xc - 1)];
    }
  }

  int grp = blockIdx.x * kWaves + wave;
  int ch = 0;
  load_step(min(grp, groups - 1), 0);

  if (!norm) {
#pragma unroll
    for (int j = 0; j < kXPre; ++j) {
      const int i = tid + j * kThreads;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      if (i < nxc) reinterpret_cast<u32x4*>(xs)[i] = (i < valid_xc) ? xpre[j] : zero;
    }
    for (int i = tid + kXPre * kThreads; i < nxc; i += kThreads) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const u32x4 v = reinterpret_cast<const u32x4*>(X)[min(i, valid_xc - 1)];
      reinterpret_cast<u32x4*>(xs)[i] = (i < valid_xc) ? v : zero;
    }
  } else {
    // RMSNorm prologue: x = bf16(h * r * g)
    stage_norm_rows<NB>(fu, K, batch, xs, reinterpret_cast<float*>(lds + NB * KD + (T::kBias ? NB * U : 0)));
  }
  __syncthreads();

  if constexpr (T::kBias) {
    // per-unit sums of x, pre-multiplied by -8 (the dot chain's start value)
    constexpr uint32_t kOnes = 0x3f803f80u;          // bf16 pair (1.0, 1.0)
    for (int i = tid; i < NB * U; i += kThreads) {
      const int b = i / U, t = i - b * U;
      uint32_t xv[P];
      read_x<FMT>(xs + b * KD, t, xv);
      float s = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) s = dot2(xv[p], kOnes, s);
      sxs[i] = -8.f * s;
    }
    __syncthreads();
  }

  float acc[R][NB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  while (grp < groups) {
    // compute the step whose loads are in flight
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int t = ch * 64 * UC + u * 64 + lane;
      if (t < U) {
        uint32_t pr[R][P];
        float dsc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          unpack<FMT>(wv[r][u], pr[r]);
          dsc[r] = unit_scale<FMT>(sv[r][u]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          uint32_t xv[P];
          read_x<FMT>(xs + b * KD, t, xv);
          const float init = T::kBias ? sxs[b * U + t] : 0.f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if constexpr (FMT == QGEMV_BF16) {
              float a = acc[r][b];
#pragma unroll
              for (int p = 0; p < P; ++p) a = dot2(pr[r][p], xv[p], a);
              acc[r][b] = a;
            } else {
              float a = init;
#pragma unroll
              for (int p = 0; p < P; ++p) a = dot2(pr[r][p], xv[p], a);
              acc[r][b] = __builtin_fmaf(dsc[r], a, acc[r][b]);
            }
          }
        }
      }
    }

    const int cur = grp;
    if (++ch == nchunk) { ch = 0; grp += waves_total; }
    if (grp < groups) load_step(grp, ch);

    if (ch == 0) {
      constexpr int V = R * NB;
      float v[V];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) { v[r * NB + b] = acc[r][b]; acc[r][b] = 0.f; }
      const float res = reduce_wave<V>(v, lane);
      constexpr int SH = 6 - ilog2(V);
      // every lane of a 2^SH-lane segment holds the segment's value; the
      // paired row of a gate/up pair (index + NB) is NB segments further
      float partner = 0.f;
      if constexpr (FUSED) {
        if (fu.epi == kEpiSwiglu) partner = __shfl_xor(res, NB << SH);
      }
      if ((lane & ((1 << SH) - 1)) == 0) {
        const int idx = lane >> SH;
        const int r = idx / NB, b = idx % NB;
        const int row = cur * R + r;
        if (row < M && b < batch) {
          if constexpr (FUSED) epi_store(fu, Y, M, b, row, res, partner);
          else Y[static_cast<size_t>(b) * M + row] = res;
        }
      }
    }
  }
}

// A table of GEMVs of one format, K and batch. Workgroup w takes the
// contiguous units [w*units/G, (w+1)*units/G), entry by entry (x is staged
// again when the entry changes), so most workgroups stage x once.
// The matrix-core launch: workgroup b belongs to the entry whose
// [wg0, wg0 + nwg) holds b and takes the b-th of its nwg balanced tile ranges.
// AM: workgroup 0 collects the argmax keys of entry tab.am (into am_idx),
// the workers are workgroups 1.. (b = blockIdx.x - 1).
template <int FMT, int NB, int N, bool FUSED = false, bool AM = false>
__global__ __launch_bounds__(kMfmaMaxThreads) void gemv_mfma_kernel(const MfmaTable<N> tab, int batch,
                                                                    const Fusion fu, uint64_t* am_slots,
                                                                    int32_t* am_idx) {
  extern __shared__ u32x4 lds_v4[];
  if constexpr (AM) {
    if (blockIdx.x == 0) {
      mfma_argmax_collect<NB>(am_slots, tab.e[tab.am].nwg, batch, am_idx, reinterpret_cast<uint64_t*>(lds_v4));
      return;
    }
  }
  const int b = static_cast<int>(blockIdx.x) - (AM ? 1 : 0);
  int j = 0;
  if constexpr (N > 1) j = find_entry(tab, b, [](const MfmaEntry& e) { return e.wg0; });
  const MfmaEntry& ent = tab.e[j];
  const long tiles = (ent.M + kMfmaTileRows<NB> - 1) / kMfmaTileRows<NB>;
  const int r = b - ent.wg0;
  const int t0 = static_cast<int>(r * tiles / ent.nwg);
  const int t1 = static_cast<int>((r + 1) * tiles / ent.nwg);
  MfmaArgmax amx;
  if (AM && j == tab.am) {
    amx.slots = am_slots;
    amx.wg = r;
  }
  mfma_tiles<FMT, NB, FUSED, AM>(ent, t0, t1, batch, lds_v4, fu, amx);
}

int round_batch(int batch) { return batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8; }

template <int FMT, int NB>
hipError_t launch_fr(const GemvArgs& a, int R, int grid, size_t lds, hipStream_t st) {
  const uint8_t* W = static_cast<const uint8_t*>(a.W);
  switch (R) {
    case 1: gemv_kernel<FMT, NB, 1><<<grid, kThreads, lds, st>>>(W, a.scales, a.x, a.y, a.M, a.K, a.batch, Fusion{}); break;
    case 2: gemv_kernel<FMT, NB, 2><<<grid, kThreads, lds, st>>>(W, a.scales, a.x, a.y, a.M, a.K, a.batch, Fusion{}); break;
    default: gemv_kernel<FMT, NB, 4><<<grid, kThreads, lds, st>>>(W, a.scales, a.x, a.y, a.M, a.K, a.batch, Fusion{}); break;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_f(const GemvArgs& a, int R, int grid, size_t lds, hipStream_t st, int nb) {
  switch (nb) {
    case 1: return launch_fr<FMT, 1>(a, R, grid, lds, st);
    case 2: return launch_fr<FMT, 2>(a, R, grid, lds, st);
    case 4: return launch_fr<FMT, 4>(a, R, grid, lds, st);
    default: return launch_fr<FMT, 8>(a, R, grid, lds, st);
  }
}

template <int FMT, int NB, int R, bool FUSED = false>
void allow_big_lds() {
  // (a failure here shows up as the error of the launch that needs it)
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<FMT, NB, R, FUSED>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

// Workgroups of kThreads threads of `kernel` resident per CU (at least 1).
int resident_per_cu(const void* kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

template <int FMT, int NB, int R, int NCH>
hipError_t launch_xreg3(const GemvArgs& a, int grid, hipStream_t st) {
  GemvTable<1> tab{};
  tab.n = 1;
  tab.total = (a.M + R - 1) / R;
  tab.e[0] = TableEntry{static_cast<const uint8_t*>(a.W), a.scales, a.x, a.y, a.M, a.K, 0,
                        xreg_shape(R, NCH)};
  static const int per_cu = resident_per_cu(reinterpret_cast<const void*>(&gemv_xreg_kernel<FMT, NB, R, NCH>));
  grid = std::min(grid, device_cu_count() * per_cu);     // one resident round (see launch_group2)
  gemv_xreg_kernel<FMT, NB, R, NCH><<<grid, kThreads, 0, st>>>(tab, a.batch);
  return hipGetLastError();
}

template <int FMT, int NB, int NCH>
hipError_t launch_xreg2(const GemvArgs& a, int R, int grid, hipStream_t st) {
  switch (R) {
    case 1: return launch_xreg3<FMT, NB, 1, NCH>(a, grid, st);
    case 2: return launch_xreg3<FMT, NB, 2, NCH>(a, grid, st);
    default: return launch_xreg3<FMT, NB, 4, NCH>(a, grid, st);
  }
}

template <int FMT, int NB>
hipError_t launch_xreg1(const GemvArgs& a, int R, int nch, int grid, hipStream_t st) {
  switch (nch) {
    case 1: return launch_xreg2<FMT, NB, 1>(a, R, grid, st);
    case 2: return launch_xreg2<FMT, NB, 2>(a, R, grid, st);
    case 3: return launch_xreg2<FMT, NB, 3>(a, R, grid, st);
    case 4: return launch_xreg2<FMT, NB, 4>(a, R, grid, st);
    default:
      if constexpr (is_int8_fmt(FMT) && NB == 1) return launch_xreg3<FMT, NB, 1, 8>(a, grid, st);
      else return hipErrorInvalidValue;          // (not produced by the host)
  }
}

template <int FMT>
hipError_t launch_xreg(const GemvArgs& a, int R, int nch, int grid, hipStream_t st) {
  if (round_batch(a.batch) == 1) return launch_xreg1<FMT, 1>(a, R, nch, grid, st);
  return launch_xreg1<FMT, 2>(a, R, nch, grid, st);
}

constexpr int kGroupMax = 64;       // GEMVs per grouped launch (kernel-argument table)
static_assert(kGroupMax <= 64, "find_entry reads one entry per lane");

// Entries of one format and batch with their (R, NCH) already chosen; am >= 0:
// also the argmax of entry am's output (into idx, through slots).
template <int FMT, int NB>
hipError_t launch_group2(const GemvArgs* a, const int* R_in, const int* nch, int n, int grid, int am,
                         uint64_t* slots, int32_t* idx, hipStream_t st) {
  GemvTable<kGroupMax> tab{};
  tab.n = n;
  // the argmax entry goes first, so its keys are complete while the other
  // entries still stream (the rest in the given order: with row groups
  // strided over the waves, sorting them by row-group size, or the long
  // rows right after the argmax entry, measured slower)
  int order[kGroupMax];
  for (int t = 0; t < n; ++t) order[t] = am < 0 ? t : t == 0 ? am : (t <= am ? t - 1 : t);
  int R[kGroupMax];
  for (int i = 0; i < n; ++i) R[i] = R_in[i];
  auto build = [&]() {
    tab.am = -1;
    int start = 0;
    for (int t = 0; t < n; ++t) {
      const int i = order[t];
      if (i == am) tab.am = t;
      tab.e[t] = TableEntry{static_cast<const uint8_t*>(a[i].W), a[i].scales, a[i].x, a[i].y,
                            a[i].M, a[i].K, start, xreg_shape(R[i], nch[i])};
      start += (a[i].M + R[i] - 1) / R[i];
    }
    tab.total = start;
    for (int t = n; t < kGroupMax; ++t) tab.e[t].start = INT_MAX;   // never a wave's entry
  };
  build();
  // The grid is at most what is resident at once (workgroups per CU from the
  // kernel's register budget): a second, partial round of workgroups would
  // restart row groups' x loads and leave most CUs idle at its end
  // (measured: 15.1 vs 17.3 us for the TinyLlama set at 3 resident
  // workgroups per CU against a grid of 8 per CU).
  const int cus = device_cu_count();
  static const int per_cu_am = resident_per_cu(reinterpret_cast<const void*>(
      &gemv_xreg_group_kernel<FMT, NB, kGroupMax, true>));
  static const int per_cu = resident_per_cu(reinterpret_cast<const void*>(
      &gemv_xreg_group_kernel<FMT, NB, kGroupMax, false>));
  // (with the argmax: workers plus the collector, workgroup 0, all resident
  // at once, since the collector waits for every worker's key)
  const int workers = am >= 0 ? std::max(1, std::min({grid, cus * per_cu_am - 1, kFusedMaxWorkers}))
                              : std::min(grid, cus * per_cu);
  tab.contig = tab.total >= QGEMV_GROUP_CONTIG_MIN * workers * kWaves;
  if (tab.contig) {
    // contiguous ranges: the entries of long rows (more than one unit per
    // lane-column) together, after the argmax entry and before the others,
    // so that fewer waves' ranges cross from one shape to another (each
    // crossing drains the wave's loads; 89-GEMV decode step at batch 1:
    // 105 against 108 us with the layers' GEMVs in layer order)
    int m = 0;
    if (am >= 0) order[m++] = am;
    for (int i = 0; i < n; ++i)
      if (i != am && nch[i] > 1) order[m++] = i;
    for (int i = 0; i < n; ++i)
      if (i != am && nch[i] == 1) order[m++] = i;
    build();
  }
  if (tab.contig && NB == 1) {
    // contiguous ranges: the short rows eight at a time (more bytes in
    // flight per wave; the tail balance that favours four is moot here)
    bool any = false;
    for (int i = 0; i < n; ++i)
      if (nch[i] == 1 && R[i] == 4) { R[i] = 8; any = true; }
    if (any) {
      build();
      if (tab.total < QGEMV_GROUP_CONTIG_MIN * workers * kWaves) {
        // (too few row groups per wave at eight rows: keep four)
        for (int i = 0; i < n; ++i) R[i] = R_in[i];
        build();
      }
    }
  }
  if (am >= 0) {
    gemv_xreg_group_kernel<FMT, NB, kGroupMax, true><<<workers + 1, kThreads, 0, st>>>(tab, a[0].batch, slots, idx);
  } else {
    gemv_xreg_group_kernel<FMT, NB, kGroupMax, false><<<workers, kThreads, 0, st>>>(tab, a[0].batch, nullptr, nullptr);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_group1(const GemvArgs* a, const int* R, const int* nch, int n, int grid, int am,
                         uint64_t* slots, int32_t* idx, hipStream_t st) {
  if (round_batch(a[0].batch) == 1) return launch_group2<FMT, 1>(a, R, nch, n, grid, am, slots, idx, st);
  return launch_group2<FMT, 2>(a, R, nch, n, grid, am, slots, idx, st);
}

// ---- matrix-core kernel: launch plan
int mfma_step_elems(int fmt) {
  return with_fmt(fmt, [](auto F) { return M4<decltype(F)::value>::kStepElems; });
}

// LDS of one workgroup: partial tiles of `waves` waves, x of NB rows in the
// padded layout, and the 4-bit formats' unit sums (extra: the fused
// prologue's scratch)
size_t mfma_lds_bytes(int fmt, int K, int NB, int waves, size_t extra) {
  return with_fmt(fmt, [&](auto F) {
    constexpr int FMT = decltype(F)::value;
    size_t b = static_cast<size_t>(waves) * 2 * 16 * 16 + extra;
    b += static_cast<size_t>(NB) * m4_xrow<FMT>(K);
    if (M4<FMT>::kBias) b += static_cast<size_t>(K / M4<FMT>::kUnitElems) * NB * 4;
    return b;
  });
}

constexpr size_t kLdsPerCu = 160 * 1024;

// Whether the matrix-core kernel takes (fmt, K) at this batch: batch 3..8, K a
// multiple of one step, x of the compiled batch rows in LDS.
bool mfma_fits(int fmt, int K, int batch, size_t extra) {
  const int NB = round_batch(batch);
  if (NB < 4) return false;
  const int step = mfma_step_elems(fmt);
  return K % step == 0 && K / step >= 1 && mfma_lds_bytes(fmt, K, NB, 16, extra) <= kLdsPerCu;
}

struct MfmaPlan {
  int grid = 0;
  int waves = 16;
  size_t lds = 0;
};

// Launch shape and workgroups per entry. Workgroups of 8 waves, two per CU,
// where two fit in LDS (a workgroup's x staging and start-up then overlap
// the other's streaming), else 16 waves, one per CU; one round of
// workgroups, so that no CU waits for a second round. Every entry gets one
// workgroup, the rest go one at a time to the entry with the most (tile,
// step) pairs per workgroup, never more than one per tile. Depends on (fmt,
// M, K) of the entries and the CU count only, not on the batch.
MfmaPlan plan_mfma(const GemvArgs* a, int n, int cus, int nb, size_t extra, int reserve, int* nwg) {
  const int step = mfma_step_elems(a[0].fmt);
  const int tr = nb == 8 ? kMfmaTileRows<8> : kMfmaTileRows<4>;
  long total = 0, tiles_all = 0;
  int kmax = 0;
  long pairs[kGroupMax], tiles[kGroupMax];
  for (int e = 0; e < n; ++e) {
    tiles[e] = (a[e].M + tr - 1) / tr;
    pairs[e] = tiles[e] * (a[e].K / step);
    total += pairs[e];
    tiles_all += tiles[e];
    kmax = std::max(kmax, a[e].K);
  }
  MfmaPlan p;
  p.waves = 8;
  p.lds = mfma_lds_bytes(a[0].fmt, kmax, nb, 8, extra);
  int per_cu = 2;
  if (2 * p.lds > kLdsPerCu) {
    p.waves = 16;
    p.lds = mfma_lds_bytes(a[0].fmt, kmax, nb, 16, extra);
    per_cu = 1;
  }
  // (reserve: workgroups kept free for the argmax collector; at most
  // kMaxArgmaxKeyWords workgroups, as many as the collector has threads)
  const long target = std::max<long>(
      std::min<long>({static_cast<long>(cus) * per_cu - reserve, tiles_all, static_cast<long>(kMaxArgmaxKeyWords)}),
      n);
  // a proportional start (every entry at least one, at most one per tile),
  // then the remainder one at a time
  long grid = 0;
  for (int e = 0; e < n; ++e) {
    nwg[e] = static_cast<int>(std::max<long>(1, std::min(tiles[e], target * pairs[e] / std::max<long>(total, 1))));
    grid += nwg[e];
  }
  while (grid < target) {
    int best = -1;
    for (int e = 0; e < n; ++e) {
      if (nwg[e] >= tiles[e]) continue;
      // the entry whose workgroups have the most pairs each (compared exactly)
      if (best < 0 || pairs[e] * nwg[best] > pairs[best] * nwg[e]) best = e;
    }
    if (best < 0) break;
    ++nwg[best];
    ++grid;
  }
  p.grid = static_cast<int>(grid);
  return p;
}

// n GEMVs of one format and batch on the matrix cores (one entry for
// qgemv_run), NB batch rows compiled; am >= 0: also the argmax of entry am's
// output into idx (slots: zero on entry, zero on exit).
template <int FMT, int NB, int N, bool FUSED = false, bool AM = false>
hipError_t launch_mfma_table(const GemvArgs* a, int n, hipStream_t st, const Fusion& fu = Fusion{},
                             int am = -1, uint64_t* slots = nullptr, int32_t* idx = nullptr) {
  MfmaTable<N> tab{};
  // the argmax entry first: its workgroups are dispatched first and finish
  // before most others, so the collector's wait overlaps their streaming
  // (last, it held the launch open about 3 us at batch 8)
  GemvArgs o[N];
  for (int t = 0; t < n; ++t) o[t] = a[am < 0 ? t : t == 0 ? am : (t <= am ? t - 1 : t)];
  int nwg[N];
  const MfmaPlan p = plan_mfma(o, n, device_cu_count(), NB, FUSED ? kNormScratchBytes : 0, AM ? 1 : 0, nwg);
  tab.n = n;
  tab.am = am < 0 ? -1 : 0;
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    tab.e[i] = MfmaEntry{static_cast<const uint8_t*>(o[i].W), o[i].scales, o[i].x, o[i].y,
                         o[i].M, o[i].K, wg, nwg[i]};
    wg += nwg[i];
  }
  if (p.lds > 64 * 1024) {
    static const hipError_t once = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemv_mfma_kernel<FMT, NB, N, FUSED, AM>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsPerCu));
    if (once != hipSuccess) return once;
  }
  // (with the argmax, workgroup 0 collects the keys: the workers get one
  // workgroup fewer, so that all of them and the collector are resident)
  gemv_mfma_kernel<FMT, NB, N, FUSED, AM><<<p.grid + (AM ? 1 : 0), 64 * p.waves, p.lds, st>>>(
      tab, a[0].batch, fu, slots, idx);
  return hipGetLastError();
}

// nb: batch rows the kernel is compiled for (4 or 8; >= batch)
template <int FMT, int N>
hipError_t launch_mfma(const GemvArgs* a, int n, hipStream_t st, int nb, int am, uint64_t* slots, int32_t* idx) {
  if (am >= 0) {
    if (nb == 4) return launch_mfma_table<FMT, 4, N, false, true>(a, n, st, Fusion{}, am, slots, idx);
    return launch_mfma_table<FMT, 8, N, false, true>(a, n, st, Fusion{}, am, slots, idx);
  }
  if (nb == 4) return launch_mfma_table<FMT, 4, N>(a, n, st);
  return launch_mfma_table<FMT, 8, N>(a, n, st);
}

template <int N>
hipError_t launch_mfma_fmt(const GemvArgs* a, int n, hipStream_t st, int nb, int am = -1,
                           uint64_t* slots = nullptr, int32_t* idx = nullptr) {
  return with_fmt(a[0].fmt, [&](auto F) { return launch_mfma<decltype(F)::value, N>(a, n, st, nb, am, slots, idx); });
}
}  // namespace

FmtInfo fmt_info(int fmt) {
  switch (fmt) {
    case QGEMV_BF16: return {1, 8};
    case QGEMV_INT8_G32: return {32, 16};
    case QGEMV_Q4_0_G32: return {32, 32};
    case QGEMV_INT4_G128: return {128, 32};
    case QGEMV_INT8_ROW: return {0, 16};
    default: return {64, 32};
  }
}

size_t gemv_lds_bytes(int fmt, int K, int batch) {
  const int nb = round_batch(batch);             // (batch 8 for the invariant mode's size)
  size_t bytes = static_cast<size_t>(nb) * K * 2;
  if (fmt == QGEMV_Q4_0_G32 || fmt == QGEMV_INT4_G128 || fmt == QGEMV_INT4_G64)
    bytes += static_cast<size_t>(nb) * (K / 32) * 4;                  // -8 * sum(x) per 16-byte unit
  return bytes;
}

// Units per lane-column whose x a register-x kernel holds: 4, and 8 (taken
// as one shape, rows one at a time) for int8 at batch 1, where 8 units of x
// are 64 registers, as many as 4 units of a 4-bit format. The fused kernels,
// whose row groups hold a gate/up pair, stop at 4.
int xreg_max_units(int fmt, int batch, bool fused) {
  return !fused && (fmt == QGEMV_INT8_G32 || fmt == QGEMV_INT8_ROW) && round_batch(batch) == 1 ? 8 : 4;
}

int xreg_units(int fmt, int K) {
  const int U = K / fmt_info(fmt).elems_per_unit;
  const int nch = (U + 63) / 64;
  return nch <= 4 || nch > 8 ? nch : 8;
}

bool gemv_uses_lds(int fmt, int K, int batch, bool fused) {
  return !(round_batch(batch) <= 2 && xreg_units(fmt, K) <= xreg_max_units(fmt, batch, fused));
}

// A lone GEMV at batch 3..8 (qgemv_run) below these weight sizes runs faster
// on the dot2 LDS kernel than on the matrix-core kernel, whose start-up
// (x staging by every workgroup, the first steps' round trip, the stream-K
// finisher) costs more than it saves on a few MB. Measured per GEMV,
// graph-replayed, dot2 against matrix cores: at batch 4, Q4_0 2048x2048 4.3
// against 6.6 us, 11264x2048 7.8 / 9.6, int8 16384x2048 10.7 / 12.3, but
// 4-bit 2048x8192 10.5 / 9.9 and the 32000-row Q4_0 LM head 14.0 / 12.1; at
// batch 8, bf16 2048x2048 5.9 / 7.4, int8 3072x2048 6.3 / 8.8, but Q4_0
// 11264x2048 11.6 / 10.3 and Q4_0 2048x5632 16.9 / 11.4.
bool lone_prefers_lds(const GemvArgs& a) {
  const FmtInfo f = fmt_info(a.fmt);
  const double code = static_cast<double>(a.K) / f.elems_per_unit * 16;
  const double scale = f.group > 1 ? static_cast<double>(a.K) / f.group * 2 : (f.group == 0 ? 2 : 0);
  const double bytes = static_cast<double>(a.M) * (code + scale);
  const bool four_bit = f.elems_per_unit == 32;
  if (round_batch(a.batch) <= 4) return bytes <= 36e6 && !(four_bit && a.K > 6144);
  return bytes <= 9e6 && a.K <= 4096;
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream, int flags) {
  const int cus = device_cu_count();
  const int nch = xreg_units(a.fmt, a.K);
  // batch invariance: every batch runs the kernels compiled for 8 batch rows
  // with launch shapes chosen from (fmt, M, K) alone, so a row's arithmetic
  // is the same at every batch (the register-x kernel is never used: its
  // reduction tree depends on the batch)
  const bool inv = (flags & QGEMV_FLAG_BATCH_INVARIANT) != 0;
  const int nb = inv ? 8 : round_batch(a.batch);
  if (!inv && !gemv_uses_lds(a.fmt, a.K, a.batch)) {
    // rows per step: up to 8 / NCH units in flight per lane, while keeping
    // at least two workgroups per CU
    int R = std::min(QGEMV_XREG_MAX_R, nch <= 2 ? 4 : nch <= 4 ? 2 : 1);
    while (R > 1 && (a.M + R - 1) / R < QGEMV_MIN_WAVES_PER_CU * cus) R >>= 1;
    const int groups = (a.M + R - 1) / R;
    const int wg_needed = (groups + kWaves - 1) / kWaves;
    const int grid = std::max(1, std::min(wg_needed, cus * QGEMV_MAX_WG_PER_CU));
    return with_fmt(a.fmt, [&](auto F) { return launch_xreg<decltype(F)::value>(a, R, nch, grid, stream); });
  }
  if (mfma_fits(a.fmt, a.K, inv ? 8 : a.batch, 0) && (inv || !lone_prefers_lds(a)))
    return launch_mfma_fmt<1>(&a, 1, stream, nb);
  const size_t lds = gemv_lds_bytes(a.fmt, a.K, nb);
  // rows per wave step: as many as keep at least two workgroups per CU busy
  int R = 4;
  while (R > 1 && (a.M + R - 1) / R < QGEMV_MIN_WAVES_PER_CU * cus) R >>= 1;
  const int groups = (a.M + R - 1) / R;
  const int wg_needed = (groups + kWaves - 1) / kWaves;
  int wg_per_cu = static_cast<int>(std::min<size_t>(QGEMV_MAX_WG_PER_CU, (160 * 1024) / std::max<size_t>(lds, 1)));
  if (wg_per_cu < 1) wg_per_cu = 1;
  const int grid = std::max(1, std::min(wg_needed, cus * wg_per_cu));
  if (lds > 64 * 1024) {
    static bool once = [] {
#define QG_ALLOW(F) allow_big_lds<F, 8, 1>(); allow_big_lds<F, 8, 2>(); allow_big_lds<F, 8, 4>(); \
                    allow_big_lds<F, 4, 1>(); allow_big_lds<F, 4, 2>(); allow_big_lds<F, 4, 4>(); \
                    allow_big_lds<F, 2, 1>(); allow_big_lds<F, 2, 2>(); allow_big_lds<F, 2, 4>(); \
                    allow_big_lds<F, 1, 1>(); allow_big_lds<F, 1, 2>(); allow_big_lds<F, 1, 4>();
      QG_ALLOW(QGEMV_BF16) QG_ALLOW(QGEMV_INT8_G32) QG_ALLOW(QGEMV_Q4_0_G32) QG_ALLOW(QGEMV_INT4_G128)
      QG_ALLOW(QGEMV_INT8_ROW) QG_ALLOW(QGEMV_INT4_G64)
#undef QG_ALLOW
      return true;
    }();
    (void)once;
  }
  return with_fmt(a.fmt, [&](auto F) { return launch_f<decltype(F)::value>(a, R, grid, lds, stream, nb); });
}

int gemv_group_class(int fmt, int K, int batch) {
  if (gemv_uses_lds(fmt, K, batch)) return 0;
  return xreg_units(fmt, K);
}

int gemv_group_max() { return kGroupMax; }

bool gemv_mfma_groupable(int fmt, int K, int batch) { return mfma_fits(fmt, K, batch, 0); }

hipError_t launch_gemv_mfma_group(const GemvArgs* a, int n, hipStream_t stream, int am, uint64_t* slots,
                                  int32_t* idx) {
  return launch_mfma_fmt<kGroupMax>(a, n, stream, round_batch(a[0].batch), am, slots, idx);
}

hipError_t launch_gemv_group(const GemvArgs* a, int n, hipStream_t stream, int am, uint64_t* slots,
                             int32_t* idx) {
  const int cus = device_cu_count();
  long rows = 0;
  for (int i = 0; i < n; ++i) rows += a[i].M;
  // rows per wave step: for 1 unit per lane-column, 4 while that still gives
  // every CU's waves work, else 2; fewer for longer rows, which keep more x
  // and weights in registers (one kernel serves all entries, and its
  // register budget, hence its occupancy, is that of its largest shape)
  const bool r4 = rows / 4 >= static_cast<long>(QGEMV_MIN_WAVES_PER_CU) * cus;
  int R[kGroupMax], nch[kGroupMax];
  long total = 0;
  for (int i = 0; i < n; ++i) {
    nch[i] = gemv_group_class(a[i].fmt, a[i].K, a[i].batch);
    R[i] = nch[i] == 1 ? (r4 ? 4 : 2) : nch[i] == 2 ? QGEMV_GROUP_R2 : nch[i] <= 4 ? QGEMV_GROUP_RLONG : 1;
    total += (a[i].M + R[i] - 1) / R[i];
  }
  long cap = static_cast<long>(cus) * QGEMV_GROUP_MAX_WG_PER_CU;
  if (am >= 0 && cap > kFusedMaxWorkers) cap = kFusedMaxWorkers;   // one argmax slot per worker wave
  const int grid = static_cast<int>(std::max<long>(1, std::min<long>((total + kWaves - 1) / kWaves, cap)));
  return with_fmt(a[0].fmt, [&](auto F) {
    return launch_group1<decltype(F)::value>(a, R, nch, n, grid, am, slots, idx, stream);
  });
}

// ---- qgemv_run_fused: one GEMV with the RMSNorm prologue and an epilogue.
// Batch <= 2 with short rows: the register-x table kernel with one entry
// (rows per step >= 2, so the rows of a gate/up pair share a wave; the
// argmax fused in as in the grouped launch); otherwise the matrix-core or
// LDS dot2 kernel, followed by the argmax kernel when asked for.
template <int FMT, int NB, int R, int NCH>
hipError_t launch_fused_xreg(const GemvArgs& a, const Fusion& f, uint64_t* slots, int32_t* idx, hipStream_t st) {
  GemvTable<1> tab{};
  tab.n = 1;
  tab.am = idx ? 0 : -1;
  tab.total = (a.M + R - 1) / R;
  tab.e[0] = TableEntry{static_cast<const uint8_t*>(a.W), a.scales, a.x, a.y, a.M, a.K, 0, xreg_shape(R, NCH)};
  const int cus = device_cu_count();
  int grid = (tab.total + kWaves - 1) / kWaves;
  // LDS of the prologue (at most 2 rows x 8192 bf16 + scratch: under the
  // default 64 KiB), which can also bound the workgroups per CU
  const size_t lds = f.h ? static_cast<size_t>(NB) * a.K * 2 + kNormScratchBytes : 0;
  const int lds_cap = lds ? static_cast<int>((160 * 1024) / lds) : 1 << 20;
  if (idx) {
    static const int per_cu = resident_per_cu(reinterpret_cast<const void*>(
        &gemv_xreg_fused_kernel<FMT, NB, R, NCH, true>));
    // workers plus the collector (workgroup 0), all resident at once
    grid = std::max(1, std::min({grid, cus * std::min(per_cu, lds_cap) - 1, kFusedMaxWorkers})) + 1;
    gemv_xreg_fused_kernel<FMT, NB, R, NCH, true><<<grid, kThreads, lds, st>>>(tab, a.batch, slots, idx, f);
  } else {
    static const int per_cu = resident_per_cu(reinterpret_cast<const void*>(
        &gemv_xreg_fused_kernel<FMT, NB, R, NCH, false>));
    grid = std::max(1, std::min(grid, cus * std::min(per_cu, lds_cap)));
    gemv_xreg_fused_kernel<FMT, NB, R, NCH, false><<<grid, kThreads, lds, st>>>(tab, a.batch, nullptr, nullptr, f);
  }
  return hipGetLastError();
}

// rows per step: 4 at one unit per lane-column while every CU's waves still
// get work, else 2 (the rows of a gate/up pair must share a row group)
template <int FMT, int NB>
hipError_t launch_fused_xreg_shape(const GemvArgs& a, int nch, bool r4, const Fusion& f, uint64_t* slots,
                                   int32_t* idx, hipStream_t st) {
  switch (nch) {
    case 1: return r4 ? launch_fused_xreg<FMT, NB, 4, 1>(a, f, slots, idx, st)
                      : launch_fused_xreg<FMT, NB, 2, 1>(a, f, slots, idx, st);
    case 2: return launch_fused_xreg<FMT, NB, 2, 2>(a, f, slots, idx, st);
    case 3: return launch_fused_xreg<FMT, NB, 2, 3>(a, f, slots, idx, st);
    default: return launch_fused_xreg<FMT, NB, 2, 4>(a, f, slots, idx, st);
  }
}

template <int FMT>
hipError_t launch_fused_fmt(const GemvArgs& a, const Fusion& f, uint64_t* slots, int32_t* idx,
                            hipStream_t st) {
  const int cus = device_cu_count();
  const int nb = round_batch(a.batch);
  if (!gemv_uses_lds(FMT, a.K, a.batch, true)) {
    const int nch = xreg_units(FMT, a.K);
    const bool r4 = a.M / 4 >= QGEMV_MIN_WAVES_PER_CU * cus;
    if (nb == 1) return launch_fused_xreg_shape<FMT, 1>(a, nch, r4, f, slots, idx, st);
    return launch_fused_xreg_shape<FMT, 2>(a, nch, r4, f, slots, idx, st);
  }
  hipError_t e;
  if (mfma_fits(FMT, a.K, a.batch, kNormScratchBytes)) {
    if (idx) {
      // the argmax inside the launch, collected by its workgroup 0 (as in
      // the grouped launch; slots: zero on entry, zero on exit)
      return nb == 4 ? launch_mfma_table<FMT, 4, 1, true, true>(&a, 1, st, f, 0, slots, idx)
                     : launch_mfma_table<FMT, 8, 1, true, true>(&a, 1, st, f, 0, slots, idx);
    }
    e = nb == 4 ? launch_mfma_table<FMT, 4, 1, true>(&a, 1, st, f)
                : launch_mfma_table<FMT, 8, 1, true>(&a, 1, st, f);
  } else {
    const size_t lds = gemv_lds_bytes(FMT, a.K, a.batch) + kNormScratchBytes;
    int R = 4;
    while (R > 2 && (a.M + R - 1) / R < QGEMV_MIN_WAVES_PER_CU * cus) R >>= 1;
    const int groups = (a.M + R - 1) / R;
    const int wg_needed = (groups + kWaves - 1) / kWaves;
    const int wg_per_cu = std::max(1, static_cast<int>(std::min<size_t>(QGEMV_MAX_WG_PER_CU, (160 * 1024) / lds)));
    const int grid = std::max(1, std::min(wg_needed, cus * wg_per_cu));
    if (lds > 64 * 1024) {
      static bool once = [] {
        allow_big_lds<FMT, 1, 2, true>(); allow_big_lds<FMT, 1, 4, true>();
        allow_big_lds<FMT, 2, 2, true>(); allow_big_lds<FMT, 2, 4, true>();
        allow_big_lds<FMT, 4, 2, true>(); allow_big_lds<FMT, 4, 4, true>();
        allow_big_lds<FMT, 8, 2, true>(); allow_big_lds<FMT, 8, 4, true>();
        return true;
      }();
      (void)once;
    }
    const uint8_t* W = static_cast<const uint8_t*>(a.W);
#define QG_FUSED_LDS(NB_)                                                                          \
    if (R == 2)                                                                                    \
      gemv_kernel<FMT, NB_, 2, true><<<grid, kThreads, lds, st>>>(W, a.scales, a.x, a.y, a.M, a.K, a.batch, f); \
    else                                                                                           \
      gemv_kernel<FMT, NB_, 4, true><<<grid, kThreads, lds, st>>>(W, a.scales, a.x, a.y, a.M, a.K, a.batch, f);
    switch (nb) {
      case 1: QG_FUSED_LDS(1) break;
      case 2: QG_FUSED_LDS(2) break;
      case 4: QG_FUSED_LDS(4) break;
      default: QG_FUSED_LDS(8) break;
    }
#undef QG_FUSED_LDS
    e = hipGetLastError();
  }
  if (e == hipSuccess && idx) e = launch_argmax(a.y, a.M, a.batch, slots, idx, st);
  return e;
}

hipError_t launch_gemv_fused(const GemvArgs& a, const Fusion& f, uint64_t* slots, int32_t* idx,
                             hipStream_t stream) {
  return with_fmt(a.fmt, [&](auto F) { return launch_fused_fmt<decltype(F)::value>(a, f, slots, idx, stream); });
}

}  // namespace qgemv
