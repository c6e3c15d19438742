// C-ABI front end of libqgemv: argument validation, the host-side weight
// packer/quantizer, and dispatch to the HIP kernels.
//
// Every entry point validates everything it can on the host before touching
// HIP, and reports problems as negative status values (never exceptions).
#include <cmath>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "qgemv.h"
#include "qgemv_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = int64_t(1) << 31;

bool valid_fmt(int fmt) { return fmt >= QGEMV_BF16 && fmt <= QGEMV_INT4_G64; }

// K must be a multiple of this (the scale group; 32 for bf16 and int8-row)
int k_align(int fmt) {
  switch (fmt) {
    case QGEMV_INT4_G128: return 128;
    case QGEMV_INT4_G64: return 64;
    default: return 32;
  }
}

// weights per scale for a row of K (int8-row: the whole row; bf16: none)
int64_t group_of(int fmt, int64_t K) {
  switch (fmt) {
    case QGEMV_INT8_G32: case QGEMV_Q4_0_G32: return 32;
    case QGEMV_INT4_G128: return 128;
    case QGEMV_INT4_G64: return 64;
    case QGEMV_INT8_ROW: return K;
    default: return 0;
  }
}

bool is_int8(int fmt) { return fmt == QGEMV_INT8_G32 || fmt == QGEMV_INT8_ROW; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int fmt, int64_t M, int64_t K) {
  if (M < 1 || K < 1 || M >= kMaxDim || K >= kMaxDim) return QGEMV_ESHAPE;
  if (K % k_align(fmt) != 0) return QGEMV_ESHAPE;
  return QGEMV_OK;
}

void sizes(int fmt, int64_t M, int64_t K, size_t* w, size_t* s) {
  const size_t mk = static_cast<size_t>(M) * static_cast<size_t>(K);
  switch (fmt) {
    case QGEMV_BF16: *w = 2 * mk; *s = 0; break;
    case QGEMV_INT8_G32: *w = mk; *s = 2 * (mk / 32); break;
    case QGEMV_INT8_ROW: *w = mk; *s = 2 * static_cast<size_t>(M); break;
    case QGEMV_Q4_0_G32: *w = mk / 2; *s = 2 * (mk / 32); break;
    case QGEMV_INT4_G64: *w = mk / 2; *s = 2 * (mk / 64); break;
    default: *w = mk / 2; *s = 2 * (mk / 128); break;
  }
}

// ---------------------------------------------------------------- binary16
// Host conversions written from the IEEE 754 binary16 definition:
// 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.

double half_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double mag;
  if (e == 0) mag = std::ldexp(static_cast<double>(f), -24);
  else if (e == 31) mag = f ? NAN : INFINITY;
  else mag = std::ldexp(static_cast<double>(1024 + f), e - 25);
  return sign ? -mag : mag;
}

// double -> binary16, round to nearest with ties to even, overflow to inf.
// Works on the double's bit pattern: take the 53-bit significand and shift
// it right to the binary16 quantum of |v|'s binade (2^-24 below 2^-14),
// rounding the shifted-out bits to nearest-even.
uint16_t double_to_half(double v) {
  uint64_t b;
  std::memcpy(&b, &v, sizeof b);
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000);
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag > 0x7FF0000000000000ull) return 0x7E00;
  if (mag == 0x7FF0000000000000ull) return sign | 0x7C00;
  const int biased = static_cast<int>(mag >> 52);
  if (biased == 0) return sign;                      // double subnormal/zero -> 0
  int e = biased - 1023;                             // |v| = m * 2^(e-52)
  const uint64_t m = (mag & ((uint64_t(1) << 52) - 1)) | (uint64_t(1) << 52);
  const int shift = (e < -14) ? 28 - e : 42;         // keep quantum 2^-24 or 2^(e-10)
  uint64_t n;
  if (shift >= 64) {
    n = 0;
  } else {
    n = m >> shift;
    const uint64_t rem = m & ((uint64_t(1) << shift) - 1);
    const uint64_t half = uint64_t(1) << (shift - 1);
    if (rem > half || (rem == half && (n & 1))) ++n;
  }
  if (e < -14) return sign | static_cast<uint16_t>(n);   // n == 1024 is the smallest normal
  if (n == 2048) { n = 1024; ++e; }
  if (e > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (n - 1024));
}

double bf16_to_double(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// Quantize one group of G bf16 weights. Returns false on a range error.
// (G up to K for int8-row; v and q_out hold G values)
bool quantize_group(int fmt, const uint16_t* w, int64_t G, double* v, uint16_t* d_out, int* q_out) {
  for (int64_t j = 0; j < G; ++j) {
    v[j] = bf16_to_double(w[j]);
    if (!std::isfinite(v[j])) return false;
  }
  double d_exact;
  if (is_int8(fmt)) {
    double amax = 0.0;
    for (int64_t j = 0; j < G; ++j) amax = std::fmax(amax, std::fabs(v[j]));
    d_exact = amax / 127.0;
  } else {
    int64_t first = 0;
    for (int64_t j = 1; j < G; ++j)
      if (std::fabs(v[j]) > std::fabs(v[first])) first = j;   // strict: first of ties
    d_exact = v[first] / -8.0;
  }
  uint16_t dh = double_to_half(d_exact);
  if ((dh & 0x7FFF) == 0) dh = 0;                              // a zero scale is +0
  if ((dh & 0x7C00) == 0x7C00) return false;                   // overflow
  const double d = half_to_double(dh);
  *d_out = dh;
  for (int64_t j = 0; j < G; ++j) {
    if (is_int8(fmt)) {
      double q = (d == 0.0) ? 0.0 : std::nearbyint(v[j] / d);
      q = std::fmin(127.0, std::fmax(-127.0, q));
      q_out[j] = static_cast<int>(q);
    } else {
      double q = (d == 0.0) ? 8.0 : std::nearbyint(v[j] / d) + 8.0;
      q = std::fmin(15.0, std::fmax(0.0, q));
      q_out[j] = static_cast<int>(q);
    }
  }
  return true;
}

int pack_from_bf16(int fmt, const uint16_t* src, int64_t M, int64_t K, void* dst_w,
                   uint16_t* dst_s) {
  if (fmt == QGEMV_BF16) {
    std::memcpy(dst_w, src, static_cast<size_t>(M) * K * 2);
    return QGEMV_OK;
  }
  const int64_t G = group_of(fmt, K);
  const int64_t ng = K / G;
  std::vector<int> q(static_cast<size_t>(G));
  std::vector<double> v(static_cast<size_t>(G));
  // validate everything first so that nothing is written on error
  for (int64_t i = 0; i < M * K; ++i)
    if (!std::isfinite(bf16_to_double(src[i]))) return QGEMV_ERANGE;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t g = 0; g < ng; ++g) {
      uint16_t dh;
      if (!quantize_group(fmt, src + m * K + g * G, G, v.data(), &dh, q.data())) return QGEMV_ERANGE;
    }
  }
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t g = 0; g < ng; ++g) {
      uint16_t dh;
      quantize_group(fmt, src + m * K + g * G, G, v.data(), &dh, q.data());
      dst_s[m * ng + g] = dh;
      if (is_int8(fmt)) {
        int8_t* out = static_cast<int8_t*>(dst_w) + m * K + g * G;
        for (int64_t j = 0; j < G; ++j) out[j] = static_cast<int8_t>(q[j]);
      } else {
        uint8_t* out = static_cast<uint8_t*>(dst_w) + (m * ng + g) * (G / 2);
        for (int64_t j = 0; j < G / 2; ++j)
          out[j] = static_cast<uint8_t>(q[j] | (q[j + G / 2] << 4));
      }
    }
  }
  return QGEMV_OK;
}

int check_run_args(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, const float* y,
                   int64_t M, int64_t K, int batch) {
  if (!valid_fmt(fmt)) return QGEMV_EINVAL;
  if (!W || !x || !y) return QGEMV_EINVAL;
  if (fmt != QGEMV_BF16 && !scales) return QGEMV_EINVAL;
  int st = check_shape(fmt, M, K);
  if (st) return st;
  if (batch < 1 || batch > QGEMV_MAX_BATCH) return QGEMV_ESHAPE;
  if (qgemv::gemv_uses_lds(fmt, static_cast<int>(K), batch) &&
      qgemv::gemv_lds_bytes(fmt, static_cast<int>(K), batch) > 160 * 1024)
    return QGEMV_ESHAPE;
  if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 16)) return QGEMV_EALIGN;
  if (fmt != QGEMV_BF16 && !aligned(scales, 4)) return QGEMV_EALIGN;
  return QGEMV_OK;
}

int record_hip(hipError_t e) {
  if (e == hipSuccess) return QGEMV_OK;
  g_last_hip_error = static_cast<int>(e);
  return QGEMV_EHIP;
}

}  // namespace

namespace qgemv {

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace qgemv

extern "C" {

int qgemv_packed_size(int fmt, int64_t M, int64_t K, size_t* w_bytes, size_t* s_bytes) {
  if (!valid_fmt(fmt) || !w_bytes || !s_bytes) return QGEMV_EINVAL;
  const int st = check_shape(fmt, M, K);
  if (st) return st;
  sizes(fmt, M, K, w_bytes, s_bytes);
  return QGEMV_OK;
}

int qgemv_pack(int fmt, int src_kind, const void* src_w, const uint16_t* src_scales, int64_t M,
               int64_t K, void* dst_w, uint16_t* dst_scales) {
  if (!valid_fmt(fmt)) return QGEMV_EINVAL;
  if (src_kind != QGEMV_SRC_CANONICAL && src_kind != QGEMV_SRC_BF16) return QGEMV_EINVAL;
  if (!src_w || !dst_w) return QGEMV_EINVAL;
  const bool quantized = fmt != QGEMV_BF16;
  if (quantized && !dst_scales) return QGEMV_EINVAL;
  if (quantized && src_kind == QGEMV_SRC_CANONICAL && !src_scales) return QGEMV_EINVAL;
  const int st = check_shape(fmt, M, K);
  if (st) return st;
  size_t wb, sb;
  sizes(fmt, M, K, &wb, &sb);
  if (src_kind == QGEMV_SRC_BF16)
    return pack_from_bf16(fmt, static_cast<const uint16_t*>(src_w), M, K, dst_w, dst_scales);
  std::memcpy(dst_w, src_w, wb);
  if (quantized) std::memcpy(dst_scales, src_scales, sb);
  return QGEMV_OK;
}

int qgemv_quantize(int fmt, const uint16_t* w, int64_t M, int64_t K, void* codes, uint16_t* scales,
                   int32_t* err, void* stream) {
  if (!valid_fmt(fmt) || fmt == QGEMV_BF16) return QGEMV_EINVAL;
  if (!w || !codes || !scales) return QGEMV_EINVAL;
  const int st = check_shape(fmt, M, K);
  if (st) return st;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || (err && !aligned(err, 4)))
    return QGEMV_EALIGN;
  return record_hip(qgemv::launch_quantize(fmt, w, M, K, codes, scales, err, static_cast<hipStream_t>(stream)));
}

int qgemv_run(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
              int64_t M, int64_t K, int batch, void* stream) {
  const int st = check_run_args(fmt, W, scales, x, y, M, K, batch);
  if (st) return st;
  qgemv::GemvArgs a{fmt, W, scales, x, y, static_cast<int>(M), static_cast<int>(K), batch};
  return record_hip(qgemv::launch_gemv(a, static_cast<hipStream_t>(stream)));
}

int qgemv_run_fused(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
                    int64_t M, int64_t K, int batch, const qgemv_fusion* f, void* stream) {
  if (!f) return QGEMV_EINVAL;
  const bool norm = f->norm_input != nullptr;
  const bool swiglu = f->swiglu_out != nullptr;
  const bool am = f->argmax_idx != nullptr;
  if (!valid_fmt(fmt) || !W || (fmt != QGEMV_BF16 && !scales)) return QGEMV_EINVAL;
  if (norm == (x != nullptr)) return QGEMV_EINVAL;            // exactly one input
  if (norm && (!f->norm_weight || !std::isfinite(f->norm_eps) || !(f->norm_eps >= 0.f))) return QGEMV_EINVAL;
  if (swiglu && (y || f->residual || am)) return QGEMV_EINVAL;
  if (!swiglu && !y) return QGEMV_EINVAL;
  if (am != (f->argmax_ws != nullptr)) return QGEMV_EINVAL;
  int st = check_shape(fmt, M, K);
  if (st) return st;
  if (batch < 1 || batch > QGEMV_MAX_BATCH) return QGEMV_ESHAPE;
  if (swiglu && (M % 2) != 0) return QGEMV_ESHAPE;
  if (qgemv::gemv_uses_lds(fmt, static_cast<int>(K), batch, true) &&
      qgemv::gemv_lds_bytes(fmt, static_cast<int>(K), batch) + qgemv::kNormScratchBytes > 160 * 1024)
    return QGEMV_ESHAPE;
  if (!aligned(W, 16) || (fmt != QGEMV_BF16 && !aligned(scales, 4))) return QGEMV_EALIGN;
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16))) return QGEMV_EALIGN;
  if (norm && (!aligned(f->norm_input, 16) || !aligned(f->norm_weight, 16))) return QGEMV_EALIGN;
  if (f->residual && !aligned(f->residual, 16)) return QGEMV_EALIGN;
  if (swiglu && !aligned(f->swiglu_out, 4)) return QGEMV_EALIGN;
  if (am && (!aligned(f->argmax_ws, 8) || !aligned(f->argmax_idx, 4))) return QGEMV_EALIGN;
  qgemv::Fusion fu;
  fu.h = f->norm_input;
  fu.g = f->norm_weight;
  fu.eps = f->norm_eps;
  fu.epi = swiglu ? qgemv::kEpiSwiglu : f->residual ? qgemv::kEpiResidual : qgemv::kEpiStore;
  fu.res = f->residual;
  fu.act = f->swiglu_out;
  qgemv::GemvArgs a{fmt, W, scales, x, y, static_cast<int>(M), static_cast<int>(K), batch};
  return record_hip(qgemv::launch_gemv_fused(a, fu, f->argmax_ws, f->argmax_idx, static_cast<hipStream_t>(stream)));
}

static int check_attention_shape(int batch, int n_q, int n_kv, int head_dim, int64_t max_ctx) {
  if (batch < 1 || n_kv < 1 || n_q < 1 || n_q % n_kv != 0) return QGEMV_ESHAPE;
  const int G = n_q / n_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return QGEMV_ESHAPE;
  if (head_dim != 64 && head_dim != 128) return QGEMV_ESHAPE;
  // (a block may address up to 64 positions past the context: keep the byte
  // offsets of those in 32 bits too)
  if (max_ctx < 1 || (max_ctx + 64) * head_dim * 2 >= (int64_t(1) << 32)) return QGEMV_ESHAPE;
  const qgemv::AttnPlan p = qgemv::attention_plan(batch, n_q, n_kv, head_dim, max_ctx);
  if (static_cast<int64_t>(batch) * n_kv * p.splits >= (int64_t(1) << 31)) return QGEMV_ESHAPE;
  return QGEMV_OK;
}

int qgemv_attention_workspace_size(int batch, int n_q, int n_kv, int head_dim, int64_t max_ctx,
                                   size_t* bytes) {
  if (!bytes) return QGEMV_EINVAL;
  const int st = check_attention_shape(batch, n_q, n_kv, head_dim, max_ctx);
  if (st) return st;
  const qgemv::AttnPlan p = qgemv::attention_plan(batch, n_q, n_kv, head_dim, max_ctx);
  *bytes = std::max<size_t>(256, p.part_bytes);         // (never zero: ws is always a real buffer)
  return QGEMV_OK;
}

int qgemv_attention_decode(const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* ctx_lens, float* out, int batch, int n_q, int n_kv,
                           int head_dim, int64_t max_ctx, float scale, void* ws, void* stream) {
  if (!q || !k_cache || !v_cache || !ctx_lens || !out || !ws) return QGEMV_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return QGEMV_EINVAL;
  const int st = check_attention_shape(batch, n_q, n_kv, head_dim, max_ctx);
  if (st) return st;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(ctx_lens, 4) || !aligned(ws, 16))
    return QGEMV_EALIGN;
  qgemv::AttnArgs a{q, k_cache, v_cache, ctx_lens, out, batch, n_q, n_kv, head_dim, max_ctx, scale, ws};
  return record_hip(qgemv::launch_attention(a, static_cast<hipStream_t>(stream)));
}

int qgemv_run_flags(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
                    int64_t M, int64_t K, int batch, int flags, void* stream) {
  if (flags & ~QGEMV_FLAG_BATCH_INVARIANT) return QGEMV_EINVAL;
  int st = check_run_args(fmt, W, scales, x, y, M, K, batch);
  if (st) return st;
  // the invariant mode runs every batch as 8 rows: x of 8 rows must fit in LDS
  if ((flags & QGEMV_FLAG_BATCH_INVARIANT) && qgemv::gemv_lds_bytes(fmt, static_cast<int>(K), 8) > 160 * 1024)
    return QGEMV_ESHAPE;
  qgemv::GemvArgs a{fmt, W, scales, x, y, static_cast<int>(M), static_cast<int>(K), batch};
  return record_hip(qgemv::launch_gemv(a, static_cast<hipStream_t>(stream), flags));
}


namespace {

// The grouped launches of qgemv_run_grouped; am >= 0: entry am's launch also
// computes the argmax of its output if the small-batch kernel takes it
// (*fused = true), else the caller launches the argmax.
// launch of qgemv_run_grouped an entry goes to (QGEMV_GROUP_*): the register-x
// group of its format, the matrix-core group of its format, or alone
int grouped_kind(int fmt, int K, int batch) {
  return qgemv::gemv_group_class(fmt, K, batch) != 0 ? QGEMV_GROUP_XREG
         : qgemv::gemv_mfma_groupable(fmt, K, batch) ? QGEMV_GROUP_MFMA : QGEMV_GROUP_ALONE;
}

int run_grouped_impl(const qgemv_gemv_desc* gemvs, int n, int batch, hipStream_t s, int am,
                     uint64_t* slots, int32_t* idx, bool* fused) {
  // GEMVs the register-x kernel takes are launched together, one launch per
  // format (up to gemv_group_max() entries) in order of first appearance;
  // so are those the matrix-core kernel takes, one launch per format (any
  // mix of K); the others are launched one by one.
  std::vector<qgemv::GemvArgs> todo;
  std::vector<int> ids;
  std::vector<char> done(static_cast<size_t>(n), 0);
  if (fused) *fused = false;
  std::vector<int> kind(static_cast<size_t>(n));
  for (int i = 0; i < n; ++i) kind[i] = grouped_kind(gemvs[i].fmt, gemvs[i].K, batch);
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const qgemv_gemv_desc& g = gemvs[i];
    const int cls = kind[i];
    todo.clear();
    ids.clear();
    for (int k = i; k < n; ++k) {
      const qgemv_gemv_desc& h = gemvs[k];
      if (done[k]) continue;
      if (cls == QGEMV_GROUP_ALONE ? k != i : (h.fmt != g.fmt || kind[k] != cls))
        continue;
      todo.push_back(qgemv::GemvArgs{h.fmt, h.W, h.scales, h.x, h.y, h.M, h.K, batch});
      ids.push_back(k);
      done[k] = 1;
    }
    const int maxn = cls == QGEMV_GROUP_ALONE ? 1 : qgemv::gemv_group_max();
    for (size_t off = 0; off < todo.size(); off += maxn) {
      const int cnt = static_cast<int>(std::min(todo.size() - off, static_cast<size_t>(maxn)));
      hipError_t e;
      if (cls == QGEMV_GROUP_ALONE) {
        e = qgemv::launch_gemv(todo[off], s);
      } else if (cls == QGEMV_GROUP_MFMA) {
        int local_am = -1;
        for (int t = 0; t < cnt; ++t)
          if (ids[off + t] == am) local_am = t;
        e = qgemv::launch_gemv_mfma_group(&todo[off], cnt, s, local_am, slots, idx);
        if (local_am >= 0 && fused) *fused = true;
      } else {
        int local_am = -1;
        for (int t = 0; t < cnt; ++t)
          if (ids[off + t] == am) local_am = t;
        e = qgemv::launch_gemv_group(&todo[off], cnt, s, local_am, slots, idx);
        if (local_am >= 0 && fused) *fused = true;
      }
      const int st = record_hip(e);
      if (st) return st;
    }
  }
  return QGEMV_OK;
}

int check_grouped(const qgemv_gemv_desc* gemvs, int n, int batch) {
  if (!gemvs || n < 1) return QGEMV_EINVAL;
  if (n > QGEMV_GROUP_MAX) return QGEMV_ESHAPE;
  for (int i = 0; i < n; ++i) {
    const qgemv_gemv_desc& g = gemvs[i];
    const int st = check_run_args(g.fmt, g.W, g.scales, g.x, g.y, g.M, g.K, batch);
    if (st) return st;
  }
  return QGEMV_OK;
}

}  // namespace

int qgemv_run_grouped(const qgemv_gemv_desc* gemvs, int n, int batch, void* stream) {
  const int st = check_grouped(gemvs, n, batch);
  if (st) return st;
  return run_grouped_impl(gemvs, n, batch, static_cast<hipStream_t>(stream), -1, nullptr, nullptr, nullptr);
}

int qgemv_grouped_class(int fmt, int64_t K, int batch) {
  if (!valid_fmt(fmt)) return QGEMV_EINVAL;
  const int st = check_shape(fmt, 1, K);
  if (st) return st;
  if (batch < 1 || batch > QGEMV_MAX_BATCH) return QGEMV_ESHAPE;
  const int k = static_cast<int>(K);
  return grouped_kind(fmt, k, batch);
}

int qgemv_run_grouped_argmax(const qgemv_gemv_desc* gemvs, int n, int batch, int argmax_entry,
                             uint64_t* ws, int32_t* idx, void* stream) {
  int st = check_grouped(gemvs, n, batch);
  if (st) return st;
  if (argmax_entry < 0 || argmax_entry >= n || !ws || !idx) return QGEMV_EINVAL;
  if (!aligned(ws, 8) || !aligned(idx, 4)) return QGEMV_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool fused = false;
  st = run_grouped_impl(gemvs, n, batch, s, argmax_entry, ws, idx, &fused);
  if (st) return st;
  if (fused) return QGEMV_OK;
  const qgemv_gemv_desc& g = gemvs[argmax_entry];
  return record_hip(qgemv::launch_argmax(g.y, g.M, batch, ws, idx, s));
}

int qgemv_argmax(const float* logits, int64_t V, int batch, uint64_t* ws, int32_t* idx,
                 void* stream) {
  if (!logits || !ws || !idx) return QGEMV_EINVAL;
  if (V < 1 || V > 0x7FFFFFFF || batch < 1 || batch > QGEMV_MAX_BATCH) return QGEMV_ESHAPE;
  if (!aligned(logits, 4) || !aligned(ws, 8) || !aligned(idx, 4)) return QGEMV_EALIGN;
  return record_hip(qgemv::launch_argmax(logits, V, batch, ws, idx, static_cast<hipStream_t>(stream)));
}

int qgemv_argmax_noalloc(const float* logits, int64_t V, int batch, int32_t* idx, void* stream) {
  if (!logits || !idx) return QGEMV_EINVAL;
  if (V < 1 || V > 0x7FFFFFFF || batch < 1 || batch > QGEMV_ARGMAX_NOALLOC_MAX_BATCH) return QGEMV_ESHAPE;
  if (!aligned(logits, 4) || !aligned(idx, 4)) return QGEMV_EALIGN;
  return record_hip(qgemv::launch_argmax_noalloc(logits, V, batch, idx, static_cast<hipStream_t>(stream)));
}

int qgemv_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, int unroll,
                      void* stream) {
  if (!buf || !sink) return QGEMV_EINVAL;
  if (bytes == 0 || bytes % 16 != 0) return QGEMV_ESHAPE;
  if (grid < 0 || grid > 1 << 20) return QGEMV_ESHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return QGEMV_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QGEMV_EALIGN;
  if (grid == 0) grid = 2048;
  return record_hip(qgemv::launch_stream_read(buf, bytes, sink, grid, unroll,
                                              static_cast<hipStream_t>(stream)));
}

const char* qgemv_status_str(int status) {
  switch (status) {
    case QGEMV_OK: return "QGEMV_OK";
    case QGEMV_EINVAL: return "QGEMV_EINVAL: null pointer or unknown format/kind";
    case QGEMV_ESHAPE: return "QGEMV_ESHAPE: unsupported shape or batch";
    case QGEMV_EALIGN: return "QGEMV_EALIGN: misaligned pointer";
    case QGEMV_ERANGE: return "QGEMV_ERANGE: non-finite weight or binary16 scale overflow";
    case QGEMV_EHIP: return "QGEMV_EHIP: HIP call failed";
    default: return "QGEMV: unknown status";
  }
}

int qgemv_last_hip_error(void) { return g_last_hip_error; }

const char* qgemv_version(void) { return "qgemv 0.1.0 gfx950"; }

}  // extern "C"
