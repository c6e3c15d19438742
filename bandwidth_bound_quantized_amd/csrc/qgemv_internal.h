// Internal interface between the C-ABI front end (qgemv_api.cpp) and the
// HIP kernel translation units. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qgemv {

// Per-format geometry of one 16-byte "unit" of a weight row: the amount of
// code bytes one lane loads with a single 16-byte load.
//   bf16      : 8 weights per unit
//   int8-g32  : 16 weights per unit, two units per scale group
//   4-bit g32 : 32 weights per unit (one whole block)
//   4-bit g128: 32 weights per unit, four units per scale group
struct FmtInfo {
  int group;          // weights per scale (1 for bf16)
  int elems_per_unit; // weights per 16 code bytes
};

FmtInfo fmt_info(int fmt);

// Launch-time description of one GEMV.
struct GemvArgs {
  int fmt;
  const void* W;
  const uint16_t* scales;
  const uint16_t* x;
  float* y;
  int M;
  int K;
  int batch;
};

// Operations fused into one GEMV (qgemv_run_fused): the RMSNorm prologue
// (x = bf16(h / sqrt(mean(h^2) + eps) * g) when h is set) and one epilogue.
constexpr int kEpiStore = 0;      // y = W x
constexpr int kEpiResidual = 1;   // y = res + W x (res may be y)
constexpr int kEpiSwiglu = 2;     // act[b][i] = bf16(silu(y[b][2i]) * y[b][2i+1]); y not written
struct Fusion {
  const float* h = nullptr;       // [batch][K] float32, or nullptr (x is the input)
  const uint16_t* g = nullptr;    // [K] bf16 norm weight
  float eps = 0.f;
  int epi = kEpiStore;
  const float* res = nullptr;     // [batch][M]
  uint16_t* act = nullptr;        // [batch][M/2] bf16
};

// LDS the fused prologue adds to a workgroup that stages x in LDS.
constexpr size_t kNormScratchBytes = 1024;

// Bytes of LDS the GEMV kernel stages per workgroup for this shape
// (x as bf16 for the compiled batch, plus per-unit x sums for 4-bit formats).
size_t gemv_lds_bytes(int fmt, int K, int batch);

// Whether the GEMV of this shape (fused: through launch_gemv_fused) stages x
// in LDS (batch > 2 or long rows); otherwise each lane keeps its share of x
// in registers and no LDS is used.
bool gemv_uses_lds(int fmt, int K, int batch, bool fused = false);

// Launch the GEMV on `stream` (flags: QGEMV_FLAG_*). Shapes have been
// validated by the caller.
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream, int flags = 0);

// One GEMV with the operations of f fused in; idx != nullptr: also the
// argmax of each row of y into idx (slots as for launch_gemv_group; not with
// kEpiSwiglu). Shapes and pointers have been validated by the caller.
hipError_t launch_gemv_fused(const GemvArgs& a, const Fusion& f, uint64_t* slots, int32_t* idx,
                             hipStream_t stream);

// Grouped launches of independent GEMVs (register-x kernel only).
// gemv_group_class: 0 if (fmt, K, batch) needs another kernel, else the number
// of 16-byte units per lane-column of a row (1..4, or 8 for int8 rows of
// 65..128 units at batch 1); GEMVs of one format and
// batch with a nonzero class can share a launch. launch_gemv_group:
// n <= gemv_group_max() such GEMVs, already validated.
// am >= 0: the launch also writes idx[b] = argmax of row b of a[am].y, using
// slots (batch * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW words, zero on entry,
// zero on exit).
int gemv_group_class(int fmt, int K, int batch);
int gemv_group_max();
hipError_t launch_gemv_group(const GemvArgs* a, int n, hipStream_t stream, int am = -1,
                             uint64_t* slots = nullptr, int32_t* idx = nullptr);

// Grouped launches on the matrix cores (batch 3..8): whether qgemv_run runs
// a GEMV of this (fmt, K, batch) on the matrix-core kernel; GEMVs of one
// format and batch for which it does can share a launch, whatever their K
// (n <= gemv_group_max(), already validated).
// am >= 0: the launch also writes idx[b] = argmax of row b of a[am].y (slots as
// for launch_gemv_group: zero on entry, zero on exit).
bool gemv_mfma_groupable(int fmt, int K, int batch);
hipError_t launch_gemv_mfma_group(const GemvArgs* a, int n, hipStream_t stream, int am = -1,
                                  uint64_t* slots = nullptr, int32_t* idx = nullptr);

// Launch the argmax (one kernel). ws: batch * 2 u64 words, zero on entry.
hipError_t launch_argmax(const float* logits, int64_t V, int batch, uint64_t* ws, int32_t* idx,
                         hipStream_t stream);

// The argmax with its workspace in the library's per-device static scratch
// (qgemv_argmax_noalloc); batch <= QGEMV_ARGMAX_NOALLOC_MAX_BATCH.
hipError_t launch_argmax_noalloc(const float* logits, int64_t V, int batch, int32_t* idx,
                                 hipStream_t stream);

// Quantizer (bf16 -> codes + scales) on the device; err may be null.
hipError_t launch_quantize(int fmt, const uint16_t* w, int64_t M, int64_t K, void* codes, uint16_t* scales,
                           int32_t* err, hipStream_t stream);

// Grouped-query decode attention (qgemv_attention_decode); shapes validated.
struct AttnArgs {
  const float* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lens;
  float* out;
  int batch, n_q, n_kv, head_dim;
  int64_t max_ctx;
  float scale;
  void* ws;
};
// How the context is split: `splits` workgroups per (sequence, key/value
// head), `positions` each; the workspace holds part_bytes of per-split
// records (none with one split).
struct AttnPlan {
  int splits = 1;
  int positions = 0;
  size_t part_bytes = 0;
  bool short_blocks = false;   // softmax blocks of at most 16 positions (small calls)
};
AttnPlan attention_plan(int batch, int n_q, int n_kv, int head_dim, int64_t max_ctx);
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// Streaming-read measurement kernel.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, int unroll,
                              hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

constexpr int kArgmaxSlices = 128;   // max workgroups per batch row in the argmax

}  // namespace qgemv
