/*
 * qgemv.h - C ABI of the fused-dequantization decode GEMV library (libqgemv.so)
 *
 * The operation: y = W x for one decode step, batch 1..8, with the weight
 * dequantization done in registers while the weights stream from HBM. Decode
 * reads every weight once and does one multiply-add with it, so the kernel
 * is bound by HBM bandwidth and the only lever is the number of weight bytes
 * ("Writing an LLM inference engine from scratch in Rust", Lesson 1; "infer",
 * the roofline discussion and the quantized-GEMV table).
 *
 * Weight formats (planar: codes in one array, binary16 scales in another,
 * both row-major; this is also the device layout qgemv_run reads):
 *   QGEMV_BF16       W: uint16 bf16 bits [M][K]; no scales.
 *   QGEMV_INT8_G32   W: int8 [M][K]; scales: binary16 [M][K/32];
 *                    weight = code * scale (a 32-value int8 block with one
 *                    scale, as in the Rust page's Lesson 6 and llama.cpp's
 *                    Q8_0 cited on the infer page's perplexity notes).
 *   QGEMV_Q4_0_G32   W: uint8 [M][K/32][16]; scales: binary16 [M][K/32];
 *                    element j of a block is the low nibble of byte j,
 *                    element j+16 the high nibble; weight = (code-8)*scale
 *                    (Rust page, Lessons 1 and 6: 4.5 bits per weight, stored
 *                    value = weight + 8).
 *   QGEMV_INT4_G128  W: uint8 [M][K/128][64]; scales: binary16 [M][K/128];
 *                    element j of a block is the low nibble of byte j,
 *                    element j+64 the high nibble; weight = (code-8)*scale
 *                    ("infer", g128 rows of the decode and perplexity tables;
 *                    the nibble order is this library's reading, the same
 *                    half-split as Q4_0).
 *   QGEMV_INT8_ROW   W: int8 [M][K]; scales: binary16 [M] (one per row);
 *                    weight = code * scale ("infer", perplexity table and
 *                    notes: its int8 weights have one scale per row; the
 *                    scale type is this library's reading).
 *   QGEMV_INT4_G64   W: uint8 [M][K/64][32]; scales: binary16 [M][K/64];
 *                    element j of a block is the low nibble of byte j,
 *                    element j+32 the high nibble; weight = (code-8)*scale
 *                    ("infer", the g64 row of the perplexity table; nibble
 *                    order as for g128).
 * Activations x: bf16 bits [batch][K]. Output y: float32 [batch][M].
 *
 * Conventions for every entry point:
 *   - returns QGEMV_OK (0) or a negative status; on error nothing has been
 *     launched and no output has been written (errors are values, never
 *     exceptions or aborts, as in the Mini Inference Engine page's block
 *     pool, whose out-of-memory result is a sentinel);
 *   - the library never allocates device memory, never frees, never keeps a
 *     caller pointer past the call and never synchronizes a stream; its only
 *     device state is qgemv_argmax_noalloc's static workspace (128 bytes per
 *     GPU, part of the loaded code object);
 *   - the caller owns every buffer; device entry points run asynchronously
 *     on the caller's stream (hipStream_t passed as void*, NULL = the null
 *     stream); reading W and scales from several streams at once is safe;
 *   - thread-safe; the HIP error of the last failed launch on the calling
 *     thread is available from qgemv_last_hip_error().
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QGEMV_BF16 = 0,
  QGEMV_INT8_G32 = 1,
  QGEMV_Q4_0_G32 = 2,
  QGEMV_INT4_G128 = 3,
  QGEMV_INT8_ROW = 4,
  QGEMV_INT4_G64 = 5
};

/* source kinds for qgemv_pack */
enum {
  QGEMV_SRC_CANONICAL = 0, /* codes + binary16 scales already in the layout above */
  QGEMV_SRC_BF16 = 1       /* bf16 weights [M][K]: quantize them */
};

enum {
  QGEMV_OK = 0,
  QGEMV_EINVAL = -1, /* null pointer, unknown format or source kind */
  QGEMV_ESHAPE = -2, /* M < 1, K not a positive multiple of the group (32;
                        128 for int4-g128, 64 for int4-g64), batch outside 1..8, V < 1, or K
                        beyond what one workgroup's LDS can stage */
  QGEMV_EALIGN = -3, /* W, x or y not 16-byte aligned; scales or logits not
                        4-byte aligned; ws not 8-byte aligned */
  QGEMV_ERANGE = -4, /* quantize: a non-finite weight, or a scale whose
                        binary16 rounding overflows (|scale| > 65504) */
  QGEMV_EHIP = -5    /* a HIP call failed; see qgemv_last_hip_error() */
};

/* Largest batch qgemv_run accepts (decode verifies up to 8 tokens per pass,
 * the Rust page's speculative-decoding section). */
#define QGEMV_MAX_BATCH 8

/*
 * qgemv_packed_size - bytes of the device layout of an M x K matrix.
 * Host only, no HIP calls. *w_bytes gets the code bytes (2MK for bf16, MK
 * for the int8 formats, MK/2 for the 4-bit ones), *s_bytes the scale bytes
 * (0 for bf16, 2M for int8-row, else 2*M*K/G). These are the byte counts the pages use for
 * their bandwidth figures (4.5 bits per weight for Q4_0; "infer"'s per-token
 * weight totals). Errors: EINVAL (null out-pointer, bad fmt), ESHAPE.
 */
int qgemv_packed_size(int fmt, int64_t M, int64_t K, size_t* w_bytes, size_t* s_bytes);

/*
 * qgemv_pack - build the device layout in host memory (host only, no HIP
 * calls; upload the result with any copy routine).
 *   src_kind CANONICAL: src_w / src_scales are codes and binary16 scales in
 *     the layout above; they are validated and copied. For bf16, src_scales
 *     and dst_scales are ignored (may be NULL).
 *   src_kind BF16: src_w is bf16 bits [M][K]; for a quantized format each
 *     group is quantized (src_scales ignored): 4-bit formats take the
 *     group's element of largest magnitude with its sign, m, and set
 *     scale = binary16(m / -8) so that m maps to code 0 (Rust page, "Is the
 *     4-bit model still good?"; "infer", design notes); the int8 formats
 *     set scale = binary16(max|w| / 127) over the group (int8-row: the row). Then code = round-half-even(w / scale)
 *     (+8 for 4-bit), clamped to [0,15] or [-127,127]; ties in |w| go to the
 *     first element; a scale that rounds to zero is stored as +0 with every
 *     code 8 (4-bit) or 0 (int8). The division is done in double precision
 *     after the scale has been rounded to binary16.
 * dst_w must hold qgemv_packed_size's w_bytes, dst_scales its s_bytes.
 * Errors: EINVAL, ESHAPE, ERANGE (BF16 source only). Deterministic.
 */
int qgemv_pack(int fmt, int src_kind, const void* src_w, const uint16_t* src_scales,
               int64_t M, int64_t K, void* dst_w, uint16_t* dst_scales);

/*
 * qgemv_quantize - the quantizer of qgemv_pack (src_kind BF16) on the
 * device: bf16 weights w [M][K] -> codes and binary16 scales in the layout
 * above, bit-identical to what qgemv_pack writes for the same weights (the
 * rule and its readings as documented there: the Rust page, "Is the 4-bit
 * model still good?"; "infer", design notes and its quantizer tests).
 * fmt: any quantized format (EINVAL for BF16). Device pointers:
 * w 16-byte aligned; codes (qgemv_packed_size's w_bytes) 16-byte aligned;
 * scales (s_bytes) 4-byte aligned; err: a device int32 or NULL. A group
 * with a non-finite weight or a scale past binary16's range stores
 * unspecified codes and scale and sets *err = QGEMV_ERANGE (err is never
 * cleared: zero it before the call and read it after synchronizing).
 * Asynchronous on `stream`; one kernel, one thread per group.
 * Errors (returned): EINVAL, ESHAPE, EALIGN, EHIP.
 */
int qgemv_quantize(int fmt, const uint16_t* w, int64_t M, int64_t K, void* codes, uint16_t* scales,
                   int32_t* err, void* stream);

/*
 * qgemv_run - y[b][m] = sum_k weight(m,k) * x[b][k], 0 <= b < batch.
 * Device pointers. W / scales in the layout above (scales may be NULL for
 * bf16); x: bf16 [batch][K]; y: float32 [batch][M], overwritten (not
 * accumulated). Accumulation is float32; each 32-weight group's scale is
 * applied once to the group's partial sum. 1 <= batch <= 8, M >= 1 (any
 * value), K a multiple of 32 (128 for int4-g128, 64 for int4-g64) such that x fits in
 * one workgroup's LDS: nb * K * 2 bytes (plus nb * K / 8 for the 4-bit
 * formats) <= 163840, nb = batch rounded up to 1, 2, 4 or 8 (e.g. 4-bit:
 * K <= 9632 at batch 5..8, K <= 77088 at batch 1; bf16/int8: K <= 10240 at
 * batch 5..8).
 * Alignment: W, x, y 16 bytes; scales 4 bytes.
 * Asynchronous on `stream`; no allocation, no synchronization.
 */
int qgemv_run(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
              int64_t M, int64_t K, int batch, void* stream);

/* qgemv_run_flags flag: batch-invariant results (see qgemv_run_flags). */
#define QGEMV_FLAG_BATCH_INVARIANT 1

/*
 * qgemv_run_flags - qgemv_run with options. QGEMV_FLAG_BATCH_INVARIANT:
 * row b of y is bit-identical to what a batch-1 call on x[b] alone returns
 * with the same flag, for every batch 1..8 - the fixed per-row summation
 * order that lets a batched pass (e.g. speculative verification of several
 * draft tokens, the Rust page's speculative-decoding section) be checked
 * against single-token decoding with exact equality. Every batch then runs
 * the kernels of batch 8 with launch shapes chosen from (fmt, M, K) only,
 * so it costs the batch-8 time even at batch 1, and x of 8 rows must fit in
 * LDS (K as for batch 5..8 in qgemv_run, else ESHAPE). flags 0 is qgemv_run.
 * Errors: as qgemv_run; EINVAL for unknown flag bits.
 */
int qgemv_run_flags(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
                    int64_t M, int64_t K, int batch, int flags, void* stream);

/* One GEMV of a grouped call (same meaning and layout rules as qgemv_run). */
typedef struct {
  const void* W;          /* device: codes (or bf16 weights) */
  const uint16_t* scales; /* device: binary16 scales (NULL for bf16) */
  const uint16_t* x;      /* device: bf16 [batch][K] */
  float* y;               /* device: float32 [batch][M], overwritten */
  int32_t fmt;
  int32_t M;
  int32_t K;
  int32_t reserved;       /* set to 0 */
} qgemv_gemv_desc;

/* Largest n qgemv_run_grouped accepts in one call. */
#define QGEMV_GROUP_MAX 1024

/*
 * qgemv_run_grouped - n independent GEMVs, all at the same batch:
 * gemvs[i].y = W_i x_i for every i. Host array of descriptors (read during
 * the call only); device pointers inside. No entry may read what another
 * writes (no y of one entry may overlap any W, scales, x or y of another):
 * the order in which entries are computed is unspecified. This is the shape
 * of a decode step's independent projections (the GEMV sets and the
 * 89-GEMV weight stream of a TinyLlama step measured here; the experts of a
 * mixture-of-experts layer are another).
 * Entries of one format that the small-batch kernel handles (batch <= 2 and
 * at most 256 16-byte units per row: K <= 2048 bf16, 4096 int8, 8192 4-bit;
 * int8 at batch 1 up to 512 units, K <= 8192) share launches (one per format, up to 64 entries each), and so do entries
 * of one format that the matrix-core kernel handles, whatever their K
 * (batch 3..8, K a multiple of 512 for the 4-bit formats, 256 for int8, 128
 * for bf16, x of 8 (batch 5..8) or 4 rows in LDS), so the per-launch
 * start-up cost is paid once per group instead of once per GEMV; other
 * entries are launched one by one. All validation
 * happens before anything is launched. Errors as qgemv_run; ESHAPE also
 * for n > QGEMV_GROUP_MAX.
 */
int qgemv_run_grouped(const qgemv_gemv_desc* gemvs, int n, int batch, void* stream);

/* launches of qgemv_run_grouped (qgemv_grouped_class) */
#define QGEMV_GROUP_ALONE 0   /* a launch of its own */
#define QGEMV_GROUP_XREG 1    /* the small-batch launch of its format */
#define QGEMV_GROUP_MFMA 2    /* the matrix-core launch of its format */

/*
 * qgemv_grouped_class - which launch qgemv_run_grouped (and
 * qgemv_run_grouped_argmax) gives an entry of this format, row length and
 * batch: QGEMV_GROUP_XREG, QGEMV_GROUP_MFMA or QGEMV_GROUP_ALONE (the rule
 * stated under qgemv_run_grouped). Host only, no launch; reads the current
 * device's compute-unit count (the matrix-core plan depends on it). Returns
 * the class, or EINVAL / ESHAPE (negative) for an unknown format, a K that
 * the format does not allow, or a batch outside 1..8.
 */
int qgemv_grouped_class(int fmt, int64_t K, int batch);

/* u64 words of workspace qgemv_argmax needs per batch row */
#define QGEMV_ARGMAX_WS_WORDS_PER_ROW 2

/*
 * qgemv_argmax - greedy token: idx[b] = the first index of the largest
 * logits[b][v] over 0 <= v < V ("infer", the decode pipeline figure and the
 * per-kernel table's argmax row; its tests cover ties). Ties go to the lowest
 * index; -0.0 equals +0.0; if a row holds a NaN the result is the index of
 * its first NaN (NumPy argmax semantics); all -inf gives 0.
 * Device pointers: logits float32 [batch][V] (4-byte aligned), idx int32
 * [batch], ws: batch * QGEMV_ARGMAX_WS_WORDS_PER_ROW u64 words (8-byte
 * aligned), owned by the caller. ws must be all zero before its first use;
 * every call leaves it all zero again, so one zero-fill at allocation time
 * suffices. Calls that may run concurrently need distinct ws buffers.
 * 1 <= batch <= 8, 1 <= V <= 2^31 - 1. One kernel launch; asynchronous.
 * Rows are split into slices of 1-16 Ki logits (about 32 workgroups per
 * launch); a row of one slice is reduced by one workgroup without touching
 * ws, the slices of a longer row meet in ws with atomics.
 */
int qgemv_argmax(const float* logits, int64_t V, int batch, uint64_t* ws, int32_t* idx,
                 void* stream);

/* Largest batch qgemv_argmax_noalloc accepts (the rows its static scratch holds). */
#define QGEMV_ARGMAX_NOALLOC_MAX_BATCH 8

/*
 * qgemv_argmax_noalloc - qgemv_argmax for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernel, semantics and results,
 * with the workspace taken from a static array inside the library instead of
 * a caller buffer. The array holds QGEMV_ARGMAX_NOALLOC_MAX_BATCH rows of
 * QGEMV_ARGMAX_WS_WORDS_PER_ROW u64 words (128 bytes); each GPU the library
 * runs on keeps its own copy until the process ends. The first call on a
 * device (the current device, which must own `stream`) looks the array up
 * and clears it with a small kernel on `stream` ahead of the argmax; every
 * call leaves it zero again. Device pointers: logits float32 [batch][V]
 * (4-byte aligned), idx int32 [batch] (4-byte aligned).
 * 1 <= batch <= QGEMV_ARGMAX_NOALLOC_MAX_BATCH (else ESHAPE, nothing
 * launched), 1 <= V <= 2^31 - 1. No hipMalloc, hipFree or other allocation.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (concurrent streams, or host threads driving one device) race and
 * can return wrong indices; serialize them, or use qgemv_argmax with a
 * workspace per stream. Asynchronous on `stream`.
 * Errors: EINVAL (null pointer), ESHAPE, EALIGN, EHIP.
 */
int qgemv_argmax_noalloc(const float* logits, int64_t V, int batch, int32_t* idx, void* stream);

/* u64 words of workspace qgemv_run_grouped_argmax needs per batch row */
#define QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW 4096

/*
 * qgemv_run_grouped_argmax - a decode step's end in one call: the GEMVs of
 * qgemv_run_grouped, then idx[b] = the argmax of row b of
 * gemvs[argmax_entry].y (the LM-head logits, V = that entry's M), with
 * qgemv_argmax's semantics ("infer": the decode pipeline figure ends the
 * step with the LM head and the argmax; its design notes fuse work into the
 * producing kernel to save launches).
 * When the small-batch kernel computes the argmax entry (batch <= 2, row
 * length as in qgemv_run_grouped), the argmax runs inside that launch: each
 * wave folds the logits it writes into one key per batch row and
 * publishes it in its own word of ws, and one workgroup of the launch, which
 * does no GEMV work, collects the words while the other entries still
 * stream and takes the largest; no separate launch and no second pass over
 * the logits.
 * When the matrix-core kernel computes it (batch 3..8), each of the entry's
 * workgroups folds the logits it writes into one key per batch row and
 * publishes it in its own word of ws, and again one workgroup of the launch
 * collects the words and takes the largest (the argmax entry's workgroups
 * are dispatched first, so the collecting overlaps the other entries).
 * Otherwise the argmax is a qgemv_argmax launch after the GEMVs, on the same
 * stream, with the same ws. The logits (gemvs[argmax_entry].y) are written
 * in full either way.
 * ws: device, batch * QGEMV_FUSED_ARGMAX_WS_WORDS_PER_ROW u64 words (8-byte
 * aligned), owned by the caller, all zero before its first use; every call
 * leaves it all zero. Calls that may run concurrently need distinct ws.
 * idx: device int32 [batch], 4-byte aligned. idx -1 means that the
 * collecting workgroup's bounded wait (about 2^20 polls) ran out before every
 * wave or workgroup had published its key, which happens only if other work
 * keeps the launch's workgroups from running for that long. The collector
 * then clears every word it can, but a key published afterwards leaves its
 * word set: after idx -1, zero ws again before the next call.
 * Errors: as qgemv_run_grouped; EINVAL for argmax_entry outside [0, n) or a
 * null ws or idx; EALIGN for misaligned ws or idx. Nothing is launched on
 * error.
 */
int qgemv_run_grouped_argmax(const qgemv_gemv_desc* gemvs, int n, int batch, int argmax_entry,
                             uint64_t* ws, int32_t* idx, void* stream);

/*
 * Operations fused into one GEMV by qgemv_run_fused ("infer": the decode
 * pipeline figure and design notes apply RMSNorm while the GEMV stages its
 * input, add the residual in the GEMV's epilogue and compute SwiGLU from
 * paired gate/up rows; the Rust page's layer walk-through names the same
 * normalize / feed-forward steps). NULL fields are unused.
 *
 * norm_input  device float32 h[batch][K], 16-byte aligned: the GEMV's input
 *             becomes x[b][k] = bf16(h[b][k] / sqrt(mean_k h[b][k]^2 + eps)
 *             * norm_weight[k]) (round to nearest even; the call's x must be
 *             NULL). Must not overlap y or swiglu_out.
 * norm_weight device bf16 g[K], 16-byte aligned (required with norm_input).
 * norm_eps    eps >= 0, finite.
 * residual    device float32 [batch][M], 16-byte aligned: y = residual + W x
 *             (one float32 add per output). May be y itself (the residual
 *             stream updated in place); must not overlap it otherwise.
 * swiglu_out  device bf16 act[batch][M/2], 4-byte aligned: with the gate|up
 *             matrix storing gate row i as row 2i and up row i as row 2i+1,
 *             act[b][i] = bf16(silu(y[b][2i]) * y[b][2i+1]), silu(t) =
 *             t / (1 + exp(-t)); y itself is not written (the call's y must
 *             be NULL), M must be even. Not with residual or the argmax.
 * argmax_idx, argmax_ws  as idx and ws of qgemv_run_grouped_argmax for the
 *             argmax of each row of y (fused into the launch at batch <= 2
 *             with short rows and on the matrix-core kernel at batch 3..8,
 *             a separate launch otherwise).
 */
typedef struct qgemv_fusion {
  const float* norm_input;
  const uint16_t* norm_weight;
  float norm_eps;
  const float* residual;
  uint16_t* swiglu_out;
  int32_t* argmax_idx;
  uint64_t* argmax_ws;
} qgemv_fusion;

/*
 * qgemv_run_fused - qgemv_run with the operations of *fusion fused in: the
 * RMSNorm prologue while x is staged, then one epilogue (plain store,
 * residual add, or SwiGLU), optionally followed by the argmax of y. One
 * launch (plus an argmax launch where it is not fused). x: bf16 [batch][K]
 * or NULL with norm_input; y: float32 [batch][M] or NULL with swiglu_out.
 * Errors: as qgemv_run; EINVAL for a null fusion, both or neither of x and
 * norm_input, norm_input without norm_weight, a negative or non-finite eps,
 * swiglu_out together with y, residual or the argmax, a missing y
 * otherwise, or only one of argmax_idx / argmax_ws; ESHAPE for odd M with
 * swiglu_out, or x of the batch plus 1 KiB of scratch not fitting in LDS
 * where x is staged there; EALIGN for misaligned pointers. Nothing is
 * launched on error.
 */
int qgemv_run_fused(int fmt, const void* W, const uint16_t* scales, const uint16_t* x, float* y,
                    int64_t M, int64_t K, int batch, const qgemv_fusion* fusion, void* stream);

/*
 * Grouped-query decode attention - the other bandwidth-bound kernel of a
 * decode step: every query head compares its query with the keys of all
 * earlier positions of its sequence in the KV cache and takes the
 * softmax-weighted average of their values; groups of G = n_q / n_kv query
 * heads share one key/value head, query head h reading key/value head h / G
 * (the Rust page: layer walk-through and its attention rounds - online
 * softmax over 64-position blocks, query heads of one key/value head
 * processed together; "infer": split-KV decode attention with one block per
 * key/value head and a merge of the splits, bf16 KV cache).
 *   out[b][h][j] = sum_t p_t v[b][h/G][t][j] / sum_t p_t,
 *   p_t = exp(scale * sum_j q[b][h][j] k[b][h/G][t][j] - max_t(...)),
 *   0 <= t < ctx_lens[b].
 *
 * qgemv_attention_workspace_size - bytes of device workspace a call with
 * this shape needs (*bytes, at least 256; host only, no HIP calls). It holds
 * the splits' partial results between the call's two kernels; its contents
 * on entry do not matter. Calls that may run concurrently need distinct
 * workspaces.
 * Errors: EINVAL (null bytes), ESHAPE (as below).
 */
int qgemv_attention_workspace_size(int batch, int n_q, int n_kv, int head_dim, int64_t max_ctx,
                                   size_t* bytes);

/*
 * qgemv_attention_decode - one decode step's attention for `batch`
 * sequences. Device pointers:
 *   q        float32 [batch][n_q][head_dim], 16-byte aligned;
 *   k_cache, v_cache  bf16 bits [batch][n_kv][max_ctx][head_dim], 16-byte
 *            aligned; only positions < ctx_lens[b] of sequence b are read;
 *   ctx_lens int32 [batch], 4-byte aligned, each in 1..max_ctx (values
 *            outside are clamped into that range; on the device so that a
 *            captured graph stays valid as positions advance);
 *   out      float32 [batch][n_q][head_dim], 16-byte aligned, overwritten;
 *   ws       qgemv_attention_workspace_size bytes, 16-byte aligned.
 * Shapes: batch >= 1, n_kv >= 1, n_q = G * n_kv with G in {1, 2, 4, 8},
 * head_dim 64 or 128, 1 <= max_ctx with (max_ctx + 64) * head_dim * 2 < 2^32;
 * scale > 0 and finite (1/sqrt(head_dim) for Llama models).
 * Float32 arithmetic on the bf16 cache values. One launch, or two when the
 * context is split over several workgroups (the second merges the splits);
 * asynchronous on `stream`. Errors: EINVAL (null pointer, non-finite or
 * non-positive scale), ESHAPE, EALIGN, EHIP.
 */
int qgemv_attention_decode(const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* ctx_lens, float* out, int batch, int n_q, int n_kv,
                           int head_dim, int64_t max_ctx, float scale, void* ws, void* stream);

/*
 * qgemv_stream_read - measurement helper: read `bytes` bytes of device
 * memory at `buf` once with 16-byte loads and write one checksum word per
 * workgroup to sink[0 .. grid-1] (so the reads cannot be elided). This is the
 * streaming-read kernel whose best rate is the measured HBM peak that GEMV
 * bandwidth is reported against (the infer page reports its GEMVs against a
 * streaming-read peak it measured itself). grid: workgroups (0 = 2048),
 * unroll: 16-byte loads in flight per thread per iteration (1, 2, 4, 8 or
 * 16). buf 16-byte aligned, bytes a multiple of 16.
 */
int qgemv_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, int unroll,
                      void* stream);

/* Human-readable name of a status code (static storage). */
const char* qgemv_status_str(int status);

/* hipError_t of the last HIP failure on the calling thread (0 if none). */
int qgemv_last_hip_error(void);

/* Library version, e.g. "qgemv 0.1.0 gfx950". */
const char* qgemv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
