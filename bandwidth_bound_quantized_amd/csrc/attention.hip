// Grouped-query decode attention over a bf16 KV cache (gfx950), split over
// the context ("infer": split-KV decode attention, one block per key/value
// head serving its query heads, splits to fill the GPU at long context, then
// a merge; the Rust page: online softmax over 64-position blocks, query
// heads that share a key/value head processed together so the cache is read
// once per key/value head).
//
// out[b][h][:] = sum_t p_t v[b][h/G][t][:] / sum_t p_t,
// p_t = exp(scale * q[b][h] . k[b][h/G][t] - max), t < L_b.
//
// Work: one workgroup (4 waves) per (sequence b, key/value head, split s);
// split s covers P consecutive positions, taken by the waves in blocks of BP
// positions round-robin. Inside a wave, SUB adjacent lanes share a position
// and each owns DL = 64 / G consecutive head dims, so every lane keeps the G
// query heads' slices of q (G * DL = 64 floats) and of the output
// accumulator (64 floats) in registers; a round covers PP = 64 / SUB
// positions, whose K (then V) rows are one contiguous stretch of the cache.
// Scores: DL-long dot products per lane, summed over the SUB lanes of the
// position; softmax online per block (the block's maximum across the wave,
// one rescale of the accumulator per block). K/V are read through buffer
// resources sized to the sequence's L_b positions: positions past it read
// as zero and are masked, so nothing past the valid cache is touched.
// Float32 arithmetic throughout; exponentials in base 2 with log2(e) folded
// into q.
//
// The waves of a workgroup meet in LDS; with more than one split, each
// workgroup writes its (max, sum, accumulator) for its G heads to the
// caller's workspace, and a second kernel (one workgroup per (b, key/value
// head)) merges the splits and writes out. The kernel boundary orders the
// records' writes before the merge's reads; merging inside the first kernel
// (the last split to arrive, found with a counter) needed a device-scope
// release and acquire in every workgroup, which measured 1.5-2.5x slower.
#include <math.h>
#include <algorithm>
#include <type_traits>

#include "qgemv_internal.h"
#include "qgemv.h"

namespace qgemv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef QGEMV_ATTN_WAVES
#define QGEMV_ATTN_WAVES 4        // waves per workgroup
#endif
#ifndef QGEMV_ATTN_MIN_BLOCKS
#define QGEMV_ATTN_MIN_BLOCKS 1   // blocks per wave before the context is split further
#endif
#ifndef QGEMV_ATTN_TARGET_WGS
#define QGEMV_ATTN_TARGET_WGS 256 // workgroups worth splitting for
#endif
#ifndef QGEMV_ATTN_MAX_SPLITS
#define QGEMV_ATTN_MAX_SPLITS 32  // splits per (sequence, key/value head)
#endif
constexpr int kAttnWaves = QGEMV_ATTN_WAVES;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = QGEMV_ATTN_MAX_SPLITS;
#ifndef QGEMV_ATTN_MERGE_EARLY
#define QGEMV_ATTN_MERGE_EARLY 8  // most splits whose accumulators the merge loads up front
#endif
constexpr int kMergeEarly = QGEMV_ATTN_MERGE_EARLY;

// CAP: most positions per block (16 for small calls, see attention_plan).
template <int D, int G, int CAP = 64>
struct AttnShape {
  static constexpr int DL = 64 / G;                     // head dims per lane
  static constexpr int SUB = D / DL;                    // lanes per position
  static constexpr int PP = 64 / SUB;                   // positions per round
  static constexpr int BP0 = 131072 / (G * G * D);      // at most 32 score registers
  static constexpr int BPC0 = G * D >= 1024 ? 8 : G >= 8 ? 16 : 32;  // (two blocks' loads in flight)
  static constexpr int BPC = BPC0 < CAP ? BPC0 : CAP;
  static constexpr int BP1 = BP0 < BPC ? BP0 : BPC;
  static constexpr int BP = BP1 > PP ? BP1 : PP;        // positions per softmax block
  static constexpr int R = BP / PP;                     // rounds per block
  static_assert(DL >= 8 && DL % 8 == 0 && SUB >= 1 && SUB <= 16 && R >= 1, "shape");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// DL bf16 values (DL / 8 16-byte loads) at byte offset voff of the resource
template <int DL>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rs, uint32_t voff, u32x4 (&w)[DL / 8]) {
#pragma unroll
  for (int i = 0; i < DL / 8; ++i)
    w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, 0, 0));
}

__device__ __forceinline__ float lo_f(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float hi_f(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Cross-lane reductions without LDS: DPP inside a 16-lane row, permlane
// swaps across rows. With both operands the same register, a 32-lane swap
// returns rows (0,1,0,1) and (2,3,2,3): combining them is a butterfly over
// lane bit 5; a 16-lane swap does the same over bit 4.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float across32(float x, bool mx) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return mx ? fmaxf(__uint_as_float(a), __uint_as_float(b)) : __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float across16(float x, bool mx) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return mx ? fmaxf(__uint_as_float(a), __uint_as_float(b)) : __uint_as_float(a) + __uint_as_float(b);
}

// sum over the W lanes of each aligned group of W (every lane gets it)
template <int W>
__device__ __forceinline__ float sum_lanes(float x) {
  if constexpr (W >= 2) x += dppf<0xB1>(x);             // quad_perm [1,0,3,2]
  if constexpr (W >= 4) x += dppf<0x4E>(x);             // quad_perm [2,3,0,1]
  if constexpr (W >= 8) x += dppf<0x141>(x);            // row_half_mirror
  if constexpr (W >= 16) x += dppf<0x140>(x);           // row_mirror
  static_assert(W <= 16, "W");
  return x;
}

// reduce over the lanes that agree in the lane bits below log2(FROM): row
// rotations by FROM, 2 FROM, .. 8 cover a row's lanes of one residue, then
// the two row butterflies
template <int FROM, bool MAX>
__device__ __forceinline__ float reduce_from(float x) {
  if constexpr (FROM <= 1) x = MAX ? fmaxf(x, dppf<0x121>(x)) : x + dppf<0x121>(x);
  if constexpr (FROM <= 2) x = MAX ? fmaxf(x, dppf<0x122>(x)) : x + dppf<0x122>(x);
  if constexpr (FROM <= 4) x = MAX ? fmaxf(x, dppf<0x124>(x)) : x + dppf<0x124>(x);
  if constexpr (FROM <= 8) x = MAX ? fmaxf(x, dppf<0x128>(x)) : x + dppf<0x128>(x);
  x = across16(x, MAX);
  x = across32(x, MAX);
  return x;
}
template <int FROM>
__device__ __forceinline__ float max_lanes_from(float x) { return reduce_from<FROM, true>(x); }
template <int FROM>
__device__ __forceinline__ float sum_lanes_from(float x) { return reduce_from<FROM, false>(x); }

// Per-split partial record in the workspace: m[G], l[G], acc[G][D] (floats).
template <int D, int G>
constexpr int part_floats() { return 2 * G + G * D; }

template <int D, int G, int CAP>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ lens, float* __restrict__ out, int n_kv, int max_ctx, int S, int P,
    float scale, float* __restrict__ parts) {
  using A = AttnShape<D, G, CAP>;
  constexpr int DL = A::DL, SUB = A::SUB, PP = A::PP, BP = A::BP, R = A::R;
  // values: a lane owns 8 head dims of one position; VPI positions per load
  // instruction, VI instructions per block
  constexpr int VLN = D / 8, VPI = 64 / VLN, VI = BP / VPI;
  static_assert(BP % VPI == 0, "block");
  __shared__ float sh_p[kAttnWaves][BP][G];
  __shared__ float sh_m[kAttnWaves][G], sh_l[kAttnWaves][G];
  __shared__ float sh_acc[kAttnWaves][G][D];

  const int s = blockIdx.x % S;
  const int bh = blockIdx.x / S;                        // b * n_kv + kv head
  const int b = bh / n_kv, kvh = bh - b * n_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int sub = lane % SUB, pr = lane / SUB;          // keys: dims slice, position in the round
  const int vl = lane % VLN, vp = lane / VLN;           // values: 8-dim slice, position in the load
  const int L = min(max(lens[b], 1), max_ctx);

  // q slices of the G heads, pre-multiplied by scale * log2(e)
  float qr[G][DL];
  const float qs = scale * kLog2e;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qh = q + (static_cast<size_t>(b) * n_kv * G + kvh * G + g) * D + sub * DL;
#pragma unroll
    for (int j = 0; j < DL; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(qh + j);
      qr[g][j] = v.x * qs; qr[g][j + 1] = v.y * qs; qr[g][j + 2] = v.z * qs; qr[g][j + 3] = v.w * qs;
    }
  }
  float acc[G][8];
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  }

  // this (b, kv head)'s cache rows of this split, [p0, p0 + P) cut at
  // max_ctx (not at the sequence's length, so that the first loads need not
  // wait for it): positions past it (a prefetch of the next block) read as
  // zero and move no data; positions past the length are masked (scores) and
  // zeroed (values) in registers
  const int p0 = s * P, p1 = min(p0 + P, L);
  const int pe = min(p0 + P, max_ctx);
  const size_t head_off = static_cast<size_t>(bh) * max_ctx * D + static_cast<size_t>(p0) * D;
  const uint32_t nbytes = static_cast<uint32_t>(pe - p0) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = attn_rsrc(kc + head_off, nbytes);
  const __amdgpu_buffer_rsrc_t rv = attn_rsrc(vc + head_off, nbytes);

  // a block's keys (key-lane layout) and values (value-lane layout); u0 is
  // the block's first position relative to p0
  auto load_blk = [&](int u0, u32x4 (&kw)[R][DL / 8], u32x4 (&vw)[VI]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      load_row<DL>(rk, static_cast<uint32_t>(u0 + r * PP + pr) * D * 2 + sub * DL * 2, kw[r]);
#pragma unroll
    for (int i = 0; i < VI; ++i)
      vw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rv, static_cast<uint32_t>(u0 + i * VPI + vp) * D * 2 + vl * 16, 0, 0));
  };
  auto do_blk = [&](int u0, const u32x4 (&kw)[R][DL / 8], const u32x4 (&vw)[VI]) {
    // scores (log2 units), -inf past the split
    float sc[R][G];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
      for (int i = 0; i < DL / 8; ++i) {
        const uint32_t wd[4] = {kw[r][i].x, kw[r][i].y, kw[r][i].z, kw[r][i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float k0 = lo_f(wd[c]), k1 = hi_f(wd[c]);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            dot[g] = __builtin_fmaf(qr[g][8 * i + 2 * c], k0, dot[g]);
            dot[g] = __builtin_fmaf(qr[g][8 * i + 2 * c + 1], k1, dot[g]);
          }
        }
      }
      const int t = p0 + u0 + r * PP + pr;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float tot = sum_lanes<SUB>(dot[g]);
        sc[r][g] = t < p1 ? tot : -INFINITY;
      }
    }
    // online softmax: the block's maximum over the wave, one rescale per
    // block; the weights go to LDS for the value lanes
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = sc[0][g];
#pragma unroll
      for (int r = 1; r < R; ++r) bm = fmaxf(bm, sc[r][g]);
      bm = max_lanes_from<SUB>(bm);
      const float mn = fmaxf(m[g], bm);                  // finite: the block has a valid position
      const float alpha = exp2f(m[g] - mn);              // 0 on the first block (m = -inf)
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] *= alpha;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pw = exp2f(sc[r][g] - mn);           // 0 past the split
        l[g] += pw;
        if (sub == 0) sh_p[wave][r * PP + pr][g] = pw;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values: acc[g][0..8) += p[g][t] * v[t][8 vl .. 8 vl + 8); rows past
    // the length may hold anything (NaN * 0 is NaN): zeroed
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int tp = i * VPI + vp;
      float pg[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pg[g] = sh_p[wave][tp][g];
      const bool live = p0 + u0 + tp < p1;
      const uint32_t wd[4] = {live ? vw[i].x : 0u, live ? vw[i].y : 0u, live ? vw[i].z : 0u, live ? vw[i].w : 0u};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v0 = lo_f(wd[c]), v1 = hi_f(wd[c]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g][2 * c] = __builtin_fmaf(pg[g], v0, acc[g][2 * c]);
          acc[g][2 * c + 1] = __builtin_fmaf(pg[g], v1, acc[g][2 * c + 1]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();                    // sh_p is rewritten by the next block
  };

  // the wave's blocks: u0 = wave * BP, + 4 BP, ...; the next block's loads are
  // issued before the current block is computed (two register buffers)
  constexpr int kStep = kAttnWaves * BP;
  int u0 = wave * BP;
  u32x4 ka[R][DL / 8], kb[R][DL / 8];
  u32x4 va[VI], vb[VI];
  load_blk(u0, ka, va);                                 // (issued before the length arrives)
  const int n = p1 - p0;
  if (u0 < n) {
    while (true) {
      load_blk(u0 + kStep, kb, vb);
      do_blk(u0, ka, va);
      u0 += kStep;
      if (u0 >= n) break;
      load_blk(u0 + kStep, ka, va);
      do_blk(u0, kb, vb);
      u0 += kStep;
      if (u0 >= n) break;
    }
  }

  // the wave's totals: accumulators over its value lanes of one slice, sums
  // over all lanes (each position counted by its SUB key lanes)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = sum_lanes_from<1>(l[g]) * (1.f / SUB);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = sum_lanes_from<VLN>(acc[g][j]);
  }
  if (lane < VLN) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) sh_acc[wave][g][8 * vl + j] = acc[g][j];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { sh_m[wave][g] = m[g]; sh_l[wave][g] = l[g]; }
  }
  __syncthreads();

  // the workgroup's (max, sum, accumulator) per head: waves in order
  const int tid = threadIdx.x;
  float* rec_out = parts + (static_cast<size_t>(bh) * S + s) * part_floats<D, G>();
  for (int e = tid; e < G * D; e += kAttnThreads) {
    const int g = e / D, j = e - g * D;
    float M = sh_m[0][g];
#pragma unroll
    for (int w2 = 1; w2 < kAttnWaves; ++w2) M = fmaxf(M, sh_m[w2][g]);
    float a = 0.f, den = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float f = sh_m[w2][g] == -INFINITY ? 0.f : exp2f(sh_m[w2][g] - M);
      a += f * sh_acc[w2][g][j];
      den += f * sh_l[w2][g];
    }
    if (S == 1) {
      out[(static_cast<size_t>(b) * n_kv * G + kvh * G + g) * D + j] = a / den;
    } else {
      rec_out[2 * G + e] = a;
      if (j == 0) { rec_out[g] = M; rec_out[G + g] = den; }
    }
  }
}

// Merge of the S split records of one (b, key/value head) per workgroup:
// per head, the largest split maximum M, the splits' weights 2^(m_s - M) and
// the total weight, then each output the weighted sum of the splits'
// accumulators over the total. One thread per (split, head) works out its
// weight; the accumulators of each thread's first output are loaded together
// with the maxima and sums, so the merge makes one memory round trip.
template <int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(const float* __restrict__ parts,
                                                                  float* __restrict__ out, int n_kv, int S) {
  static_assert(kMaxSplits * G <= kAttnThreads, "one thread per (split, head)");
  __shared__ float sh_m[kMaxSplits][G], sh_f[kMaxSplits][G], sh_fl[kMaxSplits][G];
  const int bh = blockIdx.x;
  const int b = bh / n_kv, kvh = bh - b * n_kv;
  const int tid = threadIdx.x;
  constexpr int PF = part_floats<D, G>();
  const float* rec0 = parts + static_cast<size_t>(bh) * S * PF;
  // with few splits, this thread's first output's accumulators of every
  // split are loaded together with the maxima and sums (one memory round
  // trip); with more, after the weights (holding them all was slower)
  const bool early = S <= kMergeEarly;
  float pre[kMergeEarly];
#pragma unroll
  for (int s2 = 0; s2 < kMergeEarly; ++s2)
    pre[s2] = (early && s2 < S && tid < G * D) ? rec0[s2 * PF + 2 * G + tid] : 0.f;
  float sl = 0.f;
  if (tid < S * G) {
    const int s2 = tid / G, g = tid - s2 * G;
    sh_m[s2][g] = rec0[s2 * PF + g];
    sl = rec0[s2 * PF + G + g];
  }
  __syncthreads();
  // the weight of each (split, head), one per thread
  if (tid < S * G) {
    const int s2 = tid / G, g = tid - s2 * G;
    float M = -INFINITY;
    for (int t = 0; t < S; ++t) M = fmaxf(M, sh_m[t][g]);
    const float ms = sh_m[s2][g];
    const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
    sh_f[s2][g] = f;
    sh_fl[s2][g] = f * sl;
  }
  __syncthreads();
  // output e from the accumulators acc(s2)
  auto store = [&](int e, float a, float den) {
    const int g = e / D, j = e - g * D;
    out[(static_cast<size_t>(b) * n_kv * G + kvh * G + g) * D + j] = a / den;
  };
  if (early && tid < G * D) {
    const int g = tid / D;
    float den = 0.f, a = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kMergeEarly; ++s2) {
      if (s2 < S) {
        den += sh_fl[s2][g];
        a += sh_f[s2][g] * pre[s2];
      }
    }
    store(tid, a, den);
  }
  for (int e = early ? tid + kAttnThreads : tid; e < G * D; e += kAttnThreads) {
    const int g = e / D;
    float den = 0.f, a = 0.f;
#pragma unroll 16
    for (int s2 = 0; s2 < S; ++s2) {
      den += sh_fl[s2][g];
      a += sh_f[s2][g] * rec0[s2 * PF + 2 * G + e];
    }
    store(e, a, den);
  }
}

template <int D, int G>
hipError_t launch_attn_dg(const AttnArgs& a, hipStream_t st) {
  const AttnPlan p = attention_plan(a.batch, a.n_q, a.n_kv, a.head_dim, a.max_ctx);
  const int grid = a.batch * a.n_kv * p.splits;
  float* parts = static_cast<float*>(a.ws);
  if (p.short_blocks)
    attn_decode_kernel<D, G, 16><<<grid, kAttnThreads, 0, st>>>(a.q, a.k, a.v, a.lens, a.out, a.n_kv,
                                                                static_cast<int>(a.max_ctx), p.splits, p.positions,
                                                                a.scale, parts);
  else
    attn_decode_kernel<D, G, 64><<<grid, kAttnThreads, 0, st>>>(a.q, a.k, a.v, a.lens, a.out, a.n_kv,
                                                                static_cast<int>(a.max_ctx), p.splits, p.positions,
                                                                a.scale, parts);
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_merge_kernel<D, G><<<a.batch * a.n_kv, kAttnThreads, 0, st>>>(parts, a.out, a.n_kv, p.splits);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_d(const AttnArgs& a, hipStream_t st) {
  switch (a.n_q / a.n_kv) {
    case 1: return launch_attn_dg<D, 1>(a, st);
    case 2: return launch_attn_dg<D, 2>(a, st);
    case 4: return launch_attn_dg<D, 4>(a, st);
    default: return launch_attn_dg<D, 8>(a, st);
  }
}

}  // namespace

// Splits: up to about one workgroup per CU of a 256-CU device (the same
// for every device, so the workspace size is a function of the shape
// alone), at most 32, and down to one block per wave in a split: with the
// merge in a kernel of its own a split costs one record write and one read
// (a sweep of blocks per wave, target workgroups and split cap on MI355X:
// one block per wave is 20 % faster than two at context 2048 and equal from
// 8192 up; more target workgroups or a cap of 64 were no faster);
// positions per split a multiple of the waves' blocks.
AttnPlan attention_plan(int batch, int n_q, int n_kv, int head_dim, int64_t max_ctx) {
  const int G = n_q / n_kv;
  const int pp = 4096 / (G * head_dim);
  // small calls (few positions over all sequences and key/value heads) take
  // blocks of at most 16 positions: more, shorter blocks in flight (Llama-3.2-1B
  // heads at batch 1: context 512 8.2 -> 7.7 us, 8192 11.5 -> 11.2); larger
  // ones keep up to 32 (at 32768 positions 16 was 21.9 against 20.6 us)
  const bool short_blocks = static_cast<int64_t>(batch) * n_kv * max_ctx <= 65536;
  const int cap = short_blocks ? 16 : 64;
  const int bpc = std::min(G * head_dim >= 1024 ? 8 : G >= 8 ? 16 : 32, cap);
  const int bp = std::max(pp, std::min(bpc, 131072 / (G * G * head_dim)));
  const int64_t unit = static_cast<int64_t>(kAttnWaves) * bp;       // one block per wave
  const int64_t units = (max_ctx + unit - 1) / unit;
  const int64_t want = std::max<int64_t>(1, QGEMV_ATTN_TARGET_WGS / std::max(1, batch * n_kv));
  const int64_t by_len = std::max<int64_t>(1, units / QGEMV_ATTN_MIN_BLOCKS);
  AttnPlan p;
  p.splits = static_cast<int>(std::min<int64_t>(std::min<int64_t>(by_len, want), kMaxSplits));
  const int64_t per = (units + p.splits - 1) / p.splits;
  p.positions = static_cast<int>(per * unit);
  p.splits = static_cast<int>((max_ctx + p.positions - 1) / p.positions);
  p.part_bytes = p.splits > 1 ? static_cast<size_t>(batch) * n_kv * p.splits * (2 * G + G * head_dim) * 4 : 0;
  p.short_blocks = short_blocks;
  return p;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_attn_d<64>(a, stream);
  return launch_attn_d<128>(a, stream);
}

}  // namespace qgemv
