// merge.hip -- log-sum-exp merge of partial attention results.
//
// "Context Parallelism" (Ultralytics glossary), section "So funktioniert
// Kontextparallelität": in ring attention each device computes partial
// attention of its queries against one KV block at a time, and the combined
// result equals attention over the whole sequence.  For disjoint key blocks b
// with partial output O_b and log-sum-exp LSE_b, the softmax over the union
// renormalises by the summed exponentials:
//   LSE = M + ln sum_b exp(LSE_b - M),  M = max_b LSE_b,
//   O   = sum_b exp(LSE_b - LSE) O_b.
// Parts with LSE_b = -inf weigh zero; rows empty in every part give O = 0,
// LSE = -inf.  A part with a NaN LSE makes the merged row NaN.
//
// Kernel: HBM bound.  One thread per (row, 8 consecutive head-dim elements);
// the n_parts LSE values of a row are read by all of the row's threads (they
// hit in cache), then n_parts 16- or 32-byte slices are streamed and one
// 16-byte bf16 slice is written.
#include "device_common.hpp"
#include "launch.hpp"
#include "trace.hpp"

namespace lcattn {

constexpr int kMergeThreads = 256;

// Parts of a row's split forward that hold work (the ranges below the last
// visible key tile of the row's query tile); n_parts_max without geometry.
__device__ __forceinline__ int parts_of_row(const MergeSplits& sp, long long row, int n_parts_max) {
  if (sp.span <= 0) return n_parts_max;
  // ranges past the query tile's last visible key wrote no partial (the bound
  // uses the tile's last row, as the forward does)
  const long long qt = (row % sp.Nq) / sp.span;
  const long long q_last = min((qt + 1) * sp.span, sp.Nq) - 1;
  long long kv_end = sp.Nk;
  if (sp.causal) kv_end = max(0LL, min(sp.Nk, sp.dpos + q_last + 1));
  const long long tiles = (kv_end + sp.key_tile - 1) / sp.key_tile;
  return (int)min((long long)n_parts_max, (tiles + sp.split_tiles - 1) / sp.split_tiles);
}

// One 8-element slice of part b of a row, as floats.
template <int D, bool PART_F32>
__device__ __forceinline__ void load_slice(const void* o_parts, long long off, float (&x)[8]) {
  if (PART_F32) {
    const float* p = static_cast<const float*>(o_parts) + off;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = x0[e];
      x[4 + e] = x1[e];
    }
  } else {
    const u32x4 w = ld_global16(static_cast<const uint16_t*>(o_parts) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

// LSE merge of one row slice over its n parts and, when has_run, a running
// part (lse lr, slice xr): acc = sum_b exp(lse_b - LSE) part_b, out_lse =
// LSE.  Parts of weight 0 (empty rows, LSE = -inf) are skipped.  FAST (small
// merges, too few waves to hide memory latency) with up to kFastParts parts:
// every LSE and every slice is loaded before any is used, so a row costs one
// round trip to memory instead of one per part; large merges keep the loop,
// whose fewer registers leave more waves in flight.
constexpr int kFastParts = 8;
template <int D, bool PART_F32, bool FAST>
__device__ __forceinline__ void merge_row(const void* o_parts, const float* lse_parts, int n, long long rows,
                                          long long row, int u, bool has_run, float lr, const float (&xr)[8],
                                          float (&acc)[8], float& out_lse) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  out_lse = -INFINITY;
  float m = has_run ? lr : -INFINITY;
  bool nan = has_run && lr != lr;
  if (FAST && n <= kFastParts) {
    float lb[kFastParts];
    float x[kFastParts][8];
#pragma unroll
    for (int b = 0; b < kFastParts; ++b)
      if (b < n) lb[b] = lse_parts[(long long)b * rows + row];
#pragma unroll
    for (int b = 0; b < kFastParts; ++b)
      if (b < n) load_slice<D, PART_F32>(o_parts, ((long long)b * rows + row) * D + 8 * u, x[b]);
#pragma unroll
    for (int b = 0; b < kFastParts; ++b)
      if (b < n) {
        nan |= lb[b] != lb[b];
        m = fmaxf(m, lb[b]);  // ignores NaN operands
      }
    // a NaN part (NaN inputs reached it) makes the row NaN, also when every
    // other part is empty: reference 0 lets exp(NaN - 0) carry it through
    if (nan && m == -INFINITY) m = 0.f;
    if (m == -INFINITY) return;
    float wr = has_run ? fast_exp2((lr - m) * kLog2e) : 0.f;
    float w[kFastParts];
    float tot = wr;
#pragma unroll
    for (int b = 0; b < kFastParts; ++b)
      if (b < n) {
        w[b] = fast_exp2((lb[b] - m) * kLog2e);
        tot += w[b];
      }
    const float inv = 1.0f / tot;
    out_lse = m + fast_log2(tot) * kLn2;
    wr *= inv;
    if (has_run && wr != 0.f)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wr * xr[e];
#pragma unroll
    for (int b = 0; b < kFastParts; ++b)
      if (b < n) {
        const float wb = w[b] * inv;
        if (wb != 0.f)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += wb * x[b][e];
      }
    return;
  }
  for (int b = 0; b < n; ++b) {
    const float lb = lse_parts[(long long)b * rows + row];
    nan |= lb != lb;
    m = fmaxf(m, lb);
  }
  if (nan && m == -INFINITY) m = 0.f;
  if (m == -INFINITY) return;
  float tot = has_run ? fast_exp2((lr - m) * kLog2e) : 0.f;
  for (int b = 0; b < n; ++b) tot += fast_exp2((lse_parts[(long long)b * rows + row] - m) * kLog2e);
  const float inv = 1.0f / tot;
  out_lse = m + fast_log2(tot) * kLn2;
  if (has_run) {
    const float wr = fast_exp2((lr - m) * kLog2e) * inv;
    if (wr != 0.f)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wr * xr[e];
  }
  for (int b = 0; b < n; ++b) {
    const float w = fast_exp2((lse_parts[(long long)b * rows + row] - m) * kLog2e) * inv;
    if (w == 0.f) continue;
    float x[8];
    load_slice<D, PART_F32>(o_parts, ((long long)b * rows + row) * D + 8 * u, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * x[e];
  }
}

template <int D, bool PART_F32, bool FAST>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const void* __restrict__ o_parts,
                                                              const float* __restrict__ lse_parts,
                                                              int n_parts_max, long long rows,
                                                              uint16_t* __restrict__ o,
                                                              float* __restrict__ lse, MergeSplits sp) {
  constexpr int U = D / 8;  // 8-element slices per row
  const long long idx = (long long)blockIdx.x * kMergeThreads + threadIdx.x;
  const long long row = idx / U;
  const int u = (int)(idx % U);
  if (row >= rows) return;
  const int n_parts = parts_of_row(sp, row, n_parts_max);
  float acc[8], out_lse;
  const float none[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  merge_row<D, PART_F32, FAST>(o_parts, lse_parts, n_parts, rows, row, u, false, 0.f, none, acc, out_lse);
  const bf16x8 r = pack_bf16x8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
  st_global16(o + row * D + 8 * u, as_u32x4(r));
  if (u == 0) lse[row] = out_lse;
}

// The same merge with the running result of a streaming ring as one more
// part: o_run, lse_run (fp32, the attention over the earlier KV blocks) are
// read unless `first`, and overwritten with the merged result; o_final, if
// set, receives it rounded to bf16.  A row's threads are consecutive lanes
// of one wave (D / 8 of 64), so every lane reads lse_run[row] before the
// lane of slice 0 writes it.
template <int D, bool FAST>
__global__ __launch_bounds__(kMergeThreads) void merge_into_kernel(const float* __restrict__ o_parts,
                                                                   const float* __restrict__ lse_parts,
                                                                   int n_parts_max, long long rows,
                                                                   float* __restrict__ o_run,
                                                                   float* __restrict__ lse_run, int first,
                                                                   uint16_t* __restrict__ o_final, MergeSplits sp) {
  constexpr int U = D / 8;
  static_assert(64 % U == 0, "a row's threads lie in one wave");
  const long long idx = (long long)blockIdx.x * kMergeThreads + threadIdx.x;
  const long long row = idx / U;
  const int u = (int)(idx % U);
  if (row >= rows) return;
  const int n_parts = parts_of_row(sp, row, n_parts_max);
  const long long off = row * D + 8 * u;
  float xr[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lr = -INFINITY;
  if (!first) {
    lr = lse_run[row];
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(o_run + off);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(o_run + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xr[e] = x0[e];
      xr[4 + e] = x1[e];
    }
  }
  float acc[8], out_lse;
  merge_row<D, true, FAST>(o_parts, lse_parts, n_parts, rows, row, u, !first, lr, xr, acc, out_lse);
  *reinterpret_cast<f32x4*>(o_run + off) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4*>(o_run + off + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  if (o_final) {
    const bf16x8 r = pack_bf16x8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
    st_global16(o_final + off, as_u32x4(r));
  }
  if (u == 0) lse_run[row] = out_lse;
}

// Merges with fewer than 4 waves per SIMD of the GPU (1024 SIMDs) are
// latency-bound: they take the kernel that loads all of a row's parts at once.
static bool merge_fast(long long threads) { return threads / 64 < 4LL * 1024; }

hipError_t launch_merge_into(const float* o_parts, const float* lse_parts, int n_parts, const MergeSplits& sp,
                             float* o_run, float* lse_run, bool first, uint16_t* o_final, long long rows, int D,
                             hipStream_t stream) {
  const long long threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + kMergeThreads - 1) / kMergeThreads);
  const bool fast = merge_fast(threads);
#define LCATTN_MERGE_INTO(DD, FF)                                                                              \
  LCATTN_LAUNCH("merge_into_kernel", (merge_into_kernel<DD, FF>), dim3(blocks), dim3(kMergeThreads), 0, stream, \
                o_parts, lse_parts, n_parts, rows, o_run, lse_run, first ? 1 : 0, o_final, sp)
  if (D == 64) {
    if (fast) LCATTN_MERGE_INTO(64, true); else LCATTN_MERGE_INTO(64, false);
  } else {
    if (fast) LCATTN_MERGE_INTO(128, true); else LCATTN_MERGE_INTO(128, false);
  }
#undef LCATTN_MERGE_INTO
  return hipGetLastError();
}

hipError_t launch_partial_merge(const void* o_parts, bool parts_f32, const float* lse_parts, int n_parts,
                                uint16_t* o, float* lse, long long rows, int D, hipStream_t stream,
                                const MergeSplits* splits) {
  const long long threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + kMergeThreads - 1) / kMergeThreads);
  const MergeSplits sp = splits ? *splits : MergeSplits{};
  const bool fast = merge_fast(threads);
#define LCATTN_MERGE(DD, F32, FF)                                                                        \
  LCATTN_LAUNCH("merge_kernel", (merge_kernel<DD, F32, FF>), dim3(blocks), dim3(kMergeThreads), 0, stream, \
                o_parts, lse_parts, n_parts, rows, o, lse, sp)
  if (D == 64) {
    if (parts_f32) {
      if (fast) LCATTN_MERGE(64, true, true); else LCATTN_MERGE(64, true, false);
    } else {
      if (fast) LCATTN_MERGE(64, false, true); else LCATTN_MERGE(64, false, false);
    }
  } else {
    if (parts_f32) {
      if (fast) LCATTN_MERGE(128, true, true); else LCATTN_MERGE(128, true, false);
    } else {
      if (fast) LCATTN_MERGE(128, false, true); else LCATTN_MERGE(128, false, false);
    }
  }
#undef LCATTN_MERGE
  return hipGetLastError();
}

}  // namespace lcattn
