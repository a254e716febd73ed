// relayout.hip -- the Ulysses sequence<->head exchange's data movement on one GPU.
//
// "Million-Token-Kontexte im Training ..." (section "Ulysses: Die Sequenz als
// Verteilungseinheit") and "Ulysses Sequence Parallelism: как тренировать
// модели с контекстом в миллион токенов" (section "Как работает Ulysses:
// технические детали") split the sequence into equal contiguous parts and use
// an all-to-all so that each GPU ends up with the whole sequence for a subset
// of the heads.  With contiguous token shards and contiguous head groups,
// [P, N/P, H, D] -> [P, H/P, N, D] is the transpose [N, H, D] -> [H, N, D] of
// (token, head) rows of D elements, and the inverse is the transpose back.
//
// Kernel: a pure copy of 16-byte units, HBM bound.  Work is laid out in output
// order so each wave stores 1 KiB contiguous; the matching loads are whole
// rows (D*elem bytes, 128 or 256 B) that are contiguous in the source.  Each
// thread keeps kUnroll loads in flight before its stores; stores are
// non-temporal because the output is not re-read by this kernel.
#include "device_common.hpp"
#include "launch.hpp"
#include "trace.hpp"

namespace lcattn {

constexpr int kRelayoutThreads = 256;
constexpr int kRelayoutUnroll = 4;

// out[a, b, :] = in[b, a, :] for rows of `units` 16-byte units.
// a in [0, A), b in [0, Bn).  A * Bn * units < 2^32 is checked on the host.
__global__ __launch_bounds__(kRelayoutThreads) void transpose_rows_kernel(const u32x4* __restrict__ in,
                                                                            u32x4* __restrict__ out,
                                                                            unsigned A, unsigned Bn,
                                                                            unsigned units_log2,
                                                                            unsigned total) {
  const unsigned per_block = kRelayoutThreads * kRelayoutUnroll;
  const unsigned base = blockIdx.x * per_block + threadIdx.x;
  const unsigned umask = (1u << units_log2) - 1u;
  u32x4 vals[kRelayoutUnroll];
  unsigned dst[kRelayoutUnroll];
#pragma unroll
  for (int i = 0; i < kRelayoutUnroll; ++i) {
    const unsigned idx = base + i * kRelayoutThreads;
    dst[i] = idx;
    if (idx < total) {
      const unsigned u = idx & umask;
      const unsigned row = idx >> units_log2;  // output row = a * Bn + b
      const unsigned a = row / Bn;
      const unsigned b = row - a * Bn;
      const unsigned src = ((b * A + a) << units_log2) | u;
      vals[i] = __builtin_nontemporal_load(in + src);
    }
  }
#pragma unroll
  for (int i = 0; i < kRelayoutUnroll; ++i) {
    if (dst[i] < total) __builtin_nontemporal_store(vals[i], out + dst[i]);
  }
}

hipError_t launch_transpose_rows(const void* in, void* out, unsigned A, unsigned Bn, unsigned row_bytes,
                                 hipStream_t stream) {
  unsigned units = row_bytes / 16, lg = 0;
  while ((1u << lg) < units) ++lg;
  const unsigned total = A * Bn * units;
  const unsigned per_block = kRelayoutThreads * kRelayoutUnroll;
  const unsigned blocks = (total + per_block - 1) / per_block;
  LCATTN_LAUNCH("transpose_rows_kernel", transpose_rows_kernel, dim3(blocks), dim3(kRelayoutThreads), 0, stream,
                     static_cast<const u32x4*>(in), static_cast<u32x4*>(out), A, Bn, lg, total);
  return hipGetLastError();
}

}  // namespace lcattn
