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
// Kernel: a pure copy of 16-byte units, HBM bound.  Each workgroup moves one
// tile of TA x TB rows (TA consecutive a, TB consecutive b), so that the
// rows it reads and the rows it writes both sit in a few small contiguous
// runs: with 256-byte rows a 4 x 4 tile reads four runs of 1 KiB and writes
// four runs of 1 KiB.  Measured on MI355X with the last-level cache flushed
// before every launch, this beats the row-at-a-time mapping (every wave
// writing 1 KiB contiguous, reading four rows 256 B apart in different
// places) by 5-10%.  Loads and stores are non-temporal: each byte is touched
// once, and cached loads measured markedly slower.
#include "device_common.hpp"
#include "launch.hpp"
#include "trace.hpp"

namespace lcattn {

constexpr int kRelayoutThreads = 256;
constexpr int kRelayoutUnroll = 4;

// out[a, b, :] = in[b, a, :] for rows of 2^units_log2 16-byte units, a in
// [0, A), b in [0, Bn).  Tile (a-tile, b-tile) = blockIdx.x split as
// (blockIdx.x / nbt, blockIdx.x % nbt); TA = 2^ta_log2, TB = 2^tb_log2 rows.
// A * Bn * units < 2^32 is checked on the host.
__global__ __launch_bounds__(kRelayoutThreads) void transpose_rows_kernel(const u32x4* __restrict__ in,
                                                                            u32x4* __restrict__ out,
                                                                            unsigned A, unsigned Bn,
                                                                            unsigned units_log2, unsigned ta_log2,
                                                                            unsigned tb_log2, unsigned nbt) {
  const unsigned bt = blockIdx.x % nbt, at = blockIdx.x / nbt;
  const unsigned a0 = at << ta_log2, b0 = bt << tb_log2;
  const unsigned umask = (1u << units_log2) - 1u, tbmask = (1u << tb_log2) - 1u;
  const unsigned per = 1u << (ta_log2 + tb_log2 + units_log2);  // units in the tile
  for (unsigned k0 = 0; k0 < per; k0 += kRelayoutThreads * kRelayoutUnroll) {
    u32x4 vals[kRelayoutUnroll];
    unsigned dst[kRelayoutUnroll];
    bool ok[kRelayoutUnroll];
#pragma unroll
    for (int i = 0; i < kRelayoutUnroll; ++i) {
      const unsigned k = k0 + i * kRelayoutThreads + threadIdx.x;
      const unsigned r = k >> units_log2;  // row in the tile, b fastest
      const unsigned a = a0 + (r >> tb_log2), b = b0 + (r & tbmask);
      ok[i] = k < per && a < A && b < Bn;
      dst[i] = ((a * Bn + b) << units_log2) | (k & umask);
      if (ok[i]) vals[i] = __builtin_nontemporal_load(in + (((b * A + a) << units_log2) | (k & umask)));
    }
#pragma unroll
    for (int i = 0; i < kRelayoutUnroll; ++i)
      if (ok[i]) __builtin_nontemporal_store(vals[i], out + dst[i]);
  }
}

hipError_t launch_transpose_rows(const void* in, void* out, unsigned A, unsigned Bn, unsigned row_bytes,
                                 hipStream_t stream) {
  unsigned units = row_bytes / 16, lg = 0;
  while ((1u << lg) < units) ++lg;
  // 4 x 4 rows, with more b rows when rows are short, so a tile is at least
  // one unit per thread
  const unsigned ta_lg = 2;
  unsigned tb_lg = 2;
  while ((1u << (ta_lg + tb_lg + lg)) < (unsigned)kRelayoutThreads) ++tb_lg;
  const unsigned nbt = (Bn + (1u << tb_lg) - 1) >> tb_lg;
  const unsigned nat = (A + (1u << ta_lg) - 1) >> ta_lg;
  LCATTN_LAUNCH("transpose_rows_kernel", transpose_rows_kernel, dim3(nbt * nat), dim3(kRelayoutThreads), 0, stream,
                static_cast<const u32x4*>(in), static_cast<u32x4*>(out), A, Bn, lg, ta_lg, tb_lg, nbt);
  return hipGetLastError();
}

}  // namespace lcattn
