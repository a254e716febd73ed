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

// One tensor of a batched relayout, as the kernel sees it (passed by value).
struct RelayoutJob {
  const void* in;
  void* out;
  unsigned A, Bn, rep;
  unsigned nbt, nat;  // b-tiles, a-tiles
  unsigned first;  // first workgroup of this job
};
struct RelayoutBatch {
  RelayoutJob job[kMaxRelayoutBatch];
  int n;
  unsigned units_log2, ta_log2, tb_log2;
  // tile order within a job: a-tiles fastest (else b-tiles fastest); the
  // launcher picks the order that walks the token-major side sequentially
  unsigned a_fast;
};

// out[a * rep + i, b, :] = in[b, a, :] (i < rep) for rows of 2^units_log2
// 16-byte units, a in [0, A), b in [0, Bn), for each job of a batch (the
// tensors that one exchange moves together, e.g. Q, K, V and dO): rep > 1
// replicates every a-row block (a key/value head shared by rep ranks).  The
// jobs' tiles are numbered one after another; job j owns workgroups
// [first, first + nat * nbt) and tile (a-tile, b-tile) = (w / nbt, w % nbt)
// of its local index w.  TA = 2^ta_log2, TB = 2^tb_log2 rows.
// A * rep * Bn * units < 2^32 per job is checked on the host.
__global__ __launch_bounds__(kRelayoutThreads) void transpose_rows_kernel(RelayoutBatch jobs) {
  // the job of this workgroup (uniform: a scalar scan of at most 8 entries)
  int j = 0;
  while (j + 1 < jobs.n && blockIdx.x >= jobs.job[j + 1].first) ++j;
  const RelayoutJob& J = jobs.job[j];
  const u32x4* __restrict__ in = static_cast<const u32x4*>(J.in);
  u32x4* __restrict__ out = static_cast<u32x4*>(J.out);
  const unsigned A = J.A, Bn = J.Bn, rep = J.rep, nbt = J.nbt;
  const unsigned units_log2 = jobs.units_log2, ta_log2 = jobs.ta_log2, tb_log2 = jobs.tb_log2;
  const unsigned w = blockIdx.x - J.first;
  const unsigned bt = jobs.a_fast ? w / J.nat : w % nbt, at = jobs.a_fast ? w % J.nat : w / nbt;
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
      dst[i] = ((a * rep * Bn + b) << units_log2) | (k & umask);
      if (ok[i]) vals[i] = __builtin_nontemporal_load(in + (((b * A + a) << units_log2) | (k & umask)));
    }
    for (unsigned c = 0; c < rep; ++c) {
      const unsigned step = (c * Bn) << units_log2;  // c-th copy of the a-row block
#pragma unroll
      for (int i = 0; i < kRelayoutUnroll; ++i)
        if (ok[i]) __builtin_nontemporal_store(vals[i], out + dst[i] + step);
    }
  }
}

// out[b, a, :] = sum over i < rep of in[a * rep + i, b, :] for rows of D
// elements (bf16 or fp32 in, summed in fp32 in order i = 0, 1, ..., bf16 out
// rounded to nearest even): the inverse exchange of gradients of a
// key/value head that rep ranks shared (rep = 1: the transpose with a
// conversion).  One thread per 8 output elements.
template <bool IN_F32>
__global__ __launch_bounds__(256) void sum_replicas_kernel(const void* __restrict__ in, uint16_t* __restrict__ out,
                                                           long long A, long long Bn, int D, int rep) {
  const long long units = (long long)D / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;  // over Bn * A * units
  if (idx >= Bn * A * units) return;
  const long long u = idx % units, ab = idx / units;
  const long long a = ab % A, b = ab / A;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < rep; ++i) {
    const long long src = ((a * rep + i) * Bn + b) * D + 8 * u;
    if (IN_F32) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(in) + src);
      const f32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += x[e];
        acc[4 + e] += y[e];
      }
    } else {
      const u32x4 x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(in) + src));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16);
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xFFFF0000u);
      }
    }
  }
  const u32x2 lo = pack_bf16x4_bits(acc[0], acc[1], acc[2], acc[3]);
  const u32x2 hi = pack_bf16x4_bits(acc[4], acc[5], acc[6], acc[7]);
  const u32x4 o = {lo[0], lo[1], hi[0], hi[1]};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + idx * 8));
}

hipError_t launch_transpose_rows_batch(const TransposeJob* jobs, int n, unsigned row_bytes, bool a_fast,
                                       hipStream_t stream) {
  unsigned units = row_bytes / 16, lg = 0;
  while ((1u << lg) < units) ++lg;
  // 4 x 4 rows, with more b rows when rows are short, so a tile is at least
  // one unit per thread
  const unsigned ta_lg = 2;
  unsigned tb_lg = 2;
  while ((1u << (ta_lg + tb_lg + lg)) < (unsigned)kRelayoutThreads) ++tb_lg;
  RelayoutBatch b{};
  b.n = n;
  b.units_log2 = lg;
  b.ta_log2 = ta_lg;
  b.tb_log2 = tb_lg;
  b.a_fast = a_fast ? 1u : 0u;
  unsigned long long blocks = 0;
  for (int j = 0; j < n; ++j) {
    RelayoutJob& J = b.job[j];
    J.in = jobs[j].in;
    J.out = jobs[j].out;
    J.A = jobs[j].A;
    J.Bn = jobs[j].Bn;
    J.rep = jobs[j].rep;
    J.nbt = (J.Bn + (1u << tb_lg) - 1) >> tb_lg;
    J.nat = (J.A + (1u << ta_lg) - 1) >> ta_lg;
    J.first = (unsigned)blocks;
    blocks += (unsigned long long)J.nbt * J.nat;
  }
  if (blocks == 0) return hipSuccess;
  if (blocks > 0xFFFFFFFFull) return hipErrorInvalidValue;
  LCATTN_LAUNCH("transpose_rows_kernel", transpose_rows_kernel, dim3((unsigned)blocks), dim3(kRelayoutThreads), 0,
                stream, b);
  return hipGetLastError();
}

hipError_t launch_sum_replicas(const void* in, bool in_f32, uint16_t* out, long long A, long long Bn, int D, int rep,
                               hipStream_t stream) {
  const long long threads = A * Bn * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (in_f32)
    LCATTN_LAUNCH("sum_replicas_kernel", (sum_replicas_kernel<true>), grid, dim3(256), 0, stream, in, out, A, Bn, D,
                  rep);
  else
    LCATTN_LAUNCH("sum_replicas_kernel", (sum_replicas_kernel<false>), grid, dim3(256), 0, stream, in, out, A, Bn, D,
                  rep);
  return hipGetLastError();
}

}  // namespace lcattn
