// attn_bwd.hip -- causal attention backward for gfx950 (bf16 MFMA, fp32 accumulation).
//
// Gradients of sum(O * dO) for O = softmax(scale * Q K^T + causal mask) V, the
// backward pass the example program of "Context Parallelism" (Ultralytics
// glossary, "Praktische Anwendung und Kompromisse") runs after its causal
// attention call.  P is recomputed from Q, K and the forward's LSE:
//   Dv_i = <dO_i, O_i>,  P_ij = exp(scale <q_i, k_j> - LSE_i),
//   dS_ij = P_ij (<dO_i, v_j> - Dv_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j.
// dK, dV of a key/value head sum over the query heads that read it.
//
// Three kernels, none of them with atomics (results are deterministic):
//  * bwd_delta: Dv per query row, HBM bound.
//  * bwd_dkdv: a workgroup owns 128 keys of one key/value head (4 waves x 32
//    keys, K and V of its keys resident in registers as MFMA operands) and
//    walks every query tile that can see them, for each query head of the
//    group.  Per tile Q and dO are staged in LDS twice, row-major for the
//    S = Q K^T and dP = dO V^T products and transposed for the
//    dV^T += dO^T P and dK^T += Q^T dS products.  Query rows are fed to the
//    MFMA in the pi order, so P and dS leave the accumulators already in the
//    operand layout of the next product.
//  * bwd_dq: like the forward, a workgroup owns query rows (the heads of a
//    group packed together), walks the key tiles, recomputes S^T and
//    dP^T = V dO^T, and accumulates dQ^T += K^T dS^T.  K is staged both
//    row-major and transposed.
// dQ by a separate pass costs two recomputed products (7 contractions instead
// of 5) but avoids fp32 atomic traffic proportional to N^2 / tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace lcattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// Dv_i = <dO_i, O_i> (fp32), one thread per 8 elements
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ d_o,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int U = D / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = idx / U;
  const int u = (int)(idx % U);
  float s = 0.f;
  if (row < rows) {
    const u32x4 x = ld_global16(o + row * D + 8 * u);
    const u32x4 y = ld_global16(d_o + row * D + 8 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
      s += __uint_as_float(x[e] & 0xFFFF0000u) * __uint_as_float(y[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int off = U / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && u == 0) delta[row] = s;
}

// Stage a 64-row x D tile (rows [r0, r0+64) of a [rows_total, D] bf16 matrix)
// into LDS twice: row-major (rows read in pi order) and transposed (D rows of
// 64 columns).  One 4-row x 8-column block per thread.  Rows past rows_total
// are zero.
template <int D>
struct TileIO {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int T_ROW_BYTES = 64 * 2;
  static constexpr int BLOCKS = 16 * (D / 8);  // 4-row x 8-col blocks
  static_assert(BLOCKS <= kThreads, "one block per thread at most");

  __device__ static void load(const uint16_t* base, long long r0, long long rows_total, int tid, u32x4 reg[4]) {
    if (tid < BLOCKS) {
      const int dq = tid % (D / 8), kq = tid / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long row = r0 + 4 * kq + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < rows_total) x = ld_global16(base + row * D + 8 * dq);
        reg[r] = x;
      }
    }
  }
  __device__ static void store_rows(unsigned char* lds, int tid, const u32x4 reg[4]) {
    if (tid < BLOCKS) {
      const int dq = tid % (D / 8), kq = tid / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * kq + r;
        st_lds16(lds, row * ROW_BYTES + ((dq ^ swz_rows_pi(row)) << 4), reg[r]);
      }
    }
  }
  __device__ static void store_cols(unsigned char* lds, int tid, const u32x4 reg[4]) {
    if (tid < BLOCKS) {
      const int dq = tid % (D / 8), kq = tid / (D / 8);
      u32x2 cols[8];
      transpose4x8(reg, cols);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * dq + e;
        st_lds8(lds, d * T_ROW_BYTES + (((kq >> 1) ^ swz_cols(d)) << 4) + ((kq & 1) << 3), cols[e]);
      }
    }
  }
  // A operand of a product reducing over D: row (block-local, already in pi
  // order) and reduction step t.
  __device__ static bf16x8 rows_frag(const unsigned char* lds, int row, int t, int grp) {
    return as_bf16x8(ld_lds16(lds, row * ROW_BYTES + (((2 * t + grp) ^ swz_rows_pi(row)) << 4)));
  }
  // A operand of a product reducing over the 64 tile rows: row d of the
  // transposed tile, 8 consecutive tile rows starting at 8 * unit.
  __device__ static bf16x8 cols_frag(const unsigned char* lds, int d, int unit) {
    return as_bf16x8(ld_lds16(lds, d * T_ROW_BYTES + ((unit ^ swz_cols(d)) << 4)));
  }
};

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one key/value head
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int BQ = 64;     // queries per tile
  constexpr int BK = 128;    // keys per workgroup
  using IO = TileIO<D>;
  constexpr int TILE = BQ * D * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TILE + 2 * BQ * 4];
  unsigned char* q_rows = smem;
  unsigned char* q_cols = smem + TILE;
  unsigned char* o_rows = smem + 2 * TILE;   // dO
  unsigned char* o_cols = smem + 3 * TILE;
  float* lse_t = reinterpret_cast<float*>(smem + 4 * TILE);  // LSE * log2(e), +inf past N
  float* dv_t = lse_t + BQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const long long N = a.N;
  const long long bz = blockIdx.z;
  const int kvh = blockIdx.y;
  const long long kt0 = (long long)blockIdx.x * BK;
  const long long kw0 = kt0 + 32 * wave;       // this wave's first key
  const long long key = kw0 + c;               // this lane's key
  const float sl = a.scale * kLog2e;

  const uint16_t* kbase = a.k + (bz * a.Hkv + kvh) * N * D;
  const uint16_t* vbase = a.v + (bz * a.Hkv + kvh) * N * D;

  // K and V rows of this lane's key as B operands (reduction over D)
  bf16x8 kf[KT], vf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < N) {
      x = ld_global16(kbase + key * D + 16 * t + 8 * grp);
      y = ld_global16(vbase + key * D + 16 * t + 8 * grp);
    }
    kf[t] = as_bf16x8(x);
    vf[t] = as_bf16x8(y);
  }

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dk_acc[db][v] = 0.f;
      dv_acc[db][v] = 0.f;
    }

  const long long first_tile = a.causal ? kt0 / BQ : 0;
  const long long n_qt = (N + BQ - 1) / BQ;
  const long long tiles_per_head = n_qt - first_tile;
  const long long total = tiles_per_head * a.G;

  u32x4 qreg[4], oreg[4];
  float lse_reg = 0.f;
  auto load = [&](long long it) {
    const int hh = (int)(it / tiles_per_head);
    const long long qt = first_tile + it % tiles_per_head;
    const int h = kvh * a.G + hh;
    const long long hb = (bz * a.Hq + h) * N;
    IO::load(a.q + hb * D, qt * BQ, N, tid, qreg);
    IO::load(a.d_o + hb * D, qt * BQ, N, tid, oreg);
    if (tid < 2 * BQ) {
      const long long row = qt * BQ + (tid & (BQ - 1));
      if (tid < BQ) lse_reg = row < N ? a.lse[hb + row] * kLog2e : INFINITY;
      else lse_reg = row < N ? a.delta[hb + row] : 0.f;
    }
  };
  auto store = [&]() {
    IO::store_rows(q_rows, tid, qreg);
    IO::store_cols(q_cols, tid, qreg);
    IO::store_rows(o_rows, tid, oreg);
    IO::store_cols(o_cols, tid, oreg);
    if (tid < 2 * BQ) lse_t[tid] = lse_reg;  // lse_t and dv_t are adjacent
  };

  if (total > 0) load(0);
  for (long long it = 0; it < total; ++it) {
    __syncthreads();  // previous tile's readers are done
    store();
    __syncthreads();
    if (it + 1 < total) load(it + 1);
    const long long qt0 = (first_tile + it % tiles_per_head) * BQ;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const long long qb0 = qt0 + qb * 32;
      // all 32 queries of the block precede every key of the wave: nothing visible
      if (a.causal && qb0 + 31 < kw0) continue;
      if (qb0 >= N || kw0 >= N) continue;
      f32x16 s, dp;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[v] = 0.f;
        dp[v] = 0.f;
      }
      const int arow = qb * 32 + swap_bits23(c);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        s = mfma32x32x16(IO::rows_frag(q_rows, arow, t, grp), kf[t], s);
        dp = mfma32x32x16(IO::rows_frag(o_rows, arow, t, grp), vf[t], dp);
      }
      const bool need_mask = a.causal && (qb0 < kw0 + 31);
      bf16x8 pb[2], db16[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = qb * 32 + 16 * u + 8 * grp;  // tile rows of registers 8u..8u+7
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_t + r0);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_t + r0 + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dv_t + r0);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dv_t + r0 + 4);
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lv = e < 4 ? l0[e] : l1[e - 4];
          const float dvv = e < 4 ? d0[e] : d1[e - 4];
          float pe = fast_exp2(__builtin_fmaf(s[8 * u + e], sl, -lv));
          if (need_mask && qt0 + r0 + e < key) pe = 0.f;
          p[e] = pe;
          ds[e] = pe * (dp[8 * u + e] - dvv);
        }
        pb[u] = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        db16[u] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
#pragma unroll
      for (int dbk = 0; dbk < DB; ++dbk) {
        const int d = dbk * 32 + c;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int unit = 4 * qb + 2 * u + grp;
          dv_acc[dbk] = mfma32x32x16(IO::cols_frag(o_cols, d, unit), pb[u], dv_acc[dbk]);
          dk_acc[dbk] = mfma32x32x16(IO::cols_frag(q_cols, d, unit), db16[u], dk_acc[dbk]);
        }
      }
    }
  }

  if (key < N) {
    const long long base = ((bz * a.Hkv + kvh) * N + key) * D;
#pragma unroll
    for (int dbk = 0; dbk < DB; ++dbk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dbk * 32 + 8 * j + 4 * grp;
        *reinterpret_cast<u32x2*>(a.dk + base + d) =
            pack_bf16x4_bits(dk_acc[dbk][4 * j] * a.scale, dk_acc[dbk][4 * j + 1] * a.scale,
                             dk_acc[dbk][4 * j + 2] * a.scale, dk_acc[dbk][4 * j + 3] * a.scale);
        *reinterpret_cast<u32x2*>(a.dv + base + d) =
            pack_bf16x4_bits(dv_acc[dbk][4 * j], dv_acc[dbk][4 * j + 1], dv_acc[dbk][4 * j + 2],
                             dv_acc[dbk][4 * j + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = query rows of HP heads sharing a key/value head
// ---------------------------------------------------------------------------
template <int D, int HP>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a, int n_qtiles) {
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int BN = 64;
  constexpr int SPAN = (kWaves / HP) * 32;
  using IO = TileIO<D>;
  constexpr int TILE = BN * D * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[3 * TILE];
  unsigned char* k_rows = smem;
  unsigned char* k_cols = smem + TILE;
  unsigned char* v_rows = smem + 2 * TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const long long N = a.N;
  const long long bz = blockIdx.z;
  const int qt = n_qtiles - 1 - (int)blockIdx.x;  // longest causal rows first
  const int h = blockIdx.y * HP + (wave % HP);
  const int kvh = (blockIdx.y * HP) / a.G;
  const long long q_start = (long long)qt * SPAN;
  const long long wq0 = q_start + (long long)(wave / HP) * 32;
  const long long qrow = wq0 + c;
  const float sl = a.scale * kLog2e;
  const long long hb = (bz * a.Hq + h) * N;

  bf16x8 qf[KT], of[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      x = ld_global16(a.q + (hb + qrow) * D + 16 * t + 8 * grp);
      y = ld_global16(a.d_o + (hb + qrow) * D + 16 * t + 8 * grp);
    }
    qf[t] = as_bf16x8(x);
    of[t] = as_bf16x8(y);
  }
  const float lse2 = qrow < N ? a.lse[hb + qrow] * kLog2e : INFINITY;
  const float dvv = qrow < N ? a.delta[hb + qrow] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

  long long kv_end = N;
  if (a.causal) kv_end = min(N, q_start + SPAN);
  const int n_tiles = (int)((kv_end + BN - 1) / BN);
  const long long wq_last = min(wq0 + 32, N) - 1;
  const bool wave_live = wq0 < N;

  const uint16_t* kbase = a.k + (bz * a.Hkv + kvh) * N * D;
  const uint16_t* vbase = a.v + (bz * a.Hkv + kvh) * N * D;
  u32x4 kreg[4], vreg[4];
  auto load = [&](int j) {
    IO::load(kbase, (long long)j * BN, N, tid, kreg);
    IO::load(vbase, (long long)j * BN, N, tid, vreg);
  };
  auto store = [&]() {
    IO::store_rows(k_rows, tid, kreg);
    IO::store_cols(k_cols, tid, kreg);
    IO::store_rows(v_rows, tid, vreg);
  };

  if (n_tiles > 0) load(0);
  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();
    store();
    __syncthreads();
    if (j + 1 < n_tiles) load(j + 1);
    const long long kt = (long long)j * BN;
    if (!wave_live || (a.causal && kt > wq_last)) continue;
    const bool need_mask = (kt + BN > N) || (a.causal && kt + BN - 1 > wq0);
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[v] = 0.f;
        dp[v] = 0.f;
      }
      const int arow = kb * 32 + swap_bits23(c);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        s = mfma32x32x16(IO::rows_frag(k_rows, arow, t, grp), qf[t], s);
        dp = mfma32x32x16(IO::rows_frag(v_rows, arow, t, grp), of[t], dp);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 8 * u + e;
          float p = fast_exp2(__builtin_fmaf(s[v], sl, -lse2));
          if (need_mask) {
            const long long kk = kt + kb * 32 + acc_row_pi(v, grp);
            if (kk >= N || (a.causal && kk > qrow)) p = 0.f;
          }
          ds[e] = p * (dp[v] - dvv);
        }
        dsb[2 * kb + u] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + c;
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[db] = mfma32x32x16(IO::cols_frag(k_cols, d, 2 * u + grp), dsb[u], acc[db]);
    }
  }

  if (qrow < N) {
    const long long base = (hb + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * grp;
        *reinterpret_cast<u32x2*>(a.dq + base + d) =
            pack_bf16x4_bits(acc[db][4 * j] * a.scale, acc[db][4 * j + 1] * a.scale, acc[db][4 * j + 2] * a.scale,
                             acc[db][4 * j + 3] * a.scale);
      }
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int B, hipStream_t stream) {
  const long long rows = (long long)B * a.Hq * a.N;
  const long long threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.o,
                     a.d_o, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)((a.N + 127) / 128), (unsigned)a.Hkv, (unsigned)B),
                     dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int HP = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);
  const long long span = (kWaves / HP) * 32;
  const int n_qt = (int)((a.N + span - 1) / span);
  dim3 grid((unsigned)n_qt, (unsigned)(a.Hq / HP), (unsigned)B);
  if (HP == 4)
    hipLaunchKernelGGL((bwd_dq_kernel<D, 4>), grid, dim3(kThreads), 0, stream, a, n_qt);
  else if (HP == 2)
    hipLaunchKernelGGL((bwd_dq_kernel<D, 2>), grid, dim3(kThreads), 0, stream, a, n_qt);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, 1>), grid, dim3(kThreads), 0, stream, a, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a, int B, int D, hipStream_t stream) {
  return D == 64 ? launch_d<64>(a, B, stream) : launch_d<128>(a, B, stream);
}

}  // namespace lcattn
