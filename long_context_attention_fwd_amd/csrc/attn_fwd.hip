// attn_fwd.hip -- fused causal attention forward for gfx950 (bf16 MFMA, fp32 accumulation).
//
// Computes O = softmax(scale * Q K^T + causal mask) V and the per-row natural
// log-sum-exp, the call made by the example program of "Context Parallelism"
// (Ultralytics glossary), section "Praktische Anwendung und Kompromisse".  The
// mask uses global token positions (key k_pos0+j visible to query q_pos0+i iff
// k_pos0+j <= q_pos0+i), so a call restricted to one KV block is one ring
// step's partial attention (same page, "So funktioniert Kontextparallelität").
//
// Design (CDNA4, wave64):
//  * A workgroup is 4 waves.  Each wave owns 32*QB query rows of one query
//    head; the HP query heads that share a key/value head (grouped-query
//    attention) are packed into one workgroup so each K/V tile staged in LDS
//    serves all of them.
//  * The wave computes S^T = K Q^T (keys on the MFMA rows, queries on the
//    columns), so each lane owns one query row: the row max needs one swap
//    with the partner lane (lane ^ 32), the row sum stays lane-local, and the
//    rescale factor of the output accumulator is lane-local too.
//  * K rows are fed to the MFMA in the pi order (bits 2 and 3 of the row index
//    swapped), which makes the fp32 S^T accumulator, packed to bf16, exactly
//    the B operand of O^T += V^T P^T.  P never leaves registers.
//  * V is staged transposed in LDS (V^T[d][key]) so that the A operand of the
//    PV product is one 16-byte LDS read per lane.
//  * K/V tiles of 64 keys are double buffered in LDS; the next tile's global
//    loads are issued before the current tile's math, and one barrier per tile
//    separates the buffers.
//  * Online softmax in base 2 with the exact running maximum, so the largest
//    weight of a row is exactly 1 and carries no bf16 rounding into P V (a
//    stale maximum would let it pick up 2^-9 relative error, which shows on
//    near one-hot rows).  The accumulator (64 registers per query block) is
//    rescaled only when the maximum of some row in the wave has moved; late
//    in a long row that is rare.
//  * Causal: tiles past the workgroup's last query are never loaded, tiles
//    past a wave's last query are skipped by that wave, and only tiles that
//    straddle the diagonal (or the end of the keys) apply the element mask.
//    Workgroups are issued longest-first.
#include "device_common.hpp"
#include "launch.hpp"

namespace lcattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;         // keys per tile

template <int D, int QB, int HP, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(FwdArgs a, int n_qtiles) {
  constexpr int NU = D / 8;        // 16-byte units per K row
  constexpr int KT = D / 16;       // reduction steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int QW = 32 * QB;      // query rows per wave
  constexpr int SPAN = (kWaves / HP) * QW;  // query rows per workgroup (per head)
  constexpr int K_TILE = kBN * D * 2;       // bytes of one K tile
  constexpr int V_TILE = D * kBN * 2;       // bytes of one V^T tile
  constexpr int K_CHUNKS = kBN * NU;        // 16-byte units of a K tile
  constexpr int V_BLOCKS = (kBN / 4) * (D / 8);  // 4-key x 8-dim blocks of a V tile
  static_assert(K_CHUNKS % kThreads == 0, "K tile staging must divide evenly");
  static_assert(V_BLOCKS <= kThreads, "one V block per thread at most");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (K_TILE + V_TILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const int qt = n_qtiles - 1 - (int)blockIdx.x;  // longest causal rows first
  const int h = blockIdx.y * HP + (wave % HP);
  const int kvh = (blockIdx.y * HP) / a.G;
  const long long bz = blockIdx.z;
  const long long q_start = (long long)qt * SPAN;
  const long long wq0 = q_start + (long long)(wave / HP) * QW;

  const uint16_t* qh = a.q + (bz * a.Hq + h) * a.Nq * D;
  const uint16_t* kh = a.k + (bz * a.Hkv + kvh) * a.Nk * D;
  const uint16_t* vh = a.v + (bz * a.Hkv + kvh) * a.Nk * D;

  // keys the workgroup can see
  long long kv_end = a.Nk;
  if (a.causal) {
    const long long q_last = min(q_start + SPAN, a.Nq) - 1;
    kv_end = max(0LL, min(a.Nk, a.q_pos0 + q_last - a.k_pos0 + 1));
  }
  const int n_tiles = (int)((kv_end + kBN - 1) / kBN);

  // this wave's query range (global positions) for tile skipping and masking
  const long long wq_end = min(wq0 + QW, a.Nq);
  const bool wave_live = wq0 < a.Nq;
  const long long wpos_first = a.q_pos0 + wq0;
  const long long wpos_last = a.q_pos0 + wq_end - 1;

  // Q fragments (B operand of S^T = K Q^T): lane holds its query row's dims
  // 16t + 8*grp .. +7 for every reduction step t.
  bf16x8 qf[QB][KT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long row = wq0 + qb * 32 + c;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < a.Nq) x = ld_global16(qh + row * D + 16 * t + 8 * grp);
      qf[qb][t] = as_bf16x8(x);
    }
  }

  f32x16 acc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[qb][db][v] = 0.f;
  }

  // ---- staging of one K/V tile: global -> registers -> LDS -------------------
  u32x4 kreg[K_CHUNKS / kThreads];
  u32x4 vreg[4];
  const int v_dq = tid % (D / 8), v_kq = tid / (D / 8);
  auto load_tile = [&](int j) {
    const long long kt = (long long)j * kBN;
#pragma unroll
    for (int i = 0; i < K_CHUNKS / kThreads; ++i) {
      const int id = tid + i * kThreads;
      const int row = id / NU, u = id % NU;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kt + row < a.Nk) x = ld_global16(kh + (kt + row) * D + 8 * u);
      kreg[i] = x;
    }
    if (tid < V_BLOCKS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long key = kt + 4 * v_kq + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < a.Nk) x = ld_global16(vh + key * D + 8 * v_dq);
        vreg[r] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* ks = smem + buf * (K_TILE + V_TILE);
    unsigned char* vs = ks + K_TILE;
#pragma unroll
    for (int i = 0; i < K_CHUNKS / kThreads; ++i) {
      const int id = tid + i * kThreads;
      const int row = id / NU, u = id % NU;
      st_lds16(ks, row * (D * 2) + ((u ^ swz_rows_pi(row)) << 4), kreg[i]);
    }
    if (tid < V_BLOCKS) {
      u32x2 cols[8];
      transpose4x8(vreg, cols);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * v_dq + e;
        st_lds8(vs, d * (kBN * 2) + ((((v_kq >> 1) ^ swz_cols(d))) << 4) + ((v_kq & 1) << 3), cols[e]);
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) load_tile(j + 1);
    const unsigned char* ks = smem + (j & 1) * (K_TILE + V_TILE);
    const unsigned char* vs = ks + K_TILE;
    const long long kt = (long long)j * kBN;
    const bool wave_active = wave_live && (!a.causal || a.k_pos0 + kt <= wpos_last);
    if (wave_active) {
      const bool need_mask = (kt + kBN > a.Nk) || (a.causal && a.k_pos0 + kt + kBN - 1 > wpos_first);
      // S^T for the two 32-key halves of the tile
      f32x16 s[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[qb][kb][v] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + swap_bits23(c);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const bf16x8 kf = as_bf16x8(ld_lds16(ks, row * (D * 2) + (((2 * t + grp) ^ swz_rows_pi(row)) << 4)));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16(kf, qf[qb][t], s[qb][kb]);
        }
      }
      // mask, online softmax, pack P
      bf16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mask) {
          const long long qpos = a.q_pos0 + wq0 + qb * 32 + c;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const long long key = kt + kb * 32 + acc_row_pi(v, grp);
              const bool vis = key < a.Nk && (!a.causal || a.k_pos0 + key <= qpos);
              if (!vis) s[qb][kb][v] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[qb][kb][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = mx * a.scale_log2;
        const float m_old = m_run[qb];
        const float m_new = fmaxf(m_old, mx2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m_new == m_old) ? 1.f : fast_exp2(m_old - m_new);
        m_run[qb] = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = fast_exp2(__builtin_fmaf(s[qb][kb][v], a.scale_log2, -m_use));
            s[qb][kb][v] = p;
            lsum += p;
          }
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) {
            const int o8 = 8 * uu;
            pf[qb][2 * kb + uu] = pack_bf16x8(s[qb][kb][o8 + 0], s[qb][kb][o8 + 1], s[qb][kb][o8 + 2],
                                              s[qb][kb][o8 + 3], s[qb][kb][o8 + 4], s[qb][kb][o8 + 5],
                                              s[qb][kb][o8 + 6], s[qb][kb][o8 + 7]);
          }
        }
        l_run[qb] = l_run[qb] * alpha + lsum;
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[qb][db][v] *= alpha;
        }
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + c;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 vf = as_bf16x8(ld_lds16(vs, d * (kBN * 2) + (((2 * u + grp) ^ swz_cols(d)) << 4)));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(vf, pf[qb][u], acc[qb][db]);
        }
      }
    }
    if (j + 1 < n_tiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, write O and LSE ---------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long row = wq0 + qb * 32 + c;
    const float l = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const float lse = l > 0.f ? (m_run[qb] + fast_log2(l)) * kLn2 : -INFINITY;
    if (row < a.Nq) {
      const long long obase = ((bz * a.Hq + h) * a.Nq + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = db * 32 + 8 * jj + 4 * grp;
          const float o0 = acc[qb][db][4 * jj + 0] * inv, o1 = acc[qb][db][4 * jj + 1] * inv;
          const float o2 = acc[qb][db][4 * jj + 2] * inv, o3 = acc[qb][db][4 * jj + 3] * inv;
          if (OUT_F32) {
            f32x4 w = {o0, o1, o2, o3};
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + obase + d) = w;
          } else {
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + obase + d) = pack_bf16x4_bits(o0, o1, o2, o3);
          }
        }
      if (grp == 0) a.lse[(bz * a.Hq + h) * a.Nq + row] = lse;
    }
  }
}

template <int D, int QB, int HP, bool F32>
hipError_t launch_cfg(const FwdArgs& a, int B, hipStream_t stream) {
  constexpr int SPAN = (kWaves / HP) * 32 * QB;
  const long long n_qtiles = (a.Nq + SPAN - 1) / SPAN;
  dim3 grid((unsigned)n_qtiles, (unsigned)(a.Hq / HP), (unsigned)B);
  hipLaunchKernelGGL((attn_fwd_kernel<D, QB, HP, F32>), grid, dim3(kThreads), 0, stream, a, (int)n_qtiles);
  return hipGetLastError();
}

template <int D, int QB, bool F32>
hipError_t launch_hp(const FwdArgs& a, int B, hipStream_t stream) {
  if (a.G % 4 == 0) return launch_cfg<D, QB, 4, F32>(a, B, stream);
  if (a.G % 2 == 0) return launch_cfg<D, QB, 2, F32>(a, B, stream);
  return launch_cfg<D, QB, 1, F32>(a, B, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, int B, int D, bool out_f32, hipStream_t stream) {
  if (D == 64) return out_f32 ? launch_hp<64, 1, true>(a, B, stream) : launch_hp<64, 1, false>(a, B, stream);
  return out_f32 ? launch_hp<128, 1, true>(a, B, stream) : launch_hp<128, 1, false>(a, B, stream);
}

}  // namespace lcattn
