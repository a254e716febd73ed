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
//  * A workgroup is 8 waves, two per SIMD, so the hardware overlaps one
//    wave's softmax (VALU, exp) with the other's MFMAs.  Each wave owns
//    32*QB query rows of one query
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
//  * K and V tiles of 64 keys go global -> LDS with direct loads
//    (global_load_lds_dwordx4: no registers, no VALU), row-major with a
//    per-row XOR swizzle of 16-byte units.  K fragments are plain 16-byte
//    reads; the V^T fragments of the PV product come from the row-major V tile
//    through the transposing LDS read (ds_read_b64_tr_b16, two per fragment).
//  * Tiles are double buffered: the next tile's direct loads are issued before
//    the current tile's math, and one wait + barrier per tile hands over.
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
#include "trace.hpp"

namespace lcattn {

namespace {

constexpr int kWaves = 8;      // two waves per SIMD: one's softmax overlaps the other's MFMAs
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;         // keys per tile

template <int D, int QB, int HP, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a, int n_qtiles) {
  using T = LdsTile<D>;
  constexpr int KT = D / 16;       // reduction steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int QW = 32 * QB;      // query rows per wave
  constexpr int SPAN = (kWaves / HP) * QW;  // query rows per workgroup (per head)
  static_assert(kBN == 64, "LdsTile holds 64 rows");

  // Three buffers, each a K tile followed by a V tile (row-major, swizzled),
  // as separate objects so the compiler can tell them apart.  Iteration j
  // reads V of tile j-1 and K of tile j while the direct loads of tile j+1
  // land in the third buffer.
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2 * T::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2 * T::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char smem2[2 * T::BYTES];

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
  // q_pos0 - k_pos0, clamped to the int range (rows and keys are < 2^31)
  const int dpos = (int)max(min(a.q_pos0 - a.k_pos0, (long long)INT32_MAX), (long long)INT32_MIN + 1);

  auto issue = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    T::template load_async<kWaves>(buf, kh, (long long)j * kBN, a.Nk, wave, lane);
    T::template load_async<kWaves>(buf + T::BYTES, vh, (long long)j * kBN, a.Nk, wave, lane);
  };
  if (n_tiles > 0) issue(0, smem0);

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
  bf16x8 pf[QB][4];  // P of the previous tile, waiting for its PV product
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[qb][db][v] = 0.f;
  }
  bool prev_active = false;

  // O^T += V^T P^T for the tile whose V sits in buf
  auto pv = [&](const unsigned char* buf) __attribute__((always_inline)) {
    const unsigned char* vs = buf + T::BYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 vf = T::tr_frag(vs, 16 * u, db * 32, lane);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(vf, pf[qb][u], acc[qb][db]);
      }
    }
  };

  wait_vmem();
  __syncthreads();

  // one iteration: PV of tile j-1, prefetch of tile j+1, S and softmax of tile j
  auto step = [&](int j, const unsigned char* prev, const unsigned char* cur, unsigned char* nxt) __attribute__((always_inline)) {
    if (prev_active) pv(prev);
    if (j + 1 < n_tiles) issue(j + 1, nxt);
    const unsigned char* ks = cur;
    const long long kt = (long long)j * kBN;
    const bool wave_active = wave_live && (!a.causal || a.k_pos0 + kt <= wpos_last);
    prev_active = wave_active;
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
          const bf16x8 kf = T::row_frag(ks, row, t, grp);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16(kf, qf[qb][t], s[qb][kb]);
        }
      }
      // mask, online softmax, pack P (the PV product follows next iteration)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mask) {
          // 32-bit index math: key k is visible to query row r iff
          // k < Nk and (not causal or k - r <= q_pos0 - k_pos0)
          const int qrow = (int)(wq0 + qb * 32 + c);
          const int klim = (int)min(a.Nk, (long long)INT32_MAX);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = (int)kt + kb * 32 + acc_row_pi(v, grp);
              const bool vis = key < klim && (!a.causal || key - qrow <= dpos);
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
    }
    wait_vmem();  // this wave's part of tile j + 1 has landed in LDS
    __syncthreads();
  };
  int j = 0;
  for (; j + 3 <= n_tiles; j += 3) {
    step(j, smem2, smem0, smem1);
    step(j + 1, smem0, smem1, smem2);
    step(j + 2, smem1, smem2, smem0);
  }
  if (j < n_tiles) step(j, smem2, smem0, smem1);
  if (j + 1 < n_tiles) step(j + 1, smem0, smem1, smem2);
  // PV of the last tile
  if (prev_active) {
    const int r = (n_tiles - 1) % 3;
    pv(r == 0 ? smem0 : (r == 1 ? smem1 : smem2));
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
  LCATTN_LAUNCH("attn_fwd_kernel", (attn_fwd_kernel<D, QB, HP, F32>), grid, dim3(kThreads), 0, stream, a, (int)n_qtiles);
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
