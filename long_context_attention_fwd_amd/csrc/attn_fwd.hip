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
//  * Pipeline over three LDS buffers: iteration j issues the direct loads of
//    tile j+1, computes S(j) = K(j) Q^T, then the PV product of tile j-1 and
//    the softmax of tile j (independent MFMA and VALU work), then one
//    wait + barrier.  The transposing reads are issued through inline
//    assembly with explicit lgkmcnt waits: the compiler cannot tell which
//    LDS buffer such a read touches and would otherwise wait for the in-flight
//    direct loads of tile j+1 before it.  The K reads are ordinary loads of
//    distinct __shared__ objects, which it can tell apart.
//  * Tiles that need no element mask for any wave run in a straight-line loop
//    unrolled over the three buffers; the diagonal and tail tiles run a masked
//    copy with buffers chosen at run time.
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

#include <type_traits>


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
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int u = 0; u < 4; ++u) pf[qb][u] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
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
  const typename T::RowAddr ra = T::row_addr(swap_bits23(c), grp);
  const typename T::TrAddr ta = T::tr_addr(lane);

  // O^T += V^T P^T for the tile whose V sits in buf
  auto pv = [&](const unsigned char* buf) __attribute__((always_inline)) {
    const unsigned vbase = (unsigned)reinterpret_cast<uintptr_t>(buf + T::BYTES);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x4 f0 = tr_frag_asm_at<T::ROW_BYTES>(vbase, T::tr_off(ta, 0, db));
      u32x4 f1 = tr_frag_asm_at<T::ROW_BYTES>(vbase, T::tr_off(ta, 16, db));
      u32x4 f2 = tr_frag_asm_at<T::ROW_BYTES>(vbase, T::tr_off(ta, 32, db));
      u32x4 f3 = tr_frag_asm_at<T::ROW_BYTES>(vbase, T::tr_off(ta, 48, db));
      lds_wait_frags(f0, f1, f2, f3);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        acc[qb][db] = mfma32x32x16(as_bf16x8(f0), pf[qb][0], acc[qb][db]);
        acc[qb][db] = mfma32x32x16(as_bf16x8(f1), pf[qb][1], acc[qb][db]);
        acc[qb][db] = mfma32x32x16(as_bf16x8(f2), pf[qb][2], acc[qb][db]);
        acc[qb][db] = mfma32x32x16(as_bf16x8(f3), pf[qb][3], acc[qb][db]);
      }
    }
  };

  wait_vmem();
  __syncthreads();

  // one iteration: prefetch of tile j+1, S(j), then the PV product of tile
  // j-1 (independent MFMAs) interleaved with the softmax of tile j (VALU).
  // The body is straight-line code (one copy with the element mask, one
  // without) so the scheduler can mix the two; a tile that is entirely past
  // this wave's queries runs the masked copy and contributes nothing.
  auto body = [&](auto masked_tag, int j, const unsigned char* prev, const unsigned char* cur, float* alpha_q)
                  __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const long long kt = (long long)j * kBN;
    f32x16 s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[qb][kb][v] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 kf = T::row_frag_at(cur, ra, t, kb * 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16(kf, qf[qb][t], s[qb][kb]);
      }
    }
    pv(prev);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (MASKED) {
        const int qrow = (int)(wq0 + qb * 32 + c);
        const int klim = (int)min(a.Nk, (long long)INT32_MAX);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = (int)kt + kb * 32 + acc_row_pi(v, grp);
            const bool vis = key < klim && (!a.causal || key - qrow <= dpos);
            s[qb][kb][v] = vis ? s[qb][kb][v] : -INFINITY;
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
      alpha_q[qb] = (m_new == m_old) ? 1.f : fast_exp2(m_old - m_new);
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
      l_run[qb] = l_run[qb] * alpha_q[qb] + lsum;
    }
  };
  auto finish = [&](const float* alpha_q) __attribute__((always_inline)) {
    // rescale the accumulator (after the PV product of the previous tile)
    bool any_rescale = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any_rescale |= alpha_q[qb] != 1.f;
    if (__any(any_rescale)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[qb][db][v] *= alpha_q[qb];
    }
    wait_vmem();  // this wave's part of the next tile has landed in LDS
    __syncthreads();
  };
  // Tiles [0, n_full) need no element mask for any wave of the workgroup:
  // every key precedes the workgroup's first query and lies inside Nk.
  long long full_keys = a.Nk;
  if (a.causal) full_keys = min(full_keys, max(0LL, a.q_pos0 + q_start - a.k_pos0 + 1));
  const int n_full = (int)min((long long)n_tiles, full_keys / kBN);
  auto step_full = [&](int j, const unsigned char* prev, const unsigned char* cur, unsigned char* nxt)
                       __attribute__((always_inline)) {
    issue(min(j + 1, n_tiles - 1), nxt);  // the last tile reloads itself into the free buffer
    float alpha_q[QB];
    body(std::false_type{}, j, prev, cur, alpha_q);
    finish(alpha_q);
  };
  int j = 0;
  for (; j + 3 <= n_full; j += 3) {
    step_full(j, smem2, smem0, smem1);
    step_full(j + 1, smem0, smem1, smem2);
    step_full(j + 2, smem1, smem2, smem0);
  }
  // the rest (the diagonal and tail tiles): buffers chosen at run time
  auto buf = [&](int i) __attribute__((always_inline)) {
    const int r = i % 3;
    return r == 0 ? smem0 : (r == 1 ? smem1 : smem2);
  };
  for (; j < n_tiles; ++j) {
    issue(min(j + 1, n_tiles - 1), buf(j + 1));
    float alpha_q[QB];
    body(std::true_type{}, j, buf(j + 2), buf(j), alpha_q);
    finish(alpha_q);
  }
  // PV of the last tile
  if (n_tiles > 0) pv(buf(n_tiles - 1));

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
  LCATTN_LAUNCH(F32 ? "attn_fwd_kernel_fp32out" : "attn_fwd_kernel", (attn_fwd_kernel<D, QB, HP, F32>), grid,
                dim3(kThreads), 0, stream, a, (int)n_qtiles);
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
