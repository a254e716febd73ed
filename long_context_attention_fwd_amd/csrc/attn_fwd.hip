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
//    The three pipeline buffers sit in one LDS object (K tiles, then V
//    tiles), so every fragment read is a lane-constant address plus an
//    immediate offset: no address arithmetic in the loop.
//  * Pipeline over 32-key sub-tiles; step t runs in phases that no
//    instruction crosses: [1] transposing reads of the V^T fragments of
//    sub-tile t-1, row max of S(t); [2] the 8 MFMAs of O^T += V^T P(t-1)^T,
//    one at a time between the exponentials of S(t); [3] the 8 K fragment
//    reads of sub-tile t+1 (all in flight at once; at D = 64 they go out in
//    [1] with the V^T reads), row sum and bf16 P(t);
//    [4] the 8 MFMAs of S(t+1) = K Q^T.  Fragment reads are inline assembly
//    with explicit lgkmcnt waits (the compiler would otherwise wait for the
//    direct loads in flight, or read and wait for one K fragment at a time).
//    Odd steps issue the direct loads of the tile two steps ahead, even steps
//    end with one wait + barrier.
//  * Tiles that need no element mask for any wave run in a straight-line loop
//    unrolled over the three buffers; the diagonal and tail tiles run a masked
//    copy with buffers chosen at run time.
//  * Online softmax in base 2 with the exact running maximum, so the largest
//    weight of a row is exactly 1 and carries no bf16 rounding into P V (a
//    stale maximum would let it pick up 2^-9 relative error, which shows on
//    near one-hot rows).  The accumulator (64 registers per query block) is
//    rescaled only when the maximum of some row in the wave has moved; late
//    in a long row that is rare.
//  * Causal: tiles past the workgroup's last query are never loaded, and
//    only tiles that straddle the diagonal (or the end of the keys) apply the
//    element mask.  Workgroups are issued longest-first.
#include "device_common.hpp"
#include "launch.hpp"
#include "trace.hpp"

#include <algorithm>
#include <type_traits>


namespace lcattn {

namespace {

constexpr int kWaves = kFwdWaves;  // two waves per SIMD: one's softmax overlaps the other's MFMAs
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = kFwdKeyTile;   // keys per tile

// The kernel body: workgroup number lin (already in XCD-aware order) of a
// grid of nx query tiles x ny head groups x (splits x batch).
template <int D, int QB, int HP, bool OUT_F32>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a, int n_qtiles, unsigned lin, unsigned nx,
                                              unsigned ny) {
  using T = SwzTile<D>;
  constexpr int KT = D / 16;       // reduction steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int QW = 32 * QB;      // query rows per wave
  constexpr int SPAN = (kWaves / HP) * QW;  // query rows per workgroup (per head)
  static_assert(QB == 1, "one block of 32 query rows per wave");
  static_assert(kBN == 64, "SwzTile holds 64 rows");
  // D = 64: the K fragments of the next sub-tile are read at the start of a
  // step, next to the V^T reads, so their latency hides behind the row max,
  // the PV products and the exponentials (measured 10% faster there).  At
  // D = 128 the extra 32 live registers cost more than that latency (the
  // other wave of the SIMD already covers it): they are read after the
  // exponentials.
  constexpr bool kEarlyK = D <= 64;

  // LDS: the K tiles of the three pipeline buffers, then their V tiles
  // (row-major, swizzled), in one object so that every fragment read is a
  // lane-constant address plus an immediate offset below 64 KiB.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[6 * T::BYTES];
  constexpr int KB = T::BYTES;      // bytes of one tile
  constexpr int VREG = 3 * T::BYTES;  // start of the V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  // longest causal rows first; key range (split) outermost, which dispatches
  // the first ranges of every query tile before the later, shorter ones
  // XCD-aware order: neighbouring query tiles of one head group share an XCD
  // and its L2 while they stream the same key/value tiles
  // workgroup-uniform: kept in scalar registers
  const unsigned lxy = __builtin_amdgcn_readfirstlane(lin / nx);
  const int by = __builtin_amdgcn_readfirstlane(lxy % ny);
  const unsigned bzs = __builtin_amdgcn_readfirstlane(lxy / ny);
  const unsigned xi = __builtin_amdgcn_readfirstlane(lin - lxy * nx);
  int qt, split;
  long long bz;
  if (a.compact) {
    // x enumerates the (key range, query tile) pairs with work: range r holds
    // the query tiles that see one of its keys, longest first (the host
    // sizes the grid by the same count)
    const long long tiles = (a.Nk + kBN - 1) / kBN;
    const int st = a.split_tiles;
    const long long dp = a.q_pos0 - a.k_pos0;
    unsigned i = xi;
    int r = 0;
    for (; r < a.n_splits; ++r) {
      long long c = 0;
      if ((long long)r * st < tiles) {  // the range's first key exists
        const long long y = (long long)r * st * kBN - dp;  // a tile has work iff its last row >= y
        if (!a.causal || y <= 0)
          c = n_qtiles;
        else if (y + 1 <= a.Nq)
          c = n_qtiles - ((y + SPAN) / SPAN - 1);
      }
      if (i < c) break;
      i -= (unsigned)c;
    }
    if (r >= a.n_splits) return;  // past the pairs with work
    qt = n_qtiles - 1 - (int)i;
    split = r;
    bz = bzs;
  } else {
    qt = n_qtiles - 1 - (int)xi;
    const unsigned split_u = __builtin_amdgcn_readfirstlane(bzs / (unsigned)a.B);
    bz = bzs - split_u * (unsigned)a.B;
    split = (int)split_u;
  }
  if (qt < 0) return;  // a grouped launch's grid covers its longest call
  const int h = by * HP + (wave % HP);
  const int kvh = (by * HP) / a.G;
  const long long q_start = (long long)qt * SPAN;
  const long long wq0 = q_start + (long long)(wave / HP) * QW;

  const uint16_t* qh = a.q + bz * a.qs[0] + h * a.qs[1];
  const uint16_t* kh = a.k + bz * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vh = a.v + bz * a.ks[0] + kvh * a.ks[1];

  // keys the workgroup can see
  long long kv_end = a.Nk;
  if (a.causal) {
    const long long q_last = min(q_start + SPAN, a.Nq) - 1;
    kv_end = max(0LL, min(a.Nk, a.q_pos0 + q_last - a.k_pos0 + 1));
  }
  // this workgroup's key tiles: [j0, j0 + n_tiles) of its split
  const int j0 = split * a.split_tiles;
  const int n_tiles = max(0, min((int)((kv_end + kBN - 1) / kBN), j0 + a.split_tiles) - j0);
  // a key range of the split forward that no query of the tile sees writes
  // no partial: the merge reads only the ranges below the tile's last visible
  // key tile
  if (a.n_splits > 1 && n_tiles == 0) return;
  const int n_sub = 2 * n_tiles;  // 32-key sub-tiles
  // q_pos0 - k_pos0, clamped to the int range (rows and keys are < 2^31)
  const int dpos = (int)max(min(a.q_pos0 - a.k_pos0, (long long)INT32_MAX), (long long)INT32_MIN + 1);
  const int qrow = (int)(wq0 + c);
  const int klim = (int)min(a.Nk, (long long)INT32_MAX);

  typename T::template AsyncLoader<kWaves> kload, vload;
  kload.init(wave, lane, false, a.ks[2]);
  vload.init(wave, lane, true, a.ks[2]);
  // the wave index in a scalar register: the LDS side of a direct load is
  // then scalar arithmetic
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int j, int b) __attribute__((always_inline)) {
    const long long r0 = (long long)(j0 + j) * kBN;
    if (r0 + kBN <= a.Nk) {  // uniform: every row of the tile exists
      kload.load_full(smem + b * KB, kh, r0, wave_s);
      vload.load_full(smem + VREG + b * KB, vh, r0, wave_s);
    } else {
      kload.load(smem + b * KB, kh, r0, a.Nk, wave_s);
      vload.load(smem + VREG + b * KB, vh, r0, a.Nk, wave_s);
    }
  };
  if (n_tiles > 0) issue(0, 0);

  // Q fragments (B operand of S^T = K Q^T): lane holds its query row's dims
  // 16t + 8*grp .. +7 for every reduction step t.
  bf16x8 qf[KT];
  {
    const long long row = wq0 + c;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < a.Nq) x = ld_global16(qh + row * a.qs[2] + 16 * t + 8 * grp);
      qf[t] = as_bf16x8(x);
    }
  }

  f32x16 acc[DB];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
  bf16x8 pf[2];  // P of the sub-tile waiting for its PV product (zero: no-op)
  pf[0] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  pf[1] = pf[0];
  // per-lane LDS addresses of the K row fragments (in the K tile of buffer 0)
  // and of the V^T fragments (in the V tile of buffer 0); a sub-tile adds an
  // offset: (buffer) * KB + (half) * 32 rows
  const unsigned lds0 = (unsigned)reinterpret_cast<uintptr_t>(smem);
  unsigned koff[KT], voff[DB];
#pragma unroll
  for (int t = 0; t < KT; ++t) koff[t] = lds0 + T::row_off(c, grp, t);
#pragma unroll
  for (int db = 0; db < DB; ++db) voff[db] = lds0 + VREG + T::tr_off(lane, db);

  // Fragment reads of one 32-key sub-tile at byte offset `off` from buffer 0:
  // a compile-time offset (std::integral_constant) becomes the immediate of
  // each read, a run-time one is added to the address.
  auto read_k = [&](auto off, u32x4 (&kf)[KT]) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(off)>) {
#pragma unroll
      for (int t = 0; t < KT; ++t) kf[t] = lds_read16_rt(koff[t] + off);
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t) kf[t] = lds_read16_imm<decltype(off)::value>(koff[t]);
    }
  };
  auto read_v = [&](auto off, u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(off)>) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f[db][0] = tr_frag_asm_at<T::ROW_BYTES>(voff[db], off);
        f[db][1] = tr_frag_asm_at<T::ROW_BYTES>(voff[db], off + 16 * T::ROW_BYTES);
      }
    } else {
      constexpr int O = decltype(off)::value;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f[db][0] = tr_frag_asm_imm<O, T::ROW_BYTES>(voff[db]);
        f[db][1] = tr_frag_asm_imm<O + 16 * T::ROW_BYTES, T::ROW_BYTES>(voff[db]);
      }
    }
  };
  auto wait_k = [&](u32x4 (&kf)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KT; t += 4) lds_wait_frags(kf[t], kf[t + 1], kf[t + 2], kf[t + 3]);
  };
  auto wait_v = [&](u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; db += 2) lds_wait_frags(f[db][0], f[db][1], f[db + 1][0], f[db + 1][1]);
  };
  // the V^T fragments while the KT reads of the next K fragments, issued
  // after them, may still be in flight
  auto wait_v_before_k = [&](u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; db += 2) lds_wait_frags_n<KT>(f[db][0], f[db][1], f[db + 1][0], f[db + 1][1]);
  };
  // S^T of one sub-tile from its K fragments (rows in pi order)
  auto s_mfma = [&](u32x4 (&kf)[KT]) __attribute__((always_inline)) {
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) s = mfma32x32x16(as_bf16x8(kf[t]), qf[t], s);
    return s;
  };
  auto pv_mfma = [&](u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma32x32x16(as_bf16x8(f[db][0]), pf[0], acc[db]);
      acc[db] = mfma32x32x16(as_bf16x8(f[db][1]), pf[1], acc[db]);
    }
  };

  // Online softmax of one sub-tile in three parts: S^T (one query per lane,
  // 16 of its 32 keys; the other 16 sit in lane ^ 32) -> the row maximum
  // (masked tiles mask s in place; updates m_run, returns the reference
  // used by the exponentials), the weights exp2(s * scale - m) in place, and
  // P packed as the B operand of the next PV product with this sub-tile's
  // part of the row sum.  The maximum is exact, so a row's largest weight is
  // exactly 1 and carries no bf16 rounding; the caller rescales O and the
  // sum when m_run moved.
  auto row_max = [&](auto masked_tag, f32x16& s, int t, float& m_old) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if (MASKED) {
      const int kt = kBN * j0 + 32 * t;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kt + acc_row_pi(v, grp);
        const bool vis = key < klim && (!a.causal || key - qrow <= dpos);
        s[v] = vis ? s[v] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, s[v]), s[v + 1]);
    mx = fmaxf(mx, s[15]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max with lane ^ 32
    }
    m_old = m_run;
    m_run = fmaxf(m_run, mx * a.scale_log2);
    // a row with no visible key so far keeps m_run = -inf; its weights are
    // exp2(-inf) = 0 against reference 0 (an unmasked sub-tile has a visible
    // key in every row, so m_run is finite there)
    if (MASKED) return (m_run == -INFINITY) ? 0.f : m_run;
    return m_run;
  };
  auto weights = [&](f32x16& s, float m_use) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = fast_exp2(__builtin_fmaf(s[v], a.scale_log2, -m_use));
  };
  auto pack = [&](const f32x16& s) __attribute__((always_inline)) {
    float ls[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
    for (int v = 4; v < 16; ++v) ls[v & 3] += s[v];
    pf[0] = pack_bf16x8(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
    pf[1] = pack_bf16x8(s[8], s[9], s[10], s[11], s[12], s[13], s[14], s[15]);
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // the accumulator holds PV up to the previous sub-tile: bring it and the
  // sum to the new reference maximum
  auto rescale = [&](float m_old, float psum) __attribute__((always_inline)) {
    if (__any(m_run != m_old)) {
      const float alpha = m_run != m_old ? fast_exp2(m_old - m_run) : 1.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
      l_run *= alpha;
    }
    l_run += psum;
  };

  auto pin16 = [&](f32x16& x) __attribute__((always_inline)) {
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]),
                 "+v"(x[14]), "+v"(x[15]));
  };

  // One step t of the pipeline over 32-key sub-tiles, in phases that no
  // instruction crosses:
  //   [1] transposing reads of the V^T fragments of sub-tile t-1; row max of S(t)
  //   [2] O^T += V^T P(t-1)^T (8 MFMAs), one at a time between the
  //       exponentials of S(t) (independent VALU work)
  //   [3] reads of the K fragments of sub-tile t+1 (all eight in flight at
  //       once; in [1] when kEarlyK); row sum and bf16 P(t)
  //   [4] S(t+1) = K Q^T (8 MFMAs); rescale when some row's maximum moved
  // koff_t / voff_t: byte offsets of sub-tiles t+1 (K) and t-1 (V) from
  // buffer 0 (compile-time in the unrolled loop).  Returns S(t+1).
  auto step = [&](auto masked_tag, int t, f32x16 s_cur, auto koff_t, auto voff_t) __attribute__((always_inline)) {
    u32x4 f[DB][2];
    read_v(voff_t, f);
    u32x4 kf[KT];
    if constexpr (kEarlyK) read_k(koff_t, kf);
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the row max
    float m_old;
    const float m_use = row_max(masked_tag, s_cur, t, m_old);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kEarlyK)
      wait_v_before_k(f);
    else
      wait_v(f);
    pv_mfma(f);
    weights(s_cur, m_use);
    constexpr int NPV = 2 * DB;
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 32 / NPV, 0);
    }
    // the weights are computed here, next to the PV products (otherwise they
    // are sunk past the rescale branch below, out of reach of the MFMAs)
    pin16(s_cur);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!kEarlyK) read_k(koff_t, kf);
    float psum = pack(s_cur);
    {
      u32x4 p0 = as_u32x4(pf[0]), p1 = as_u32x4(pf[1]);
      asm volatile("" : "+v"(p0), "+v"(p1), "+v"(psum));
      pf[0] = as_bf16x8(p0);
      pf[1] = as_bf16x8(p1);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_k(kf);
    const f32x16 s_next = s_mfma(kf);
    rescale(m_old, psum);
    return s_next;
  };
  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmem();  // this wave's part of the next tile has landed in LDS
    __syncthreads();
  };
  using std::integral_constant;
  constexpr int H32 = 32 * T::ROW_BYTES;  // second half of a tile

  // Tiles [0, n_full) need no element mask for any wave of the workgroup:
  // every key precedes the workgroup's first query and lies inside Nk.
  long long full_keys = a.Nk;
  if (a.causal) full_keys = min(full_keys, max(0LL, a.q_pos0 + q_start - a.k_pos0 + 1));
  const int n_full = (int)min((long long)n_tiles, max(0LL, full_keys / kBN - j0));

  // Schedule: tile j lives in buffer j % 3.  Step t reads the K half of
  // sub-tile t+1 and the V half of sub-tile t-1; odd steps t issue the direct
  // loads of tile (t+3)/2 (its buffer was last read before the barrier that
  // ended step t-1), even steps end with a barrier after which tile t/2+1 is
  // resident.  Past the last tile the loads repeat it into the free buffer
  // and S of the missing sub-tile is computed and dropped.
  if (n_tiles > 0) {
    wait_vmem();
    __syncthreads();
    issue(min(1, n_tiles - 1), 1);
    f32x16 s;
    {
      u32x4 kf[KT];
      read_k(integral_constant<int, 0>{}, kf);
      wait_k(kf);
      s = s_mfma(kf);
    }
    // step 0: nothing to multiply with V yet
    {
      float m_old;
      const float m_use = n_full > 0 ? row_max(std::false_type{}, s, 0, m_old) : row_max(std::true_type{}, s, 0, m_old);
      weights(s, m_use);
      l_run = pack(s);
      u32x4 kf[KT];
      read_k(integral_constant<int, H32>{}, kf);
      wait_k(kf);
      s = s_mfma(kf);
    }
    sync();
    int t = 1;
    // unmasked steps, unrolled over the buffer pattern (period 6)
    for (; t + 6 <= 2 * n_full; t += 6) {
      const int jb = (t - 1) / 2;  // multiple of 3
      issue(min(jb + 2, n_tiles - 1), 2);
      s = step(std::false_type{}, t, s, integral_constant<int, KB>{}, integral_constant<int, 0>{});
      s = step(std::false_type{}, t + 1, s, integral_constant<int, KB + H32>{}, integral_constant<int, H32>{});
      sync();
      issue(min(jb + 3, n_tiles - 1), 0);
      s = step(std::false_type{}, t + 2, s, integral_constant<int, 2 * KB>{}, integral_constant<int, KB>{});
      s = step(std::false_type{}, t + 3, s, integral_constant<int, 2 * KB + H32>{}, integral_constant<int, KB + H32>{});
      sync();
      issue(min(jb + 4, n_tiles - 1), 1);
      s = step(std::false_type{}, t + 4, s, integral_constant<int, 0>{}, integral_constant<int, 2 * KB>{});
      s = step(std::false_type{}, t + 5, s, integral_constant<int, H32>{}, integral_constant<int, 2 * KB + H32>{});
      sync();
    }
    // the rest (diagonal and tail tiles, and leftovers): offsets at run time
    for (; t < n_sub; ++t) {
      if (t & 1) issue(min((t + 3) / 2, n_tiles - 1), ((t + 3) / 2) % 3);
      const int ko = ((t + 1) / 2 % 3) * KB + ((t + 1) & 1) * H32;
      const int vo = ((t - 1) / 2 % 3) * KB + ((t - 1) & 1) * H32;
      s = step(std::true_type{}, t, s, ko, vo);
      if (!(t & 1)) sync();
    }
    // PV of the last sub-tile
    {
      u32x4 f[DB][2];
      read_v(((n_tiles - 1) % 3) * KB + H32, f);
      wait_v(f);
      pv_mfma(f);
    }
    wait_vmem();  // no direct load may still be in flight when the workgroup ends
  }

  // ---- epilogue: normalise, write O and LSE ---------------------------------
  {
    const long long row = wq0 + c;
    const float l = l_run + __shfl_xor(l_run, 32);
    // A row is empty (O = 0, LSE = -inf) when the first key of this call's
    // range is past the end of the keys or masked for it: decided from
    // positions, not from l, so that NaN scores (l = NaN) give a NaN row
    // instead of the empty-row result.
    const int kfirst = kBN * j0;
    const bool has_key = kfirst < klim && (!a.causal || kfirst - qrow <= dpos);
    const float inv = has_key ? 1.0f / l : 0.f;
    const float lse = has_key ? (m_run + fast_log2(l)) * kLn2 : -INFINITY;
    if (row < a.Nq) {
      const long long obase = split * a.part_stride + bz * a.os[0] + h * a.os[1] + row * a.os[2];
      const long long lidx = split * (a.part_stride / D) + (bz * a.Hq + h) * a.Nq + row;
      // weights of the running result and of this call's in the merged one
      // (a streaming ring step: the merge of "So funktioniert
      // Kontextparallelität", one KV block at a time)
      float w_old = 0.f, w_new = inv, lse_out = lse;
      if (OUT_F32 && a.accum) {
        const float l_old = a.lse[lidx];  // read by both lane groups before either writes
        // This file is compiled without NaN semantics, under which the
        // compiler may turn x == -inf into !(x > -inf) (true for NaN) or
        // lse - max(l_old, lse) into min(0, lse - l_old) (which drops a NaN).
        // So the emptiness of this call comes from key positions, that of
        // the running result from its bit pattern, and the maximum from an
        // opaque instruction: a NaN on either side stays NaN.
        unsigned old_bits;
        asm("v_mov_b32 %0, %1" : "=v"(old_bits) : "v"(l_old));
        if (!has_key) {
          w_old = 1.f;
          w_new = 0.f;
          lse_out = l_old;
        } else if (old_bits != 0xff800000u) {  // the running result is not empty
          float M;
          asm("v_max_f32 %0, %1, %2" : "=v"(M) : "v"(l_old), "v"(lse));
          const float e_old = fast_exp2((l_old - M) * kLog2e), e_new = fast_exp2((lse - M) * kLog2e);
          const float r = 1.0f / (e_old + e_new);
          w_old = e_old * r;
          w_new = e_new * r * inv;
          lse_out = M + fast_log2(e_old + e_new) * kLn2;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = db * 32 + 8 * jj + 4 * grp;
          float o0 = acc[db][4 * jj + 0] * w_new, o1 = acc[db][4 * jj + 1] * w_new;
          float o2 = acc[db][4 * jj + 2] * w_new, o3 = acc[db][4 * jj + 3] * w_new;
          if (OUT_F32) {
            float* op = static_cast<float*>(a.o) + obase + d;
            if (a.accum) {
              const f32x4 prev = *reinterpret_cast<const f32x4*>(op);
              o0 += w_old * prev[0];
              o1 += w_old * prev[1];
              o2 += w_old * prev[2];
              o3 += w_old * prev[3];
            }
            f32x4 w = {o0, o1, o2, o3};
            *reinterpret_cast<f32x4*>(op) = w;
            if (a.o_final)
              *reinterpret_cast<u32x2*>(a.o_final + ((bz * a.Hq + h) * a.Nq + row) * D + d) =
                  pack_bf16x4_bits(o0, o1, o2, o3);
          } else {
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + obase + d) = pack_bf16x4_bits(o0, o1, o2, o3);
          }
        }
      if (grp == 0) a.lse[lidx] = lse_out;
    }
  }
}

template <int D, int QB, int HP, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a, int n_qtiles) {
  attn_fwd_body<D, QB, HP, OUT_F32>(a, n_qtiles, wg_number(), gridDim.x, gridDim.y);
}

// Independent calls in one launch (a ring step's query chunks against one
// key/value chunk): grid z = (call * splits + split) * B + batch, zc = splits
// * B workgroup layers per call; call c covers n_qtiles[c] <= gridDim.x query
// tiles.
struct FwdGroup {
  FwdArgs a[kMaxFwdGroup];
  int n_qtiles[kMaxFwdGroup];
};

template <int D, int QB, int HP, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_group_kernel(FwdGroup g, int zc) {
  const unsigned lin = wg_number();
  const unsigned per_call = gridDim.x * gridDim.y * (unsigned)zc;
  const unsigned c = lin / per_call;
  attn_fwd_body<D, QB, HP, OUT_F32>(g.a[c], g.n_qtiles[c], lin - c * per_call, gridDim.x, gridDim.y);
}

template <int D, int QB, int HP, bool F32>
hipError_t launch_cfg(const FwdArgs& a, int B, hipStream_t stream) {
  constexpr int SPAN = (kWaves / HP) * 32 * QB;
  const long long n_qtiles = (a.Nq + SPAN - 1) / SPAN;
  dim3 grid((unsigned)n_qtiles, (unsigned)(a.Hq / HP), (unsigned)(B * a.n_splits));
  if (a.compact) {
    const long long pairs = splitkv_pairs(a.Nq, a.Nk, a.q_pos0 - a.k_pos0, a.causal, SPAN, a.n_splits);
    if (pairs == 0) return hipSuccess;  // no query sees a key: the merge writes the empty rows
    if (pairs >= (1LL << 31)) return hipErrorInvalidConfiguration;
    grid = dim3((unsigned)pairs, (unsigned)(a.Hq / HP), (unsigned)B);
  }
  if (!grid_fits(grid)) return hipErrorInvalidConfiguration;
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

template <int D, int HP>
hipError_t launch_group_hp(FwdGroup& g, int n, int B, int splits, hipStream_t stream) {
  constexpr int SPAN = (kWaves / HP) * 32;
  long long nx = 0;
  for (int c = 0; c < n; ++c) {
    g.n_qtiles[c] = (int)((g.a[c].Nq + SPAN - 1) / SPAN);
    nx = std::max<long long>(nx, g.n_qtiles[c]);
  }
  dim3 grid((unsigned)nx, (unsigned)(g.a[0].Hq / HP), (unsigned)(B * splits * n));
  if (!grid_fits(grid)) return hipErrorInvalidConfiguration;
  LCATTN_LAUNCH("attn_fwd_kernel_fp32out", (attn_fwd_group_kernel<D, 1, HP, true>), grid, dim3(kThreads), 0, stream,
                g, B * splits);
  return hipGetLastError();
}

template <int D>
hipError_t launch_group_d(FwdGroup& g, int n, int B, int splits, hipStream_t stream) {
  const int G = g.a[0].G;
  if (G % 4 == 0) return launch_group_hp<D, 4>(g, n, B, splits, stream);
  if (G % 2 == 0) return launch_group_hp<D, 2>(g, n, B, splits, stream);
  return launch_group_hp<D, 1>(g, n, B, splits, stream);
}

}  // namespace

hipError_t launch_attn_fwd_group(const FwdArgs* calls, int n, int B, int D, hipStream_t stream) {
  FwdGroup g{};
  for (int c = 0; c < n; ++c) {
    FwdArgs a = calls[c];
    a.B = B;
    a.qs[2] = D; a.qs[1] = a.Nq * D; a.qs[0] = a.Hq * a.Nq * D;
    a.ks[2] = D; a.ks[1] = a.Nk * D; a.ks[0] = a.Hkv * a.Nk * D;
    a.os[2] = D; a.os[1] = a.Nq * D; a.os[0] = a.Hq * a.Nq * D;
    g.a[c] = a;
  }
  return D == 64 ? launch_group_d<64>(g, n, B, 1, stream) : launch_group_d<128>(g, n, B, 1, stream);
}

hipError_t launch_attn_fwd_group_split(const FwdArgs* calls, float* const* parts, int n, int B, int D, int splits,
                                       hipStream_t stream) {
  FwdGroup g{};
  MergeSplits ms[kMaxFwdGroup];
  const int HP = calls[0].G % 4 == 0 ? 4 : (calls[0].G % 2 == 0 ? 2 : 1);
  for (int c = 0; c < n; ++c) {
    FwdArgs a = calls[c];
    a.B = B;
    a.qs[2] = D; a.qs[1] = a.Nq * D; a.qs[0] = a.Hq * a.Nq * D;
    a.ks[2] = D; a.ks[1] = a.Nk * D; a.ks[0] = a.Hkv * a.Nk * D;
    a.os[2] = D; a.os[1] = a.Nq * D; a.os[0] = a.Hq * a.Nq * D;  // partials: contiguous [B, Hq, Nq, D]
    const long long tiles = (a.Nk + kBN - 1) / kBN;
    const long long stride = (long long)B * a.Hq * a.Nq * D;
    a.o = parts[c];
    a.lse = parts[c] + (long long)splits * stride;
    a.n_splits = splits;
    a.split_tiles = (int)((tiles + splits - 1) / splits);
    a.part_stride = stride;
    a.accum = 0;
    a.o_final = nullptr;
    g.a[c] = a;
    ms[c].span = (kWaves / HP) * 32;
    ms[c].split_tiles = a.split_tiles;
    ms[c].key_tile = kBN;
    ms[c].Nq = a.Nq;
    ms[c].Nk = a.Nk;
    ms[c].dpos = a.q_pos0 - a.k_pos0;
    ms[c].causal = a.causal;
  }
  hipError_t e = D == 64 ? launch_group_d<64>(g, n, B, splits, stream) : launch_group_d<128>(g, n, B, splits, stream);
  if (e != hipSuccess) return e;
  for (int c = 0; c < n; ++c) {
    const FwdArgs& a = calls[c];
    e = launch_merge_into(parts[c], g.a[c].lse, splits, ms[c],
                          static_cast<float*>(a.o), a.lse, a.accum == 0, a.o_final, (long long)B * a.Hq * a.Nq, D,
                          stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_fwd(const FwdArgs& a0, int B, int D, bool out_f32, hipStream_t stream) {
  FwdArgs a = a0;
  a.B = B;
  auto contiguous = [&](long long (&st)[3], int H, long long N) {
    if (st[0] == 0 && st[1] == 0 && st[2] == 0) {
      st[2] = D;
      st[1] = N * D;
      st[0] = H * N * D;
    }
  };
  contiguous(a.qs, a.Hq, a.Nq);
  contiguous(a.ks, a.Hkv, a.Nk);
  contiguous(a.os, a.Hq, a.Nq);
  if (D == 64) return out_f32 ? launch_hp<64, 1, true>(a, B, stream) : launch_hp<64, 1, false>(a, B, stream);
  return out_f32 ? launch_hp<128, 1, true>(a, B, stream) : launch_hp<128, 1, false>(a, B, stream);
}

hipError_t launch_attn_fwd_splitkv(const FwdArgs& a0, int B, int D, int n_splits, float* o_parts, float* lse_parts,
                                   hipStream_t stream) {
  FwdArgs a = a0;
  uint16_t* o = static_cast<uint16_t*>(a0.o);
  float* lse = a0.lse;
  const long long tiles = (a.Nk + kBN - 1) / kBN;
  a.o = o_parts;
  a.lse = lse_parts;
  a.os[0] = a.os[1] = a.os[2] = 0;  // partials: contiguous [B, Hq, Nq, D]
  a.n_splits = n_splits;
  a.split_tiles = (int)((tiles + n_splits - 1) / n_splits);
  a.part_stride = (long long)B * a.Hq * a.Nq * D;
  a.compact = n_splits > 1 ? 1 : 0;
  hipError_t e = launch_attn_fwd(a, B, D, true, stream);
  if (e != hipSuccess) return e;
  const int HP = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);
  MergeSplits ms;
  ms.span = (kWaves / HP) * 32;
  ms.split_tiles = a.split_tiles;
  ms.key_tile = kBN;
  ms.Nq = a.Nq;
  ms.Nk = a.Nk;
  ms.dpos = a.q_pos0 - a.k_pos0;
  ms.causal = a.causal;
  return launch_partial_merge(o_parts, true, lse_parts, n_splits, o, lse, (long long)B * a.Hq * a.Nq, D, stream, &ms);
}

}  // namespace lcattn
