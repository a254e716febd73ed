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
// Kernels (no atomics anywhere: results are deterministic):
//  * bwd_delta: Dv per query row, HBM bound.
//  * bwd_dkdv: a workgroup owns 128 keys and one query head; the work of each
//    group of 32 keys is split over two waves of one SIMD.  Wave A holds K
//    (MFMA operand in registers) and accumulates dV: S = Q K^T, P, dV^T +=
//    dO^T P; it hands P (bf16) through LDS to wave B, which holds V and
//    accumulates dK: dP = dO V^T, dS = P (dP - Dv), dK^T += Q^T dS, one query
//    tile behind.  Query rows are fed to the MFMA in the pi order, so P and dS
//    leave the accumulators already in the operand layout of the next
//    product.  64-row Q and dO tiles arrive by direct loads (three buffers);
//    the unmasked tiles run a loop unrolled over the buffers with immediate
//    LDS offsets.
//  * bwd_dkdv_reduce (grouped-query attention only): the per-query-head fp32
//    partials of dK, dV are summed over the group and rounded to bf16.  One
//    workgroup per (key tile, query head) gives G times more workgroups than
//    one per key/value head, which a one-KV-head Ulysses share needs.
//  * bwd_dq: like the forward, 8 waves own query rows (the heads of a group
//    packed together) and walk the key tiles, recomputing S^T = K Q^T and
//    dP^T = V dO^T and accumulating dQ^T += K^T dS^T (K through the
//    transposing read), pipelined the same way.
// dQ by a separate pass costs two recomputed products (7 contractions instead
// of 5) but avoids fp32 atomic traffic proportional to N^2 / tile (measured:
// adding dQ blocks with fp32 atomics runs at 1.35 TB/s, too slow to pay).
// Small problems split both passes into ranges (query ranges for dK/dV, key
// ranges for dQ; grid z = range * B + batch), each range writing fp32
// partials that bwd_dkdv_reduce / bwd_dq_reduce sum in range order.
#include "device_common.hpp"
#include "launch.hpp"
#include "trace.hpp"

#include <algorithm>
#include <mutex>
#include <type_traits>


namespace lcattn {

namespace {

// ---------------------------------------------------------------------------
// Dv_i = <dO_i, O_i> (fp32), one thread per 8 elements; row n of head h of
// batch b (grid z = b, y = h) at element b*s0 + h*s1 + n*s2 of o and d_o,
// Dv contiguous [B, H, N]
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ d_o,
                                                        float* __restrict__ delta, long long N, long long s0,
                                                        long long s1, long long s2) {
  constexpr int U = D / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = idx / U;
  const int u = (int)(idx % U);
  const long long b = blockIdx.z, h = blockIdx.y;
  float s = 0.f;
  if (n < N) {
    const long long off = b * s0 + h * s1 + n * s2 + 8 * u;
    const u32x4 x = ld_global16(o + off);
    const u32x4 y = ld_global16(d_o + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
      s += __uint_as_float(x[e] & 0xFFFF0000u) * __uint_as_float(y[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int off = U / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (n < N && u == 0) delta[(b * gridDim.y + h) * N + n] = s;
}

constexpr int kBQ = 64;   // query rows per tile

// ---------------------------------------------------------------------------
// dK, dV with the work of a key group split over two waves of one SIMD:
// workgroup = 128 keys of one key/value head x one query head, 8 waves.
// Wave w < 4 ("A") holds K of keys 32 w .. +31 and accumulates dV: per 32-row
// query block it computes S = Q K^T, P = exp(S - LSE) (masked), hands the
// bf16 P to its partner through LDS and adds dV^T += dO^T P.  Wave w + 4
// ("B"), on the same SIMD, holds V of the same keys and accumulates dK: it
// computes dP = dO V^T, takes P from LDS, forms dS = P (dP - Dv) and adds
// dK^T += Q^T dS, one query tile behind A.  Each wave runs half of the
// block's products, so two waves share every SIMD: one's exponentials and
// LDS waits overlap the other's matrix-core work.
// Query tiles of 64 rows arrive by direct loads (rows-swizzled LDS, three
// buffers); LSE and Dv of a tile through registers; one barrier per tile.
// LDS is one object (Q tiles | dO tiles | LSE, Dv | P slots) and every
// fragment address is a lane-constant base plus an offset: in the loop over
// the unmasked tiles, unrolled over the three buffers, the offsets are
// immediates (no address arithmetic per read).
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;

// b * MUL + ADD, as a compile-time constant when b is one
template <int MUL, int ADD, class Bf>
__device__ __forceinline__ auto lin_off(Bf b) {
  if constexpr (std::is_integral_v<Bf>) return b * MUL + ADD;
  else return std::integral_constant<int, Bf::value * MUL + ADD>{};
}

// The kernel body: workgroup number lin (already in XCD-aware order) of a
// grid of nx key tiles x ny query heads x B.  DS: wave B also stores its dS
// blocks (a.ds) for the dQ product pass.
template <int D, bool PARTIAL, bool DENSE, bool DS>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& a, float* __restrict__ dk_part,
                                              float* __restrict__ dv_part, unsigned lin, unsigned nx,
                                              unsigned ny) {
  using T = SwzTile<D>;
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int NW = kSplitWaves;
  constexpr int BK = 128;                  // keys per workgroup
  constexpr int TB = T::BYTES;             // one 64-row tile
  constexpr int RB = T::ROW_BYTES;
  constexpr int QR = 0, OR = 3 * TB;       // Q tiles, dO tiles
  constexpr int XR = 6 * TB;               // per buffer: LSE*log2(e) (64 floats), Dv (64 floats)
  constexpr int PR = XR + 3 * 512;         // P slots
  constexpr int PSLOT = 4 * 2 * 2 * 64 * 16;  // 4 key groups x 2 blocks x 2 halves x 64 lanes x 16 bytes
  __shared__ __attribute__((aligned(1024))) unsigned char smem[PR + 3 * PSLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const bool role_a = wave < 4;            // wave-uniform
  const int kg = wave & 3;                 // key group of 32 keys
  const long long Nq = a.Nq, Nk = a.Nk;
  // 64-bit decode here: with the 32-bit one the register allocator spills
  // lane offsets of the epilogue (measured: 48 MiB more writes per launch at
  // 64K); the few hundred prologue instructions do not show in a launch
  const long long llin = lin, lnx = nx, lny = ny;
  const long long zz = llin / (lnx * lny);  // query range * B + batch
  const int rr = (int)(zz / a.B);
  const long long bz = zz - (long long)rr * a.B;
  const int h = (int)(llin / lnx % lny);
  const int kvh = h / a.G;
  const long long kt0 = (llin % lnx) * BK;
  if (kt0 >= Nk) return;  // a grouped launch's grid covers its longest call
  const long long kw0 = kt0 + 32 * kg;
  const int key = (int)(kw0 + c);
  const float sl = a.scale * kLog2e;

  const long long hb = (bz * a.Hq + h) * Nq;
  const long long kst = DENSE ? D : a.ks[2];
  const uint16_t* kbase = DENSE ? a.k + (bz * a.Hkv + kvh) * Nk * D : a.k + bz * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = DENSE ? a.v + (bz * a.Hkv + kvh) * Nk * D : a.v + bz * a.ks[0] + kvh * a.ks[1];
  const uint16_t* qbase = DENSE ? a.q + hb * D : a.q + bz * a.qs[0] + h * a.qs[1];
  const uint16_t* obase = DENSE ? a.d_o + hb * D : a.d_o + bz * a.qs[0] + h * a.qs[1];
  const float* lbase = a.lse + hb;
  const float* dbase = a.delta + hb;

  const long long q_first = a.causal ? max(0LL, kt0 - a.dpos) : 0;
  const long long first_tile = q_first / kBQ;
  const int n_tiles = q_first >= Nq ? 0 : (int)((Nq + kBQ - 1) / kBQ - first_tile);
  // tiles masked for wave A: those holding the diagonal of some key group
  // (the first `head`), and the tail
  const int head = a.causal ? (int)max(0LL, min((long long)n_tiles,
                                                (kt0 + BK - a.dpos - first_tile * kBQ + kBQ - 1) / kBQ))
                            : 0;
  const bool tail = (Nq % kBQ) != 0;
  const int body_end = max(head, n_tiles - (tail ? 1 : 0));
  // tile i lives in buffer (i + shift) % 3: the first unmasked tile in buffer 0
  const int shift = (3 - head % 3) % 3;
  // this workgroup's tiles [i_lo, i_hi): query range rr of the split pass
  // (absolute tiles [rr * qst, (rr + 1) * qst)), else all of them; a range
  // that none of the key tile's queries reach writes no partial
  const int i_lo = (int)max(0LL, (long long)rr * a.qst - first_tile);
  const int i_hi = (int)min((long long)n_tiles, ((long long)rr + 1) * a.qst - first_tile);
  if (a.rkv > 1 && i_lo >= i_hi) return;

  typename T::template AsyncLoader<NW> ld;
  ld.init(wave, lane, false, DENSE ? D : a.qs[2]);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  float lv = 0.f;
  // tile i into its buffer: Q and dO by direct loads, LSE and Dv into a
  // register of threads 0..127 (stored by `deposit`)
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int bf = (i + shift) % 3;
    const long long r0 = (first_tile + i) * kBQ;
    if (r0 + kBQ <= Nq) {
      ld.load_full(smem + QR + bf * TB, qbase, r0, wave_s);
      ld.load_full(smem + OR + bf * TB, obase, r0, wave_s);
    } else {
      ld.load(smem + QR + bf * TB, qbase, r0, Nq, wave_s);
      ld.load(smem + OR + bf * TB, obase, r0, Nq, wave_s);
    }
    if (tid < 2 * kBQ) {
      long long row = r0 + (tid & (kBQ - 1));
      row = row < Nq ? row : Nq - 1;
      lv = (tid < kBQ ? lbase : dbase)[row];
    }
  };
  // stored dS (wave B): block (query tile, key tile kt0 / 64 + kg / 2), in
  // the order the stores produce it: the half of the block's keys of this
  // key group (kg % 2), then the (32-row block, 16-row half) of the query
  // tile, then the lane, 16 bytes each -- every store writes 1 KiB in one
  // piece (the product pass's loads put the units back in rows).  Keys past
  // Nk store what their scores give (the pass does not mask them; they are
  // visible without the causal mask, and with it to queries positioned past
  // the keys); the product pass masks them.
  long long ds_wave = 0;  // elements from a.ds to the wave's block of query tile 0's row
  unsigned ds_lane = 0;
  long long ds_nkt2 = 0;
  if constexpr (DS) {
    const int kg_s = __builtin_amdgcn_readfirstlane(kg);
    ds_wave = (bz * a.Hq + h) * a.ds_head + (kt0 / 64 + (kg_s >> 1)) * kDsBlockElems;
    ds_lane = (unsigned)((kg & 1) * 4096 + lane * 16);
    ds_nkt2 = (Nk + 127) / 128 * 2;
  }
  // A tile's dS is stored during wave B's next tile, after that tile's dP
  // products went out (measured: 1-3% faster than at its start or end, or
  // before the loads of the next tile; stores count in the same counter as
  // the tile loads, and stored at once they held every barrier until they
  // reached memory).  The address is a.ds
  // plus a wave-uniform element offset (scalar registers; kept as pointer
  // arithmetic on a.ds, so that the compiler knows it is global memory and
  // emits global stores -- flat stores would also count against the LDS
  // counter that every fragment wait uses) plus the lane's byte offset.
  u32x4 ds_pend[4];
  auto store_ds = [&](int i) __attribute__((always_inline)) {
    const long long qt = first_tile + i;
    const unsigned long long off =
        (unsigned long long)(ds_wave + bwd_ds_row_start(qt, a.causal && !a.ds_uniform, ds_nkt2) * kDsBlockElems);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(off >> 32));
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)off);
    unsigned char* p = reinterpret_cast<unsigned char*>(a.ds + (long long)(((unsigned long long)hi << 32) | lo)) +
                       ds_lane;
    __builtin_nontemporal_store(ds_pend[0], reinterpret_cast<u32x4*>(p));
    __builtin_nontemporal_store(ds_pend[1], reinterpret_cast<u32x4*>(p + 1024));
    __builtin_nontemporal_store(ds_pend[2], reinterpret_cast<u32x4*>(p + 2048));
    __builtin_nontemporal_store(ds_pend[3], reinterpret_cast<u32x4*>(p + 3072));
  };
  auto deposit = [&](int i) __attribute__((always_inline)) {
    if (tid < 2 * kBQ)
      reinterpret_cast<float*>(smem + XR + ((i + shift) % 3) * 512)[tid] = tid < kBQ ? lv * kLog2e : lv;
  };
  if (i_lo < i_hi) issue(i_lo);

  // this wave's operand rows: K (wave A) or V (wave B) of its lane's key
  bf16x8 kv[KT];
  {
    const uint16_t* src = role_a ? kbase : vbase;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < Nk) x = ld_global16(src + (long long)key * kst + 16 * t + 8 * grp);
      kv[t] = as_bf16x8(x);
    }
  }
  f32x16 acc[DB];  // dV^T (wave A) or dK^T (wave B) of this wave's 32 keys
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
  // lane-constant LDS bases: row fragments of Q (A) / dO (B), transposed
  // fragments of dO (A) / Q (B), LSE (A) / Dv (B) of the lane group's rows,
  // this lane's P slot entry
  const unsigned lds0 = (unsigned)reinterpret_cast<uintptr_t>(smem);
  unsigned rbase[KT], tbase[DB][2];
#pragma unroll
  for (int t = 0; t < KT; ++t) rbase[t] = lds0 + (role_a ? QR : OR) + T::row_off(c, grp, t);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) tbase[db][u] = lds0 + (role_a ? OR : QR) + T::tr_off_rows(lane, db, u);
  const unsigned xbase = lds0 + XR + (role_a ? 0u : 4u * kBQ) + 32u * grp;
  const unsigned pbase = lds0 + PR + (unsigned)((kg * 4 * 64 + lane) * 16);

  if (i_lo < i_hi) {
    wait_vmem();
    deposit(i_lo);
  }
  __syncthreads();

  auto rd16 = [&](unsigned base, auto off) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(off)>) return lds_read16_rt(base + (unsigned)off);
    else return lds_read16_imm<decltype(off)::value>(base);
  };
  auto rdtr = [&](unsigned base, auto off) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(off)>) return tr_frag_asm_at<RB>(base, off);
    else return tr_frag_asm_imm<decltype(off)::value, RB>(base);
  };
  auto wr16 = [&](unsigned base, auto off, u32x4 v) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(off)>) lds_write16_rt(base + (unsigned)off, v);
    else lds_write16_imm<decltype(off)::value>(base, v);
  };

  // Fragment reads (inline assembly, waited for explicitly) of 32-row block
  // QB of the tile in buffer bf: rows of Q (A) / dO (B) against this wave's
  // K / V, and transposed fragments of dO (A) / Q (B)
  auto read_rows = [&](auto qb_tag, auto bf, u32x4 (&f)[KT]) __attribute__((always_inline)) {
    constexpr int QB = decltype(qb_tag)::value;
    const auto ro = lin_off<TB, QB * 32 * RB>(bf);
#pragma unroll
    for (int t = 0; t < KT; ++t) f[t] = rd16(rbase[t], ro);
  };
  auto wait_rows = [&](u32x4 (&f)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KT; t += 4) lds_wait_frags(f[t], f[t + 1], f[t + 2], f[t + 3]);
  };
  auto read_tr = [&](auto qb_tag, auto bf, u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
    constexpr int QB = decltype(qb_tag)::value;
    const auto to = lin_off<TB, QB * 32 * RB>(bf);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) f[db][u] = rdtr(tbase[db][u], to);
  };
  auto wait_tr = [&](u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; db += 2) lds_wait_frags(f[db][0], f[db][1], f[db + 1][0], f[db + 1][1]);
  };
  // the block's LSE (A) or Dv (B) of the lane group's rows, and for B the
  // partner's P
  auto read_x = [&](auto qb_tag, auto bf, u32x4 (&x)[6]) __attribute__((always_inline)) {
    constexpr int QB = decltype(qb_tag)::value;
    x[0] = rd16(xbase, lin_off<512, QB * 128>(bf));
    x[1] = rd16(xbase, lin_off<512, QB * 128 + 16>(bf));
    x[2] = rd16(xbase, lin_off<512, QB * 128 + 64>(bf));
    x[3] = rd16(xbase, lin_off<512, QB * 128 + 80>(bf));
    if (!role_a) {
      x[4] = rd16(pbase, lin_off<PSLOT, (QB * 2 + 0) * 1024>(bf));
      x[5] = rd16(pbase, lin_off<PSLOT, (QB * 2 + 1) * 1024>(bf));
    }
  };
  auto wait_x = [&](u32x4 (&x)[6]) __attribute__((always_inline)) {
    lds_wait_frags(x[0], x[1], x[2], x[3]);
    if (!role_a) lds_wait_frags2(x[4], x[5]);
  };
  auto mfma_rows = [&](u32x4 (&f)[KT]) __attribute__((always_inline)) {
    f32x16 r;
#pragma unroll
    for (int v = 0; v < 16; ++v) r[v] = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) r = mfma32x32x16(as_bf16x8(f[t]), kv[t], r);
    return r;
  };
  auto mfma_tr = [&](u32x4 (&f)[DB][2], const bf16x8 (&w)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma32x32x16(as_bf16x8(f[db][0]), w[0], acc[db]);
      acc[db] = mfma32x32x16(as_bf16x8(f[db][1]), w[1], acc[db]);
    }
  };
  // P of block QB from its S (masked on diagonal and tail tiles)
  auto probs = [&](auto masked_tag, auto qb_tag, const f32x16& s, const u32x4 (&x)[6], long long qt0,
                   bf16x8 (&pb)[2]) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int QB = decltype(qb_tag)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lse2 = __uint_as_float(x[2 * u + (e >> 2)][e & 3]);
        float pe = fast_exp2(__builtin_fmaf(s[8 * u + e], sl, -lse2));
        if (MASKED) {
          const int qrow = (int)qt0 + QB * 32 + 16 * u + 8 * grp + e;
          pe = (qrow >= (int)Nq || (a.causal && qrow < key - a.dpos)) ? 0.f : pe;
        }
        p[e] = pe;
      }
      pb[u] = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    }
  };
  // dS of a block from its dP, Dv and the partner's P
  auto grads = [&](const f32x16& dp, const u32x4 (&x)[6], bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pw = as_bf16x8(x[4 + u]);
      float ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ds[e] = (float)pw[e] * (dp[8 * u + e] - __uint_as_float(x[2 * u + (e >> 2)][e & 3]));
      sb[u] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // wave A, tile i (buffer bf): S of both 32-row blocks; P of block 0
  // (written for the partner) next to block 1's S products; dV of block 0
  // next to P of block 1; dV of block 1.  Block 1's LSE is read with block
  // 0's transposed fragments, so it is not held from the start of the tile.
  auto tile_a = [&](auto masked_tag, auto bf, int i) __attribute__((always_inline)) {
    const long long qt0 = (first_tile + i) * kBQ;
    u32x4 f[KT], g[DB][2], x0[6], x1[6];
    bf16x8 p0[2], p1[2];
    read_rows(I0{}, bf, f);
    read_x(I0{}, bf, x0);
    wait_rows(f);
    wait_x(x0);
    const f32x16 s0 = mfma_rows(f);
    read_rows(I1{}, bf, f);
    wait_rows(f);
    const f32x16 s1 = mfma_rows(f);
    probs(masked_tag, I0{}, s0, x0, qt0, p0);
    wr16(pbase, lin_off<PSLOT, 0 * 1024>(bf), as_u32x4(p0[0]));
    wr16(pbase, lin_off<PSLOT, 1 * 1024>(bf), as_u32x4(p0[1]));
    read_tr(I0{}, bf, g);
    read_x(I1{}, bf, x1);
    wait_tr(g);
    wait_x(x1);
    mfma_tr(g, p0);
    probs(masked_tag, I1{}, s1, x1, qt0, p1);
    wr16(pbase, lin_off<PSLOT, 2 * 1024>(bf), as_u32x4(p1[0]));
    wr16(pbase, lin_off<PSLOT, 3 * 1024>(bf), as_u32x4(p1[1]));
    read_tr(I1{}, bf, g);
    wait_tr(g);
    mfma_tr(g, p1);
  };
  // wave B, the tile in buffer bf: the same order with dP, dS, dK (with
  // stored dS, the tile's dS is kept for store_ds, and the previous tile's,
  // ps >= 0, is stored after the dP products)
  auto tile_b = [&](auto bf, int ps) __attribute__((always_inline)) {
    u32x4 f[KT], g[DB][2], x0[6], x1[6];
    bf16x8 d0[2], d1[2];
    read_rows(I0{}, bf, f);
    read_x(I0{}, bf, x0);
    wait_rows(f);
    wait_x(x0);
    const f32x16 dp0 = mfma_rows(f);
    read_rows(I1{}, bf, f);
    wait_rows(f);
    const f32x16 dp1 = mfma_rows(f);
    if constexpr (DS) {
      if (ps >= 0) store_ds(ps);
    }
    grads(dp0, x0, d0);
    if constexpr (DS) {
      ds_pend[0] = as_u32x4(d0[0]);
      ds_pend[1] = as_u32x4(d0[1]);
    }
    read_tr(I0{}, bf, g);
    read_x(I1{}, bf, x1);
    wait_tr(g);
    wait_x(x1);
    mfma_tr(g, d0);
    grads(dp1, x1, d1);
    if constexpr (DS) {
      ds_pend[2] = as_u32x4(d1[0]);
      ds_pend[3] = as_u32x4(d1[1]);
    }
    read_tr(I1{}, bf, g);
    wait_tr(g);
    mfma_tr(g, d1);
  };
  // one iteration of the tile loop: A on tile i (buffer bfa), B on tile
  // i - 1 (buffer bfb), the prefetch of tile i + 1, one barrier
  auto iter = [&](auto masked_tag, int i, auto bfa, auto bfb) __attribute__((always_inline)) {
    if (i + 1 < i_hi) issue(i + 1);
    if (role_a) {
      if (i < i_hi) tile_a(masked_tag, bfa, i);
    } else if (i > i_lo) {
      tile_b(bfb, i - 1 > i_lo ? i - 2 : -1);
    }
    wait_vmem();
    if (i + 1 < i_hi) deposit(i + 1);
    __syncthreads();
  };
  auto bfr = [&](int i) __attribute__((always_inline)) { return (i + shift + 3) % 3; };

  int i = i_lo;
  for (; i < min(head, i_hi); ++i) iter(std::true_type{}, i, bfr(i), bfr(i - 1));
  // unmasked tiles: tile i sits in buffer i - head (mod 3); a range that
  // starts inside them first steps to that pattern
  const int b_end = min(body_end, i_hi);
  for (; i < b_end && (i - head) % 3 != 0; ++i) iter(std::false_type{}, i, bfr(i), bfr(i - 1));
  for (; i + 3 <= b_end; i += 3) {
    iter(std::false_type{}, i, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
    iter(std::false_type{}, i + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    iter(std::false_type{}, i + 2, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  }
  for (; i < b_end; ++i) iter(std::false_type{}, i, bfr(i), bfr(i - 1));
  for (; i <= i_hi; ++i) iter(std::true_type{}, i, bfr(i), bfr(i - 1));
  if constexpr (DS) {
    if (!role_a && i_hi > i_lo) store_ds(i_hi - 1);  // the last tile's dS
  }

  if (key < Nk) {
    float* part = role_a ? dv_part : dk_part;
    float* accp = role_a ? a.dv_acc : a.dk_acc;
    uint16_t* outp = role_a ? a.dv : a.dk;
    const float mul = role_a ? 1.f : a.scale;
#pragma unroll
    for (int dbk = 0; dbk < DB; ++dbk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dbk * 32 + 8 * j + 4 * grp;
        f32x4 w = {acc[dbk][4 * j] * mul, acc[dbk][4 * j + 1] * mul, acc[dbk][4 * j + 2] * mul,
                   acc[dbk][4 * j + 3] * mul};
        if (PARTIAL) {
          *reinterpret_cast<f32x4*>(part + (((rr * a.B + bz) * a.Hq + h) * Nk + key) * D + d) = w;
        } else {
          const long long base = ((bz * a.Hkv + kvh) * Nk + key) * D + d;  // fp32 accumulators
          const long long obf = DENSE ? base : bz * a.ks[0] + kvh * a.ks[1] + key * a.ks[2] + d;  // bf16 dk, dv
          if (a.dkv_mode != 0) {
            f32x4* pa = reinterpret_cast<f32x4*>(accp + base);
            if (a.dkv_mode == 2) w += *pa;  // this call's part added to the running dK, dV
            *pa = w;
          }
          if (outp) *reinterpret_cast<u32x2*>(outp + obf) = pack_bf16x4_bits(w[0], w[1], w[2], w[3]);
        }
      }
  }
}

}  // namespace

// The dK/dV kernel has external linkage: its D = 128 instances for
// contiguous tensors are compiled in units of their own, the same source with
// another instruction-scheduling strategy (attn_bwd_ds.hip: the instances
// that store dS; attn_bwd_dkdv_recompute.hip: those of the recomputing path),
// and only launched from here.
template <int D, bool PARTIAL, bool DENSE, bool DS>
__global__ __launch_bounds__(64 * kSplitWaves, 1) void bwd_dkdv_split_kernel(BwdArgs a, float* __restrict__ dk_part,
                                                                             float* __restrict__ dv_part) {
  bwd_dkdv_body<D, PARTIAL, DENSE, DS>(a, dk_part, dv_part, wg_number(), gridDim.x, gridDim.y);
}

#if defined(LCATTN_BWD_DKDV_UNIT) && LCATTN_BWD_DKDV_UNIT == 1
template __global__ void bwd_dkdv_split_kernel<128, false, true, true>(BwdArgs, float*, float*);
template __global__ void bwd_dkdv_split_kernel<128, true, true, true>(BwdArgs, float*, float*);
}  // namespace lcattn
#elif defined(LCATTN_BWD_DKDV_UNIT) && LCATTN_BWD_DKDV_UNIT == 2
template __global__ void bwd_dkdv_split_kernel<128, false, true, false>(BwdArgs, float*, float*);
template __global__ void bwd_dkdv_split_kernel<128, true, true, false>(BwdArgs, float*, float*);
}  // namespace lcattn
#else
extern template __global__ void bwd_dkdv_split_kernel<128, false, true, true>(BwdArgs, float*, float*);
extern template __global__ void bwd_dkdv_split_kernel<128, true, true, true>(BwdArgs, float*, float*);
extern template __global__ void bwd_dkdv_split_kernel<128, false, true, false>(BwdArgs, float*, float*);
extern template __global__ void bwd_dkdv_split_kernel<128, true, true, false>(BwdArgs, float*, float*);

namespace {

// Independent block-backward calls in one launch (a ring step's calls that
// share neither a query chunk nor a key/value chunk): grid z = call * B +
// batch; call c covers the first ceil(Nk_c / 128) key tiles of the grid.
struct BwdGroup {
  BwdArgs a[kMaxBwdGroup];
  float* dk_part[kMaxBwdGroup];
  float* dv_part[kMaxBwdGroup];
  int n_qtiles[kMaxBwdGroup];
};

template <int D, bool PARTIAL>
__global__ __launch_bounds__(64 * kSplitWaves, 1) void bwd_dkdv_group_kernel(BwdGroup g, int B) {
  const unsigned lin = wg_number();
  const unsigned per_call = gridDim.x * gridDim.y * (unsigned)B;
  const unsigned c = lin / per_call;
  bwd_dkdv_body<D, PARTIAL, true, false>(g.a[c], g.dk_part[c], g.dv_part[c], lin - c * per_call, gridDim.x,
                                         gridDim.y);
}

// dK[b, kvh] = sum over the query ranges that wrote a partial for the key's
// tile (all of them, unsplit: one) and over the G query heads of the group of
// the fp32 partials, written (or added) as the dK, dV modes of the arguments
// say.  One thread per 4 elements.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdArgs a, const float* __restrict__ dk_part,
                                                              const float* __restrict__ dv_part,
                                                              long long kv_heads_total, bool dense) {
  const int G = a.G;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;  // over kv_heads_total * Nk * D / 4
  const long long per_head = a.Nk * D / 4;
  if (idx >= kv_heads_total * per_head) return;
  const long long hk = idx / per_head;        // flattened (b, kvh)
  const long long rem = idx - hk * per_head;  // 4-element slot within the head
  // the query ranges of the split pass that reach the key's 128-key tile (the
  // dK/dV kernel's first query tile and tile count for it)
  int r0 = 0, r1 = 1;
  if (a.rkv > 1) {
    const long long kt0 = rem / (D / 4) / 128 * 128;
    const long long q_first = a.causal ? max(0LL, kt0 - a.dpos) : 0;
    const long long nqt = (a.Nq + kBQ - 1) / kBQ;
    r0 = (int)(q_first / kBQ / a.qst);
    r1 = q_first >= a.Nq ? r0 : (int)((nqt - 1) / a.qst + 1);
  }
  const long long rstride = kv_heads_total * G * per_head * 4;  // one range's partials
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < r1; ++r)
    for (int g = 0; g < G; ++g) {
      const long long src = r * rstride + ((hk * G + g) * per_head + rem) * 4;
      sk += *reinterpret_cast<const f32x4*>(dk_part + src);
      sv += *reinterpret_cast<const f32x4*>(dv_part + src);
    }
  if (a.dkv_mode != 0) {
    f32x4* pk = reinterpret_cast<f32x4*>(a.dk_acc + idx * 4);
    f32x4* pv = reinterpret_cast<f32x4*>(a.dv_acc + idx * 4);
    if (a.dkv_mode == 2) {
      sk += *pk;
      sv += *pv;
    }
    *pk = sk;
    *pv = sv;
  }
  if (a.dk) {
    long long obf = idx * 4;  // contiguous
    if (!dense) {
      const long long b = hk / a.Hkv, kvh = hk % a.Hkv, key = rem / (D / 4);
      obf = b * a.ks[0] + kvh * a.ks[1] + key * a.ks[2] + 4 * (rem % (D / 4));
    }
    *reinterpret_cast<u32x2*>(a.dk + obf) = pack_bf16x4_bits(sk[0], sk[1], sk[2], sk[3]);
    *reinterpret_cast<u32x2*>(a.dv + obf) = pack_bf16x4_bits(sv[0], sv[1], sv[2], sv[3]);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = query rows of HP heads sharing a key/value head
// ---------------------------------------------------------------------------
constexpr int kDqWaves = kBwdDqWaves;
constexpr int kBN = 64;

// DENSE: contiguous [B, H, N, D] tensors (row strides D known at compile
// time, which keeps the kernel within its registers); else the strides of a.
// The kernel body: workgroup number lin (already in XCD-aware order) of a
// grid of nx query tiles x ny head groups x B; the call has n_qtiles <= nx.
template <int D, int HP, bool DENSE>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int n_qtiles, unsigned lin, unsigned nx,
                                            unsigned ny) {
  using T = SwzTile<D>;  // K tiles are read both ways, V tiles by rows: rows swizzle
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int NW = kDqWaves;
  constexpr int SPAN = (NW / HP) * 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[2 * T::BYTES];  // K tile, V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[2 * T::BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char smem2[2 * T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const long long Nq = a.Nq, Nk = a.Nk;
  // XCD-aware order: neighbouring query tiles share an XCD and its L2 while
  // they stream the same key/value tiles; longest causal rows first
  // workgroup-uniform: kept in scalar registers
  const unsigned lxy = __builtin_amdgcn_readfirstlane(lin / nx);
  const int by = __builtin_amdgcn_readfirstlane(lxy % ny);
  const unsigned zz = __builtin_amdgcn_readfirstlane(lxy / ny);  // key range * B + batch
  const int rr = (int)__builtin_amdgcn_readfirstlane(zz / (unsigned)a.B);
  const long long bz = zz - (unsigned)rr * (unsigned)a.B;
  const int qt = n_qtiles - 1 - __builtin_amdgcn_readfirstlane(lin - lxy * nx);
  if (qt < 0) return;  // a grouped launch's grid covers its longest call
  const int h = by * HP + (wave % HP);
  const int kvh = (by * HP) / a.G;
  const long long q_start = (long long)qt * SPAN;
  const long long wq0 = q_start + (long long)(wave / HP) * 32;
  const long long qrow = wq0 + c;
  const int qrow_i = (int)qrow;
  const int klim = (int)Nk;
  const float sl = a.scale * kLog2e;
  const long long hb = (bz * a.Hq + h) * Nq;
  const uint16_t* kbase = DENSE ? a.k + (bz * a.Hkv + kvh) * Nk * D : a.k + bz * a.ks[0] + kvh * a.ks[1];
  const uint16_t* vbase = DENSE ? a.v + (bz * a.Hkv + kvh) * Nk * D : a.v + bz * a.ks[0] + kvh * a.ks[1];

  // keys the workgroup can see
  long long kv_end = Nk;
  if (a.causal) kv_end = max(0LL, min(Nk, min(q_start + SPAN, Nq) + a.dpos));
  // its key tiles [j0, j0 + n_tiles): key range rr of the split pass, else
  // all; a range that no query of the tile sees writes no partial
  const int j0 = rr * a.kst;
  const int n_tiles = (int)max(0LL, min((kv_end + kBN - 1) / kBN, (long long)j0 + a.kst) - j0);
  if (a.rq > 1 && n_tiles == 0) return;
  const int n_sub = 2 * n_tiles;  // 32-key sub-tiles

  typename T::template AsyncLoader<NW> ld;
  ld.init(wave, lane, false, DENSE ? D : a.ks[2]);
  // the wave index in a scalar register: the LDS side of a direct load is
  // then scalar arithmetic; full tiles skip the row clamping
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    const long long r0 = ((long long)j0 + j) * kBN;
    if (r0 + kBN <= Nk) {
      ld.load_full(buf, kbase, r0, wave_s);
      ld.load_full(buf + T::BYTES, vbase, r0, wave_s);
    } else {
      ld.load(buf, kbase, r0, Nk, wave_s);
      ld.load(buf + T::BYTES, vbase, r0, Nk, wave_s);
    }
  };
  if (n_tiles > 0) issue(0, smem0);

  // Q and dO of this lane's query row as B operands (reduction over D)
  bf16x8 qf[KT], of[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qrow < Nq) {
      const long long off =
          (DENSE ? (hb + qrow) * D : bz * a.qs[0] + h * a.qs[1] + qrow * a.qs[2]) + 16 * t + 8 * grp;
      x = ld_global16(a.q + off);
      y = ld_global16(a.d_o + off);
    }
    qf[t] = as_bf16x8(x);
    of[t] = as_bf16x8(y);
  }
  const float lse2 = qrow < Nq ? a.lse[hb + qrow] * kLog2e : INFINITY;  // rows past Nq: P = 0
  const float dvv = qrow < Nq ? a.delta[hb + qrow] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
  bf16x8 dsb[2];  // dS^T of the previous sub-tile, waiting for its product (zero: no-op)
  dsb[0] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  dsb[1] = dsb[0];
  // per-lane LDS offsets: K / V row fragments per step, K^T fragments per
  // column block and 16-row half of a 32-row block
  int roff[KT], toff[DB][2];
#pragma unroll
  for (int t = 0; t < KT; ++t) roff[t] = T::row_off(c, grp, t);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) toff[db][u] = T::tr_off_rows(lane, db, u);

  // dQ^T += K^T dS^T for the previous sub-tile: K^T fragments of its 32 keys
  // (transposing reads through inline assembly, so no wait for the direct
  // loads in flight), then the products
  auto dq_frags = [&](const unsigned char* kb, int half, u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
    const unsigned base = (unsigned)reinterpret_cast<uintptr_t>(kb);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        f[db][u] = tr_frag_asm_at<T::ROW_BYTES>(base, toff[db][u] + 32 * half * T::ROW_BYTES);
  };
  auto dq_products = [&](u32x4 (&f)[DB][2]) __attribute__((always_inline)) {
    if constexpr (DB == 4) {
      lds_wait_frags(f[0][0], f[0][1], f[1][0], f[1][1]);
      lds_wait_frags(f[2][0], f[2][1], f[3][0], f[3][1]);
    } else {
      lds_wait_frags(f[0][0], f[0][1], f[1][0], f[1][1]);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma32x32x16(as_bf16x8(f[db][0]), dsb[0], acc[db]);
      acc[db] = mfma32x32x16(as_bf16x8(f[db][1]), dsb[1], acc[db]);
    }
  };

  // One step t of the pipeline over 32-key sub-tiles: K^T reads of sub-tile
  // t-1, S^T = K Q^T and dP^T = V dO^T of sub-tile t (tile in cur, half
  // `half`), then dQ of sub-tile t-1 next to the elementwise step of t.
  auto step = [&](auto masked_tag, int t, const unsigned char* cur, int half, const unsigned char* prev,
                  int phalf) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    u32x4 f[DB][2];
    dq_frags(prev, phalf, f);
    f32x16 s, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = 0.f;
      dp[v] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const int o = roff[kk] + 32 * half * T::ROW_BYTES;
      s = mfma32x32x16(as_bf16x8(ld_lds16(cur, o)), qf[kk], s);
      dp = mfma32x32x16(as_bf16x8(ld_lds16(cur + T::BYTES, o)), of[kk], dp);
    }
    dq_products(f);
    float ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float p = fast_exp2(__builtin_fmaf(s[v], sl, -lse2));
      if (MASKED) {
        const int key = kBN * j0 + 32 * t + acc_row_pi(v, grp);
        if (key >= klim || (a.causal && key > qrow_i + a.dpos)) p = 0.f;
      }
      ds[v] = p * (dp[v] - dvv);
    }
    dsb[0] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    dsb[1] = pack_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    // S / dP products first, then each dQ product next to a slice of the
    // elementwise step
    constexpr int NMF = 2 * DB;
    constexpr int VPM = (80 + NMF - 1) / NMF;
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KT, 0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
    // keep dS here, next to the products it should overlap (otherwise it may
    // be sunk past the next step's load branch)
    {
      u32x4 d0 = as_u32x4(dsb[0]), d1 = as_u32x4(dsb[1]);
      asm volatile("" : "+v"(d0), "+v"(d1));
      dsb[0] = as_bf16x8(d0);
      dsb[1] = as_bf16x8(d1);
    }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmem();  // this wave's part of the next tile has landed in LDS
    __syncthreads();
  };
  auto buf = [&](int i) __attribute__((always_inline)) {
    const int r = i % 3;
    return r == 0 ? smem0 : (r == 1 ? smem1 : smem2);
  };

  // Tiles [0, n_full) need no element mask for any wave of the workgroup.
  long long full_keys = Nk;
  if (a.causal) full_keys = max(0LL, min(full_keys, q_start + 1 + a.dpos));
  const int n_full = (int)min((long long)n_tiles, max(0LL, full_keys / kBN - j0));

  // Schedule: tile j lives in buffer j % 3 and is read in steps 2j .. 2j+2.
  // Odd steps t issue the direct loads of tile (t+3)/2 (its buffer was last
  // read in step t-1, before the barrier that ended it); even steps end with
  // a barrier after which tile t/2+1 is resident.  Past the last tile the
  // loads repeat it into the free buffer.
  if (n_tiles > 0) {
    wait_vmem();
    __syncthreads();
    issue(min(1, n_tiles - 1), smem1);
    // step 0: no previous sub-tile (dS is zero; the fragments come from
    // tile 0, finite data)
    if (n_full > 0) step(std::false_type{}, 0, smem0, 0, smem0, 0);
    else step(std::true_type{}, 0, smem0, 0, smem0, 0);
    sync();
    int t = 1;
    for (; t + 6 <= 2 * n_full; t += 6) {
      const int j0 = (t - 1) / 2;  // multiple of 3
      issue(min(j0 + 2, n_tiles - 1), smem2);
      step(std::false_type{}, t, smem0, 1, smem0, 0);
      step(std::false_type{}, t + 1, smem1, 0, smem0, 1);
      sync();
      issue(min(j0 + 3, n_tiles - 1), smem0);
      step(std::false_type{}, t + 2, smem1, 1, smem1, 0);
      step(std::false_type{}, t + 3, smem2, 0, smem1, 1);
      sync();
      issue(min(j0 + 4, n_tiles - 1), smem1);
      step(std::false_type{}, t + 4, smem2, 1, smem2, 0);
      step(std::false_type{}, t + 5, smem0, 0, smem2, 1);
      sync();
    }
    for (; t < n_sub; ++t) {
      if (t & 1) issue(min((t + 3) / 2, n_tiles - 1), buf((t + 3) / 2));
      step(std::true_type{}, t, buf(t / 2), t & 1, buf((t - 1) / 2), (t - 1) & 1);
      if (!(t & 1)) sync();
    }
    // dQ of the last sub-tile
    {
      u32x4 f[DB][2];
      dq_frags(buf(n_tiles - 1), 1, f);
      dq_products(f);
    }
    wait_vmem();  // no direct load may still be in flight when the workgroup ends
  }

  if (qrow < Nq) {
    const long long base = (hb + qrow) * D;                                // fp32 accumulator
    const long long obf = DENSE ? base : bz * a.qs[0] + h * a.qs[1] + qrow * a.qs[2];  // bf16 dq
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = db * 32 + 8 * jj + 4 * grp;
        f32x4 g = {acc[db][4 * jj] * a.scale, acc[db][4 * jj + 1] * a.scale, acc[db][4 * jj + 2] * a.scale,
                   acc[db][4 * jj + 3] * a.scale};
        if (a.rq > 1) {  // this key range's part, summed by bwd_dq_reduce
          *reinterpret_cast<f32x4*>(a.dq_part + (long long)rr * a.B * a.Hq * Nq * D + base + d) = g;
          continue;
        }
        if (a.dq_mode != 0) {
          f32x4* p = reinterpret_cast<f32x4*>(a.dq_acc + base + d);
          if (a.dq_mode == 2) g += *p;  // this KV block's part added to the running dQ
          *p = g;
        }
        if (a.dq) *reinterpret_cast<u32x2*>(a.dq + obf + d) = pack_bf16x4_bits(g[0], g[1], g[2], g[3]);
      }
  }
}

template <int D, int HP, bool DENSE>
__global__ __launch_bounds__(64 * kDqWaves, 2) void bwd_dq_kernel(BwdArgs a, int n_qtiles) {
  // XCD-aware order: neighbouring query tiles share an XCD and its L2 while
  // they stream the same key/value tiles; longest causal rows first
  bwd_dq_body<D, HP, DENSE>(a, n_qtiles, wg_number(), gridDim.x, gridDim.y);
}

// dQ = the sum over the key ranges that wrote a partial for the row's query
// tile (tiles of `span` rows, as the dQ kernel's) of the scaled fp32
// partials, written (or added) as the dQ mode of the arguments says.  One
// thread per 4 elements.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(BwdArgs a, int span, bool dense) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;  // over B * Hq * Nq * D / 4
  constexpr long long per_row = D / 4;
  if (idx >= (long long)a.B * a.Hq * a.Nq * per_row) return;
  const long long row_all = idx / per_row;  // flattened (b, h, row)
  const long long row = row_all % a.Nq;
  const long long q_start = row / span * span;
  long long kv_end = a.Nk;
  if (a.causal) kv_end = max(0LL, min(a.Nk, min(q_start + span, a.Nq) + a.dpos));
  const long long tiles = (kv_end + kBN - 1) / kBN;
  const int r1 = (int)min((long long)a.rq, (tiles + a.kst - 1) / a.kst);
  const long long rstride = (long long)a.B * a.Hq * a.Nq * D;  // one range's partials
  f32x4 g = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < r1; ++r) g += *reinterpret_cast<const f32x4*>(a.dq_part + r * rstride + idx * 4);
  if (a.dq_mode != 0) {
    f32x4* p = reinterpret_cast<f32x4*>(a.dq_acc + idx * 4);
    if (a.dq_mode == 2) g += *p;
    *p = g;
  }
  if (a.dq) {
    long long obf = idx * 4;  // contiguous
    if (!dense) {
      const long long bh = row_all / a.Nq;
      obf = bh / a.Hq * a.qs[0] + bh % a.Hq * a.qs[1] + row * a.qs[2] + 4 * (idx % per_row);
    }
    *reinterpret_cast<u32x2*>(a.dq + obf) = pack_bf16x4_bits(g[0], g[1], g[2], g[3]);
  }
}

template <int D, int HP>
__global__ __launch_bounds__(64 * kDqWaves, 2) void bwd_dq_group_kernel(BwdGroup g, int B) {
  const unsigned lin = wg_number();
  const unsigned per_call = gridDim.x * gridDim.y * (unsigned)B;
  const unsigned c = lin / per_call;
  bwd_dq_body<D, HP, true>(g.a[c], g.n_qtiles[c], lin - c * per_call, gridDim.x, gridDim.y);
}

// ---------------------------------------------------------------------------
// dQ = scale dS K from the dS^T blocks the dK/dV pass stored (the dQ pass
// without its two recomputed products).  A workgroup owns 256 query rows (4
// query tiles) of one query head, 8 waves: a pair per query tile (64 rows),
// each wave one half of the head dimension.  It walks the key tiles its rows
// see: per key tile, the K tile and the 4 dS^T blocks of its query tiles
// arrive by direct loads (three LDS buffers, two tiles ahead, one barrier
// per tile), and each wave adds dQ^T += K^T dS^T for its rows and head dims,
// both operands through the transposing LDS read (A: K^T, 32 head dims x 16
// keys, each fragment used for both 32-row blocks; B: dS^T, 16 keys x 32
// query rows).  Bound by reading dS from HBM; the head-dimension split
// reads a fifth less from LDS than 8 waves of 32 rows with every head dim
// (measured 2% faster).
// ---------------------------------------------------------------------------
constexpr int kDsWaves = 8;

template <int D, bool DENSE>
__global__ __launch_bounds__(64 * kDsWaves, 1) void bwd_dq_ds_kernel(BwdArgs a, int n_groups) {
  using T = SwzTile<D>;   // K tiles, read transposed only
  using S = SwzTile<64>;  // dS^T blocks: 64 key rows x 64 query columns
  constexpr int DB = D / 32;
  constexpr int STAGE = T::BYTES + 4 * S::BYTES;
  constexpr int NL = T::LOADS / kDsWaves + 4;  // direct loads per wave and stage
  __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, grp = lane >> 5;
  const unsigned lin = wg_number();
  const unsigned lxy = __builtin_amdgcn_readfirstlane(lin / gridDim.x);
  const int h = (int)__builtin_amdgcn_readfirstlane(lxy % gridDim.y);
  const long long bz = __builtin_amdgcn_readfirstlane(lxy / gridDim.y);
  // query group g: tiles 4 g .. 4 g + 3, longest rows first
  const int g = n_groups - 1 - (int)__builtin_amdgcn_readfirstlane(lin - lxy * gridDim.x);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const long long Nq = a.Nq, Nk = a.Nk;
  const long long nqt = (Nq + 63) / 64, nkt = (Nk + 63) / 64, nkt2 = (Nk + 127) / 128 * 2;
  const int kvh = h / a.G;
  const int row_causal = a.causal && !a.ds_uniform;  // compact rows
  // key tiles whose stored blocks a query tile's row holds: those of the
  // key-tile pairs whose dK/dV workgroups reach the tile (causal: a pair
  // starts at query row 128 x - dpos), at most the tiles of Nk
  auto kt_end = [&](long long qt) __attribute__((always_inline)) -> long long {
    if (!a.causal) return nkt;
    const long long L = (Nq < 64 * qt + 64 ? Nq : 64 * qt + 64) + a.dpos;  // pairs x with 128 x < L
    long long x = L > 0 ? (L + 127) / 128 : 0;
    x = x < nkt2 / 2 ? x : nkt2 / 2;
    return 2 * x < nkt ? 2 * x : nkt;
  };
  const long long qt0 = 4LL * g;
  const int n_kt = (int)kt_end(min(qt0 + 3, nqt - 1));  // (nondecreasing in qt)
  const long long qt_w = qt0 + (wave_s >> 1);  // this wave's query tile (both 32-row blocks; head dims 64 (wave % 2) ..)
  const int n_kt_w = qt_w < nqt ? (int)kt_end(qt_w) : 0;
  const uint16_t* kbase = DENSE ? a.k + (bz * a.Hkv + kvh) * Nk * D : a.k + bz * a.ks[0] + kvh * a.ks[1];
  const uint16_t* dsh = a.ds + (bz * a.Hq + h) * a.ds_head;

  typename T::template AsyncLoader<kDsWaves> kld;
  kld.init(wave, lane, true, DENSE ? D : a.ks[2]);
  // a dS^T block into LDS as a row-major tile (64 key rows of 8 units of 8
  // query columns, units XOR-swizzled per row as S::off_rows): wave w fills
  // LDS bytes [w KiB, w KiB + 1 KiB), lane i its 16 bytes at 16 i, i.e. row
  // r = 8 w + i / 8, LDS unit i % 8, which holds query unit uq = (i % 8) ^
  // swz(r); in the stored order that unit of key r = 32 kh + c is unit
  // (kh * 4 + uq / 2) * 64 + (uq % 2) * 32 + c
  unsigned s_goff;
  {
    const int slot = wave * 64 + lane, r = slot >> 3;
    const int uq = (slot & 7) ^ S::swz_rows(r);
    s_goff = (unsigned)((((r >> 5) * 4 + (uq >> 1)) * 64 + (uq & 1) * 32 + (r & 31)) * 16);
  }
  // stage kt into buffer st: the K tile and the four dS^T blocks (a query
  // tile past the last, or whose row ends before kt, loads a block of its
  // row that it then ignores: every wave issues NL loads per stage)
  auto issue = [&](int kt, int st) __attribute__((always_inline)) {
    unsigned char* buf = smem + st * STAGE;
    kld.load(buf, kbase, (long long)kt * 64, Nk, wave_s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long long qt = min(qt0 + j, nqt - 1);
      // (a tile whose row ends before kt, or that sees no key at all, loads a
      // block of its row that it then ignores)
      const long long kb = max(0LL, min((long long)kt, kt_end(qt) - 1));
      const unsigned char* src = reinterpret_cast<const unsigned char*>(
          dsh + (bwd_ds_row_start(qt, row_causal, nkt2) + kb) * kDsBlockElems);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + s_goff),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(buf + T::BYTES + j * S::BYTES) + wave_s * 1024),
                                       16, 0, 0);
    }
  };

  constexpr int HB = DB / 2;  // head-dim blocks of this wave
  f32x16 acc[2][HB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < HB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[qb][db][v] = 0.f;
  const unsigned lds0 = (unsigned)reinterpret_cast<uintptr_t>(smem);
  unsigned koff[HB];
#pragma unroll
  for (int db = 0; db < HB; ++db) koff[db] = lds0 + T::tr_off(lane, (wave & 1) * HB + db);
  unsigned soff[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) soff[qb] = lds0 + T::BYTES + (wave >> 1) * S::BYTES + S::tr_off(lane, qb);

  if (n_kt > 0) issue(0, 0);
  if (n_kt > 1) issue(1, 1);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int st = kt % 3;
    if (kt + 1 < n_kt) wait_vmem_n<NL>();  // stage kt has landed (kt + 1 may be in flight)
    else wait_vmem();
    // every wave's part of stage kt is in LDS, and every wave's reads of the
    // buffer the next issue overwrites (stage kt - 1, waited for before its
    // products) are done: a plain barrier, no fence that would also wait for
    // stage kt + 1
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < n_kt) issue(kt + 2, (kt + 2) % 3);
    if (kt < n_kt_w) {
      const unsigned sh = (unsigned)(st * STAGE);
      // keys past Nk in the last tile: the dK/dV pass does not mask them
      // (their scores come from zero K rows and are visible wherever the
      // positions allow: always without the causal mask, and with it when
      // the queries lie past the keys), and their K rows here repeat row
      // Nk - 1
      const bool tail = kt == nkt - 1 && (Nk & 63);
      const int lim = (int)(Nk - (long long)kt * 64);
      constexpr int NR = 4 + 2 * HB;  // LDS reads per reduction step
      u32x4 fb[4][2], fa[4][HB];
#pragma unroll
      for (int ks = 0; ks < 5; ++ks) {
        if (ks < 4) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) fb[ks][qb] = tr_frag_asm_at<S::ROW_BYTES>(soff[qb] + sh, ks * 16 * S::ROW_BYTES);
#pragma unroll
          for (int db = 0; db < HB; ++db) fa[ks][db] = tr_frag_asm_at<T::ROW_BYTES>(koff[db] + sh, ks * 16 * T::ROW_BYTES);
        }
        const int m = ks - 1;  // step multiplied after this one's reads are issued
        if (m < 0) continue;
        // reads complete in issue order: step m has landed once only the
        // reads of step m + 1 (if issued) are outstanding
        if constexpr (HB == 2) {
          if (m < 3) lds_wait_frags_n<NR>(fb[m][0], fb[m][1], fa[m][0], fa[m][1]);
          else lds_wait_frags_n<0>(fb[m][0], fb[m][1], fa[m][0], fa[m][1]);
        } else {
          if (m < 3) lds_wait_frags_n<NR>(fb[m][0], fb[m][1], fa[m][0]);
          else lds_wait_frags_n<0>(fb[m][0], fb[m][1], fa[m][0]);
        }
        if (tail) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int k0 = 16 * m + 8 * grp + 2 * w;  // keys k0 (low half), k0 + 1 (high half)
              fb[m][qb][w] &= (k0 < lim ? 0x0000FFFFu : 0u) | (k0 + 1 < lim ? 0xFFFF0000u : 0u);
            }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int db = 0; db < HB; ++db)
            acc[qb][db] = mfma32x32x16(as_bf16x8(fa[m][db]), as_bf16x8(fb[m][qb]), acc[qb][db]);
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const long long qrow = qt_w * 64 + 32 * qb + c;
    if (qt_w < nqt && qrow < Nq) {
      const long long obf = DENSE ? ((bz * a.Hq + h) * Nq + qrow) * D : bz * a.qs[0] + h * a.qs[1] + qrow * a.qs[2];
#pragma unroll
      for (int db = 0; db < HB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = ((wave & 1) * HB + db) * 32 + 8 * jj + 4 * grp;
          f32x4 gq = {acc[qb][db][4 * jj] * a.scale, acc[qb][db][4 * jj + 1] * a.scale,
                      acc[qb][db][4 * jj + 2] * a.scale, acc[qb][db][4 * jj + 3] * a.scale};
          if (a.dq_mode != 0) {  // fp32 accumulator (contiguous): overwritten, or added to
            f32x4* pa = reinterpret_cast<f32x4*>(a.dq_acc + ((bz * a.Hq + h) * Nq + qrow) * D + d);
            if (a.dq_mode == 2) gq += *pa;
            *pa = gq;
          }
          if (a.dq) *reinterpret_cast<u32x2*>(a.dq + obf + d) = pack_bf16x4_bits(gq[0], gq[1], gq[2], gq[3]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Small problems: the dQ pass beside the dK/dV pass.  Both read only the
// inputs and Dv and write disjoint outputs, so when the dK/dV grid would not
// fill the GPU twice over, the dQ pass runs on a side stream of the library's
// own, forked from the caller's stream after Dv and joined back into it after
// the dK/dV launches (events): every launch of a call stays ordered on the
// caller's stream.  Each caller stream gets its own side stream and pair of
// events (default priority; created at its first such call with the stream's
// device current, kept until the process ends), so a side stream only ever
// carries work forked from one caller stream, in that stream's order, and adds
// no dependency between different caller streams.  At most kSideSlots caller
// streams get one; calls on further streams run on their stream alone.  A
// mutex keeps concurrent calls from interleaving their fork/join pairs.
// ---------------------------------------------------------------------------
constexpr int kSideSlots = 64;
struct SideStream {
  bool used = false;
  int dev = -1;
  hipStream_t caller = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int cus = 0;
};
std::mutex g_side_mu;
SideStream g_side[kSideSlots];

// The side stream of `caller` (nullptr with hipSuccess when every slot is
// taken); g_side_mu must be held.
hipError_t side_stream(hipStream_t caller, SideStream** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(caller, &dev);
  if (e != hipSuccess) return e;
  SideStream* slot = nullptr;
  for (SideStream& ss : g_side) {
    if (ss.used && ss.dev == dev && ss.caller == caller) {
      *out = &ss;
      return hipSuccess;
    }
    if (!ss.used && !slot) slot = &ss;
  }
  if (!slot) return hipSuccess;
  int cur = 0;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  SideStream n;
  n.used = true;
  n.dev = dev;
  n.caller = caller;
  e = hipDeviceGetAttribute(&n.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
  const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
  if (e != hipSuccess || e2 != hipSuccess) {
    if (n.join) (void)hipEventDestroy(n.join);
    if (n.fork) (void)hipEventDestroy(n.fork);
    if (n.s) (void)hipStreamDestroy(n.s);
    return e != hipSuccess ? e : e2;
  }
  *slot = n;
  *out = slot;
  return hipSuccess;
}

// Where a call's dQ pass goes.  begin() decides (the dK/dV pass has fewer
// than two workgroups per compute unit and the caller allows a second
// stream) and forks; end() joins, after the dK/dV launches were enqueued.
class DqStream {
 public:
  hipError_t begin(hipStream_t caller, bool allow, long long dkdv_workgroups) {
    caller_ = caller;
    if (!allow) return hipSuccess;
    lock_ = std::unique_lock<std::mutex>(g_side_mu);
    SideStream* ss = nullptr;
    hipError_t e = side_stream(caller, &ss);
    if (e != hipSuccess) return e;
    if (!ss || dkdv_workgroups >= 2LL * ss->cus) {
      lock_.unlock();
      return hipSuccess;
    }
    if ((e = hipEventRecord(ss->fork, caller)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
    side_ = ss;
    return hipSuccess;
  }
  hipStream_t stream() const { return side_ ? side_->s : caller_; }
  hipError_t end() {
    if (!side_) return hipSuccess;
    hipError_t e = hipEventRecord(side_->join, side_->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(caller_, side_->join, 0);
    side_ = nullptr;
    return e;
  }

 private:
  hipStream_t caller_ = nullptr;
  SideStream* side_ = nullptr;
  std::unique_lock<std::mutex> lock_;
};

template <int D>
hipError_t launch_delta(const uint16_t* o, const uint16_t* d_o, float* delta, int B, int H, long long N,
                        const long long (&st)[3], hipStream_t stream) {
  const long long threads = N * (D / 8);
  LCATTN_LAUNCH("bwd_delta_kernel", (bwd_delta_kernel<D>), dim3((unsigned)((threads + 255) / 256), (unsigned)H,
                                                                (unsigned)B),
                dim3(256), 0, stream, o, d_o, delta, N, st[0], st[1], st[2]);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a0, int B, hipStream_t stream, bool allow_side, bool split) {
  hipError_t e;
  BwdArgs a = a0;
  a.B = B;
  // stored dS: the dQ pass becomes the product pass after dK/dV (unsplit)
  const bool ds = a.ds != nullptr;
  const BwdSplit sp = split && !ds ? bwd_split_plan(B, a.Hq, a.Hkv, a.Nq, a.Nk, D) : BwdSplit{};
  a.rkv = sp.rkv;
  a.qst = sp.qst;
  a.rq = sp.rq;
  a.kst = sp.kst;
  a.dq_part = sp.rq > 1 ? a.part + bwd_split_part_floats(B, a.Hq, a.Hkv, a.Nk, D, sp) : nullptr;
  const bool dense = a.qs[0] == 0 && a.qs[1] == 0 && a.qs[2] == 0 && a.ks[0] == 0 && a.ks[1] == 0 && a.ks[2] == 0;
  if (a.qs[0] == 0 && a.qs[1] == 0 && a.qs[2] == 0) {
    a.qs[2] = D;
    a.qs[1] = a.Nq * D;
    a.qs[0] = a.Hq * a.Nq * D;
  }
  if (a.ks[0] == 0 && a.ks[1] == 0 && a.ks[2] == 0) {
    a.ks[2] = D;
    a.ks[1] = a.Nk * D;
    a.ks[0] = a.Hkv * a.Nk * D;
  }
  // 128 keys per workgroup; grid z = query range * B + batch
  const dim3 kgrid((unsigned)((a.Nk + 127) / 128), (unsigned)a.Hq, (unsigned)(B * a.rkv));
  const int HP = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);
  const long long span = (kDqWaves / HP) * 32;
  const int n_qt = (int)((a.Nq + span - 1) / span);
  dim3 grid((unsigned)n_qt, (unsigned)(a.Hq / HP), (unsigned)(B * a.rq));  // z = key range * B + batch
  if (!grid_fits(kgrid) || !grid_fits(grid)) return hipErrorInvalidConfiguration;
  if (a.o) {
    e = launch_delta<D>(a.o, a.d_o, a.delta, B, a.Hq, a.Nq, a.qs, stream);
    if (e != hipSuccess) return e;
  }
  const int n_groups = (int)((a.Nq + 255) / 256);
  const dim3 sgrid((unsigned)n_groups, (unsigned)a.Hq, (unsigned)B);
  if (ds && !grid_fits(sgrid)) return hipErrorInvalidConfiguration;
  DqStream dqs;
  if ((e = dqs.begin(stream, allow_side && !ds, (long long)kgrid.x * kgrid.y * B)) != hipSuccess) return e;
  const hipStream_t qstream = dqs.stream();
  // the dQ pass first: on the side stream it then runs beside the dK/dV pass
  if (ds) {
    // after the dK/dV pass, below
  } else if (dense) {
    if (HP == 4)
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 4, true>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
    else if (HP == 2)
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 2, true>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
    else
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 1, true>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
  } else {
    if (HP == 4)
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 4, false>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
    else if (HP == 2)
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 2, false>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
    else
      LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_kernel<D, 1, false>), grid, dim3(64 * kDqWaves), 0, qstream, a, n_qt);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!ds && a.rq > 1) {
    const long long slots = (long long)B * a.Hq * a.Nq * D / 4;
    LCATTN_LAUNCH("bwd_dq_reduce_kernel", (bwd_dq_reduce_kernel<D>), dim3((unsigned)((slots + 255) / 256)), dim3(256),
                  0, qstream, a, (int)span, dense);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const bool partial = a.G != 1 || a.rkv > 1;
    float* dk_part = partial ? a.part : nullptr;
    float* dv_part = partial ? dk_part + (long long)a.rkv * B * a.Hq * a.Nk * D : nullptr;
    const dim3 blk(64 * kSplitWaves);
#define LCATTN_DKDV(P, DN)                                                                                        \
  do {                                                                                                            \
    if (ds)                                                                                                       \
      LCATTN_LAUNCH("bwd_dkdv_kernel", (bwd_dkdv_split_kernel<D, P, DN, true>), kgrid, blk, 0, stream, a, dk_part, \
                    dv_part);                                                                                     \
    else                                                                                                          \
      LCATTN_LAUNCH("bwd_dkdv_kernel", (bwd_dkdv_split_kernel<D, P, DN, false>), kgrid, blk, 0, stream, a,         \
                    dk_part, dv_part);                                                                            \
  } while (0)
    if (!partial) {
      if (dense) LCATTN_DKDV(false, true);
      else LCATTN_DKDV(false, false);
    } else {
      if (dense) LCATTN_DKDV(true, true);
      else LCATTN_DKDV(true, false);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const long long slots = (long long)B * a.Hkv * a.Nk * D / 4;
      LCATTN_LAUNCH("bwd_dkdv_reduce_kernel", (bwd_dkdv_reduce_kernel<D>), dim3((unsigned)((slots + 255) / 256)),
                    dim3(256), 0, stream, a, dk_part, dv_part, (long long)B * a.Hkv, dense);
    }
#undef LCATTN_DKDV
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ds) {
    if (dense)
      LCATTN_LAUNCH("bwd_dq_ds_kernel", (bwd_dq_ds_kernel<D, true>), sgrid, dim3(64 * kDsWaves), 0, stream, a,
                    n_groups);
    else
      LCATTN_LAUNCH("bwd_dq_ds_kernel", (bwd_dq_ds_kernel<D, false>), sgrid, dim3(64 * kDsWaves), 0, stream, a,
                    n_groups);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return dqs.end();
}

// One launch per kernel for up to kMaxBwdGroup block calls (dense tensors,
// Dv given, shared B, Hq, Hkv, D, scale and mask kind).
template <int D>
hipError_t launch_d_group(const BwdArgs* calls, int n, int B, hipStream_t stream, bool allow_side) {
  hipError_t e;
  BwdGroup g{};
  long long nk_tiles = 0;
  const int G = calls[0].G;
  const int HP = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const long long span = (kDqWaves / HP) * 32;
  int nq_tiles = 0;
  for (int c = 0; c < n; ++c) {
    BwdArgs a = calls[c];
    a.B = B;  // grid z = call * B + batch: the bodies see z = batch (one range)
    a.rkv = a.rq = 1;
    a.qst = a.kst = 1 << 30;
    a.qs[2] = D; a.qs[1] = a.Nq * D; a.qs[0] = a.Hq * a.Nq * D;
    a.ks[2] = D; a.ks[1] = a.Nk * D; a.ks[0] = a.Hkv * a.Nk * D;
    g.a[c] = a;
    g.dk_part[c] = G == 1 ? nullptr : a.part;
    g.dv_part[c] = G == 1 ? nullptr : a.part + (long long)B * a.Hq * a.Nk * D;
    g.n_qtiles[c] = (int)((a.Nq + span - 1) / span);
    nk_tiles = std::max<long long>(nk_tiles, (a.Nk + 127) / 128);
    nq_tiles = std::max(nq_tiles, g.n_qtiles[c]);
  }
  const dim3 kgrid((unsigned)nk_tiles, (unsigned)calls[0].Hq, (unsigned)(B * n));
  const dim3 qgrid((unsigned)nq_tiles, (unsigned)(calls[0].Hq / HP), (unsigned)(B * n));
  if (!grid_fits(kgrid) || !grid_fits(qgrid)) return hipErrorInvalidConfiguration;
  DqStream dqs;
  if ((e = dqs.begin(stream, allow_side, (long long)kgrid.x * kgrid.y * kgrid.z)) != hipSuccess) return e;
  const hipStream_t qstream = dqs.stream();
  if (HP == 4)
    LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_group_kernel<D, 4>), qgrid, dim3(64 * kDqWaves), 0, qstream, g, B);
  else if (HP == 2)
    LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_group_kernel<D, 2>), qgrid, dim3(64 * kDqWaves), 0, qstream, g, B);
  else
    LCATTN_LAUNCH("bwd_dq_kernel", (bwd_dq_group_kernel<D, 1>), qgrid, dim3(64 * kDqWaves), 0, qstream, g, B);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (G == 1)
    LCATTN_LAUNCH("bwd_dkdv_kernel", (bwd_dkdv_group_kernel<D, false>), kgrid, dim3(64 * kSplitWaves), 0, stream, g,
                  B);
  else
    LCATTN_LAUNCH("bwd_dkdv_kernel", (bwd_dkdv_group_kernel<D, true>), kgrid, dim3(64 * kSplitWaves), 0, stream, g, B);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (G != 1)
    for (int c = 0; c < n; ++c) {
      const long long slots = (long long)B * g.a[c].Hkv * g.a[c].Nk * D / 4;
      LCATTN_LAUNCH("bwd_dkdv_reduce_kernel", (bwd_dkdv_reduce_kernel<D>), dim3((unsigned)((slots + 255) / 256)),
                    dim3(256), 0, stream, g.a[c], g.dk_part[c], g.dv_part[c], (long long)B * g.a[c].Hkv, true);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  return dqs.end();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free backward (attn_bwd_noalloc): the same Dv and
// per-query-head dK/dV partials as the caller's workspace of attn_bwd, in a
// file-scope device array.  Every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as memory:
// its device address comes from hipGetSymbolAddress, once per device with
// that device current, and is kept per device.  Nothing in it must start at
// zero (every word a launch reads was written earlier in the same launch
// sequence); calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attn_bwd_group(const BwdArgs* calls, int n, int B, int D, hipStream_t stream) {
  return D == 64 ? launch_d_group<64>(calls, n, B, stream, true) : launch_d_group<128>(calls, n, B, stream, true);
}

hipError_t launch_attn_bwd(const BwdArgs& a, int B, int D, hipStream_t stream, bool allow_side, bool split) {
  return D == 64 ? launch_d<64>(a, B, stream, allow_side, split) : launch_d<128>(a, B, stream, allow_side, split);
}

hipError_t launch_bwd_delta(const uint16_t* o, const uint16_t* d_o, float* delta, long long rows, int D,
                            hipStream_t stream) {
  const long long st[3] = {0, 0, D};  // contiguous rows
  return D == 64 ? launch_delta<64>(o, d_o, delta, 1, 1, rows, st, stream)
                 : launch_delta<128>(o, d_o, delta, 1, 1, rows, st, stream);
}

}  // namespace lcattn
#endif  // LCATTN_BWD_DKDV_UNIT
