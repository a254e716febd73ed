// device_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// Everything here is written for CDNA4 (gfx950, wave64): the 32x32x16 bf16
// MFMA with fp32 accumulation, 16-byte global/LDS vectors, the hardware exp2
// and log2 (v_exp_f32 / v_log_f32) and the hardware round-to-nearest-even
// bf16 pack (v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32) on the matrix cores.  Operand layout of
// lane l (r = l % 32, grp = l / 32): A gives row r, B gives column r, each
// with 8 bf16 along the reduction axis (the same 8 reduction indices for A and
// B in a lane group).  The accumulator gives column r and rows
// 8*(v/4) + 4*grp + v%4 for v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 ld_lds16(const unsigned char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void st_lds16(unsigned char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ __forceinline__ void st_lds8(unsigned char* base, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + off) = v;
}

// Eight fp32 values -> eight bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                              float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

__device__ __forceinline__ u32x2 pack_bf16x4_bits(float a0, float a1, float a2, float a3) {
  bf16x4 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  return __builtin_bit_cast(u32x2, r);
}

// Rows of a 32-row MFMA block are fed in the order pi(m) = m with bits 2 and 3
// swapped.  The accumulator then holds, in lane group grp, registers 8u..8u+7
// for the contiguous index range 16u + 8*grp .. +7 (u = 0, 1), which is exactly
// the reduction-operand layout of the next MFMA: results flow from one
// contraction into the next without leaving registers.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Index (within a 32-row block fed in pi order) of accumulator register v of a
// lane in group grp: 16*(v/8) + 8*grp + v%8.
__device__ __forceinline__ int acc_row_pi(int v, int grp) { return 16 * (v >> 3) + 8 * grp + (v & 7); }

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows x D bf16, row-major, 16-byte units XOR-swizzled per row.
//
// Two read patterns touch every tile:
//  (a) row fragments: lanes 0..31 read rows pi(0..31) (one 16-byte unit each),
//      the A operand of a product that reduces over D;
//  (b) transposed fragments via ds_read_b64_tr_b16: a 16-lane group reads
//      8-byte chunks of 4 consecutive rows, the A operand of a product that
//      reduces over the tile rows.
// f(row) = ((row & 3) << 1) | ((row >> 3) & 1) gives the 8 lanes of one LDS
// cycle in (a) 8 distinct units modulo 8, and the 4 rows x 2 units of one
// 16-lane cycle in (b) 8 distinct units modulo 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }

// Swizzles measured for the two read patterns on gfx950 (64-row x 256-byte
// tiles, eight waves reading).  tile_swz above reaches about 115 B/clk/CU for
// either pattern; these reach about 170:
//   rows: s(r) = 4 (r & 3) + ((r >> 3) & 3)      row fragments ~170, transposed ~180
//   tr:   s(r) = 4 (r & 3) + 2 ((r >> 3) & 1)    transposed fragments ~173
// Neither depends on row bit 2, so the second half of a transposed fragment
// (4 rows further) is an immediate offset.  The rows swizzle does not depend
// on row bits above 4 (row steps of 32 are immediates) and serves tiles read
// both ways; the tr swizzle does not depend on bits above 3 (row steps of 16
// are immediates) and serves tiles read only through the transposing read.
// D = 64 (128-byte rows) keeps tile_swz for both.
template <int D>
struct SwzTile {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int UNITS = D / 8;
  static constexpr int BYTES = 64 * ROW_BYTES;
  static constexpr int LOADS = BYTES / (64 * 16);

  __device__ static int swz_rows(int r) { return D == 128 ? (((r & 3) << 2) | ((r >> 3) & 3)) : tile_swz(r); }
  __device__ static int swz_tr(int r) { return D == 128 ? (((r & 3) << 2) | (((r >> 3) & 1) << 1)) : tile_swz(r); }
  __device__ static int swz(bool tr, int r) { return tr ? swz_tr(r) : swz_rows(r); }

  // Byte offset of logical unit u of row r in a rows-swizzled tile.
  __device__ static int off_rows(int r, int u) { return r * ROW_BYTES + ((u ^ swz_rows(r)) << 4); }

  // Direct global->LDS loads of rows [r0, r0 + 64) of a row-major
  // [rows_total, D] bf16 matrix.  Wave w of NW waves issues loads w, w+NW, ...;
  // load n fills LDS bytes [n KiB, n KiB + 1 KiB), lane i its 16 bytes at 16 i.
  // The per-lane part (which unit of which row) is fixed for the kernel and
  // kept in registers; the per-tile part is a base that is uniform over the
  // wave.  Rows past rows_total read row rows_total - 1 (finite data that the
  // callers mask).
  template <int NW>
  struct AsyncLoader {
    static constexpr int N = LOADS / NW;
    static_assert(LOADS % NW == 0, "tile loads split evenly over the waves");
    unsigned off[N];  // byte offset of this lane's unit within the tile (global side)
    int row[N];       // tile row of that unit
    long long rs;     // elements between consecutive rows of the matrix (>= D)
    // row_stride < 2^24 (checked on the host) keeps the offsets in 32 bits
    __device__ void init(int wave, int lane, bool tr, long long row_stride = D) {
      rs = row_stride;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int n = wave + i * NW;
        const int slot = n * 64 + lane;
        const int r = slot / UNITS, up = slot % UNITS;
        row[i] = r;
        off[i] = (unsigned)(r * row_stride + 8 * (up ^ swz(tr, r))) * 2u;
      }
    }
    // A tile whose 64 rows all exist (r0 + 64 <= rows_total); wave must be
    // wave-uniform in a scalar register (readfirstlane), so that only the
    // per-lane offset is a vector value.
    __device__ void load_full(unsigned char* lds, const uint16_t* g, long long r0, int wave) const {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(g + r0 * rs);
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + off[i]),
                                         reinterpret_cast<__attribute__((address_space(3))) void*>(
                                             reinterpret_cast<uintptr_t>(lds) + (wave + i * NW) * 1024),
                                         16, 0, 0);
    }
    __device__ void load(unsigned char* lds, const uint16_t* g, long long r0, long long rows_total, int wave) const {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(g + r0 * rs);
      if (r0 + 64 <= rows_total) {
        load_full(lds, g, r0, wave);
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const long long gr = r0 + row[i];
          const long long back = gr < rows_total ? 0 : gr - (rows_total - 1);  // rows to step back
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + off[i] - back * rs * 2),
                                           reinterpret_cast<__attribute__((address_space(3))) void*>(
                                               reinterpret_cast<uintptr_t>(lds) + (wave + i * NW) * 1024),
                                           16, 0, 0);
        }
      }
    }
  };

  // Register-staged tile load into a rows-swizzled tile: NT threads fetch
  // rows [r0, r0 + 64) into CH 16-byte registers each, then store them.  Rows
  // past rows_total read row rows_total - 1.
  template <int NT>
  struct Stage {
    static constexpr int CH = 64 * UNITS / NT;
    static_assert(CH >= 1 && 64 * UNITS % NT == 0, "threads must divide the tile");
    u32x4 r[CH];
    __device__ void load(const uint16_t* g, long long r0, long long rows_total, int tid) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int id = tid + i * NT;
        const int row = id / UNITS, u = id % UNITS;
        long long gr = r0 + row;
        gr = gr < rows_total ? gr : rows_total - 1;
        r[i] = ld_global16(g + gr * D + 8 * u);
      }
    }
    __device__ void store(unsigned char* lds, int tid) const {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int id = tid + i * NT;
        const int row = id / UNITS, u = id % UNITS;
        st_lds16(lds, off_rows(row, u), r[i]);
      }
    }
  };

  // Byte offset of the row fragment of step t for lane (c, grp) in a
  // rows-swizzled tile: row pi(c), dims 16 t + 8 grp .. +7.  Rows 32 k
  // further are + 32 k ROW_BYTES.
  __device__ static int row_off(int c, int grp, int t) {
    const int r = swap_bits23(c);
    return r * ROW_BYTES + (((2 * t + grp) ^ swz_rows(r)) << 4);
  }

  // Byte offset of the first transposing read of the fragment
  // T[r0 + 8 grp + e][32 db + c] (e = 0..7) for lane l; the second read is 4
  // rows further.  tr_off: tr-swizzled tile, r0 = 0 (multiples of 16 are
  // + r0 ROW_BYTES).  tr_off_rows: rows-swizzled tile, r0 = 16 u16 (multiples
  // of 32 are + r0 ROW_BYTES).
  __device__ static int tr_off_sw(int lane, int db, int r0, bool tr) {
    const int gi = lane >> 4, s = lane & 15;
    const int row = r0 + 8 * (gi >> 1) + (s >> 2);
    const int x = 4 * db + 2 * (gi & 1) + ((s & 3) >> 1);
    return row * ROW_BYTES + ((x ^ swz(tr, row)) << 4) + ((s & 1) << 3);
  }
  __device__ static int tr_off(int lane, int db) { return tr_off_sw(lane, db, 0, true); }
  __device__ static int tr_off_rows(int lane, int db, int u16) { return tr_off_sw(lane, db, 16 * u16, false); }
};

// Transposed fragment through inline assembly.  The compiler does not see
// this as an LDS access, so it inserts neither the vmcnt wait it would place
// before a transposing read while direct loads are in flight nor the lgkmcnt
// wait before its result is used: callers must run lds_wait_frags on the
// fragments before using them.
template <int ROW_BYTES>
__device__ __forceinline__ u32x4 tr_frag_asm_at(unsigned lds_base, int off) {
  u32x2 lo, hi;
  const unsigned addr = lds_base + off;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(addr));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(addr), "i"(4 * ROW_BYTES));
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return r;
}

// 16-byte LDS read through inline assembly at a lane-constant address plus
// an immediate offset (IMM < 64 KiB), or at a run-time address; as for
// tr_frag_asm_at, the caller runs lds_wait_frags on the result before use.
template <int IMM>
__device__ __forceinline__ u32x4 lds_read16_imm(unsigned addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(IMM));
  return r;
}
__device__ __forceinline__ u32x4 lds_read16_rt(unsigned addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// 16-byte LDS write through inline assembly (see lds_read16_imm: the
// compiler would otherwise wait for direct loads in flight before it).
// Ordering against other waves' reads comes from the barrier that follows.
__device__ __forceinline__ void lds_write16_rt(unsigned addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v));
}

template <int IMM>
__device__ __forceinline__ void lds_write16_imm(unsigned addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(IMM));
}

// Transposed fragment (two transposing reads, the second 4 rows further) at a
// lane-constant address plus an immediate offset (IMM + 4 ROW_BYTES < 64 KiB).
template <int IMM, int ROW_BYTES>
__device__ __forceinline__ u32x4 tr_frag_asm_imm(unsigned addr) {
  u32x2 lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(IMM));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(addr), "i"(IMM + 4 * ROW_BYTES));
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return r;
}

// Wait for all of this wave's LDS reads; the fragments pass through the
// statement so that their uses are ordered after the wait.
__device__ __forceinline__ void lds_wait_frags(u32x4& a, u32x4& b, u32x4& c, u32x4& d) {
  asm("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Wait until at most N of this wave's LDS operations are outstanding.  LDS
// operations complete in issue order, so every read issued before the last N
// has landed (scalar memory operations only add to the count).  The statement
// is volatile so that it keeps its place after the reads issued before it in
// the source (the reads are volatile too): moved above some of them, it would
// count fewer reads in flight and return too early.
template <int N>
__device__ __forceinline__ void lds_wait_frags_n(u32x4& a, u32x4& b, u32x4& c, u32x4& d) {
  static_assert(N >= 0 && N < 16, "lgkmcnt holds 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait_frags_n(u32x4& a, u32x4& b, u32x4& c) {
  static_assert(N >= 0 && N < 16, "lgkmcnt holds 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "i"(N));
}

// The same for two fragments.  Every operand must be a distinct variable: an
// operand passed twice makes the compiler copy the register, possibly before
// the wait, i.e. while the load into it is still in flight.
__device__ __forceinline__ void lds_wait_frags2(u32x4& a, u32x4& b) {
  asm("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}

// Wait until this wave's outstanding global loads (including direct-to-LDS
// loads) have landed.
// s_waitcnt simm16 on gfx9: vmcnt in bits [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8]; 0x0F70 = vmcnt(0) with the other counters free.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's global loads are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt values above 15 need the high field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// XCD-aware workgroup order.  The 8 XCDs of the chip take workgroups
// round-robin by linear id, and each has its own L2.  Within every round of
// 8 x 32 ids, XCD x is given 32 consecutive logical workgroups (neighbours
// that stream the same tiles through its L2 at about the same time); an XCD
// takes chunk x of even rounds and chunk 7 - x of odd ones, so that the long
// and short workgroups of a longest-first order alternate on every XCD.
// A bijection on [0, total); a last partial round keeps the identity.
__device__ __forceinline__ unsigned xcd_order(unsigned lin, unsigned total) {
  if (lin >= total / 256 * 256) return lin;
  const unsigned round = lin / 256, x = lin % 8;
  const unsigned chunk = (round & 1) ? 7 - x : x;
  return round * 256 + chunk * 32 + (lin % 256) / 8;
}

// This workgroup's number in its grid (x fastest), remapped by xcd_order.
// 32-bit: every launch keeps its grid under 2^31 workgroups (checked on the
// host), and 64-bit division by a run-time value costs hundreds of scalar
// instructions in each workgroup's prologue.
__device__ __forceinline__ unsigned wg_number() {
  return xcd_order(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                   gridDim.x * gridDim.y * gridDim.z);
}


}  // namespace lcattn
