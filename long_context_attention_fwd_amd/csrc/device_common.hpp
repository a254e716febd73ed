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

// XOR swizzles of 16-byte LDS units, chosen so that the 8 lanes served in one
// LDS cycle touch 8 distinct 16-byte bank groups.
//  * row-major tiles read in pi row order (rows pi(0..7) = 0-3, 8-11):
__device__ __forceinline__ int swz_rows_pi(int row) { return (row & 3) | ((row >> 1) & 4); }
//  * transposed tiles [col][row] read by consecutive columns and written by
//    columns 8 apart:
__device__ __forceinline__ int swz_cols(int col) { return (col ^ (col >> 3)) & 7; }

// Repack four 8-element bf16 rows x[r] (r = 0..3) into eight 4-element columns:
// column e holds x[0][e], x[1][e], x[2][e], x[3][e].
__device__ __forceinline__ void transpose4x8(const u32x4 x[4], u32x2 out[8]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned a = x[0][m], b = x[1][m], c = x[2][m], d = x[3][m];
    // element 2m sits in the low half of word m, element 2m+1 in the high half
    out[2 * m][0] = (a & 0xFFFFu) | (b << 16);
    out[2 * m][1] = (c & 0xFFFFu) | (d << 16);
    out[2 * m + 1][0] = (a >> 16) | (b & 0xFFFF0000u);
    out[2 * m + 1][1] = (c >> 16) | (d & 0xFFFF0000u);
  }
}

}  // namespace lcattn
