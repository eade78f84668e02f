// Operand helpers of the TTT-Linear bf16 scans (plain and LayerNorm inner
// model): the swizzled K/Q tile layout in LDS, the permuted column order of
// the register-resident state, and products with pre-split fp32 operands.
//
// K/Q tiles (16 tokens x 64 bf16) are stored with 16-byte chunk p of token
// row r at position p ^ (r & 7), which makes 16-row chunk reads bank-conflict
// free.  The state W lives in four MFMA accumulators per wave: register W[m]
// of lane (c, g) holds W[row c][sigma(m, 4g + r)], so the hi/lo split of W
// gives K=32 operand slots that are 8 consecutive columns, i.e. one 16-byte
// chunk of a K row.
#pragma once

#include "ttt_device.h"

namespace ttt {

__device__ __forceinline__ uint2 s4u(s16x4 v) { return __builtin_bit_cast(uint2, v); }
__device__ __forceinline__ s16x4 u2s(uint2 v) { return __builtin_bit_cast(s16x4, v); }

// s_waitcnt lgkmcnt(0): every LDS read issued so far has returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// byte offset of element (r, j) of a swizzled 16 x 64 bf16 K/Q tile
__device__ __forceinline__ int swz(int r, int j) {
  return r * 128 + ((((j >> 3) ^ (r & 7))) << 4) + ((j & 7) << 1);
}
// K=32 operand of row r: columns 32h + 8g .. 32h + 8g + 7
__device__ __forceinline__ bf16x8 row_chunk(const char* tile, int r, int h, int g) {
  return *(const bf16x8*)(tile + r * 128 + ((((4 * h + g) ^ (r & 7))) << 4));
}
__device__ __forceinline__ int sigma(int m, int row) {
  return 32 * (m >> 1) + 8 * (row >> 2) + 4 * (m & 1) + (row & 3);
}

__device__ __forceinline__ void put_split(char* p, int lane, f32x4 x) {
  const Split4 s = split4(x);
  const uint2 h = s4u(s.hi), l = s4u(s.lo);
  *(uint4*)(p + lane * 16) = make_uint4(h.x, h.y, l.x, l.y);
}

// Operand pair of a pre-split Y for products X*Y: [Yhi | Yhi] and [Ylo | 0].
struct YOps {
  bf16x8 hh, l0;
};
__device__ __forceinline__ YOps yops(const Split4& y) {
  const s16x4 z = {0, 0, 0, 0};
  return YOps{cat44(y.hi, y.hi), cat44(y.lo, z)};
}
// acc + X*Y, X given as [Xhi | Xlo] of the accumulator layout of X^T:
// [Xhi|Xlo].[Yhi|Yhi] + [Xhi|Xlo].[Ylo|0] = Xhi Yhi + Xlo Yhi + Xhi Ylo.
__device__ __forceinline__ f32x4 mm_pre(bf16x8 x, const YOps& y, f32x4 acc) {
  acc = mfma_k32(x, y.hh, acc);
  acc = mfma_k32(x, y.l0, acc);
  return acc;
}
// The same three terms of the transposed product, acc + Y^T X^T, with the
// operands in swapped roles: accumulator [col][row].
__device__ __forceinline__ f32x4 mm_pre_t(const YOps& y, bf16x8 x, f32x4 acc) {
  acc = mfma_k32(y.hh, x, acc);
  acc = mfma_k32(y.l0, x, acc);
  return acc;
}
__device__ __forceinline__ bf16x8 get8(const char* p, int lane) {
  return *(const bf16x8*)(p + lane * 16);
}

}  // namespace ttt
