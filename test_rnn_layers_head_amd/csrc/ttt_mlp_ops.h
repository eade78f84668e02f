// Operand helpers shared by the TTT-MLP scan and its backward (gfx950,
// 16x16x32 bf16 MFMA).  Lane l = c + 16 g (c < 16, g < 4); an operand lane
// supplies A[c][8g + e] / B[8g + e][c], e < 8, and the accumulator holds
// C[4g + r][c], r < 4.  An accumulator tile X used as [hi | lo] A operand is
// X^T over its 16 rows; used through yops() as a B operand it is X itself
// (the hi half twice, then the lo half against zeros), so
// mm_pre(cat44(X.hi, X.lo), yops(Y)) = X^T Y with three hi/lo products.
#pragma once

#include "ttt_device.h"

namespace ttt {

// K / Q tiles (16 tokens x 64 bf16): 16-byte chunk p of row r at position
// p ^ (r & 7), which makes the 16-row chunk reads bank-conflict free.
__device__ __forceinline__ int swz_chunk(int r, int p) { return r * 128 + ((p ^ (r & 7)) << 4); }
__device__ __forceinline__ bf16x8 row_chunk(const char* tile, int r, int h, int g) {
  return *(const bf16x8*)(tile + swz_chunk(r, 4 * h + g));
}

struct YOps {
  bf16x8 hh, l0;
};
__device__ __forceinline__ YOps yops(const Split4& y) {
  const s16x4 z = {0, 0, 0, 0};
  return YOps{cat44(y.hi, y.hi), cat44(y.lo, z)};
}
// acc + X*Y, X as [Xhi | Xlo] of the accumulator layout of X^T (three terms)
__device__ __forceinline__ f32x4 mm_pre(bf16x8 x, const YOps& y, f32x4 acc) {
  acc = mfma_k32(x, y.hh, acc);
  acc = mfma_k32(x, y.l0, acc);
  return acc;
}
// acc + A*B for 8-slot operands split into hi/lo (three terms)
__device__ __forceinline__ f32x4 mm3(const Split8& a, const Split8& b, f32x4 acc) {
  acc = mfma_k32(a.hi, b.hi, acc);
  acc = mfma_k32(a.hi, b.lo, acc);
  acc = mfma_k32(a.lo, b.hi, acc);
  return acc;
}
__device__ __forceinline__ uint4 pack_split(const Split4& s) {
  const uint2 h = __builtin_bit_cast(uint2, s.hi), l = __builtin_bit_cast(uint2, s.lo);
  return make_uint4(h.x, h.y, l.x, l.y);
}
__device__ __forceinline__ Split4 unpack_split(uint4 v) {
  return Split4{__builtin_bit_cast(s16x4, make_uint2(v.x, v.y)),
                __builtin_bit_cast(s16x4, make_uint2(v.z, v.w))};
}

// Transpose of an accumulator tile: [hi | lo] as A operand (X^T) against
// itr = [I; I] (slots 8g + e with 4g + e % 4 == c), exact for the hi + lo
// halves, which split again into the same halves.
__device__ __forceinline__ f32x4 transpose16(f32x4 x, bf16x8 itr) {
  const Split4 s = split4(x);
  return mfma_k32(cat44(s.hi, s.lo), itr, f32x4{0, 0, 0, 0});
}

}  // namespace ttt
