// Device helpers shared by the gfx950 TTT scan kernels: vector types, MFMA
// wrappers, fp32 -> bf16 hi/lo splitting, LDS-DMA staging and the raw
// workgroup barrier.
//
// MFMA operand layouts used throughout (wave64, lane l, c = l % 16,
// g = l / 16), for a 16x16 output tile C[M][N]:
//   accumulator   : lane (c,g) register r holds C[4g + r][c]
//   16x16x32 bf16 : A-operand lane (c,g) holds A[c][8g .. 8g+7],
//                   B-operand lane (c,g) holds B[8g .. 8g+7][c]
//   16x16x4  f32  : A[c][g],          B[g][c]
// The reduction index may be permuted freely as long as A and B agree, which
// is how the kernels feed a register-resident accumulator straight back in as
// an operand without a transpose.  Reductions of length 16 (over the tokens
// of a tile) also use the K=32 shape: slots 8g..8g+3 carry the high bf16
// halves and 8g+4..8g+7 the low halves of the same four indices, so one
// instruction sums both halves.  The bf16 path uses no other MFMA shape: a
// 16x16x16 MFMA that reads a 16x16x32 result as its accumulator right after
// it was issued has been seen to read stale registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define TTT_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, (bf16)x);  // round to nearest even
}
__device__ __forceinline__ float bf16_val(short h) {
  return __builtin_bit_cast(float, ((uint32_t)(uint16_t)h) << 16);
}

// x = hi + lo + O(2^-16 |x|) with hi, lo bf16: products of such pairs with
// exact bf16 operands keep ~16 significant bits, far below the fp32 budget.
struct Split4 {
  s16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(f32x4 x);
struct Split8 {
  bf16x8 hi, lo;
};
// hi/lo split of two fp32 values at once: one packed conversion for the
// high halves, the exact residuals, one packed conversion for the low halves.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
  const float r0 = x0 - __builtin_bit_cast(float, h << 16);
  const float r1 = x1 - __builtin_bit_cast(float, h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}
__device__ __forceinline__ Split4 split4(f32x4 x) {
  uint32_t h0, l0, h1, l1;
  split_pair(x[0], x[1], h0, l0);
  split_pair(x[2], x[3], h1, l1);
  return Split4{__builtin_bit_cast(s16x4, make_uint2(h0, h1)),
                __builtin_bit_cast(s16x4, make_uint2(l0, l1))};
}
// Two fp32 values rounded to bf16 (nearest even) and packed.
__device__ __forceinline__ uint32_t pack_rne(float x0, float x1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}
// Pack two accumulator registers (4 + 4 values) into one 8-wide operand.
__device__ __forceinline__ Split8 split8(f32x4 a, f32x4 b) {
  uint32_t h[4], l[4];
  split_pair(a[0], a[1], h[0], l[0]);
  split_pair(a[2], a[3], h[1], l[1]);
  split_pair(b[0], b[1], h[2], l[2]);
  split_pair(b[2], b[3], h[3], l[3]);
  Split8 s;
  s.hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  s.lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  return s;
}

// Residual split on the matrix unit.  For two accumulator blocks a (operand
// slots 0..3) and b (slots 4..7): hi = RNE bf16 of both (packed converts),
// then a - hi(a) and b - hi(b) are formed exactly by a K=32 MFMA that adds
// -hi through a negated one-hot selection (each output entry receives one
// exact product), and converted to the lo halves.  8 VALU + 2 MFMA instead of
// 24 VALU for the same 8 values.
struct NegSel {
  bf16x8 s0, s1;  // -I on slots 0..3 / on slots 4..7
};
__device__ __forceinline__ NegSel make_negsel(int c, int g) {
  NegSel n;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    n.s0[e] = (bf16)((e < 4 && c == 4 * g + e) ? -1.f : 0.f);
    n.s1[e] = (bf16)((e >= 4 && c == 4 * g + e - 4) ? -1.f : 0.f);
  }
  return n;
}
__device__ __forceinline__ Split8 split8_mfma(f32x4 a, f32x4 b, const NegSel& ns) {
  Split8 s;
  s.hi = __builtin_bit_cast(bf16x8, make_uint4(pack_rne(a[0], a[1]), pack_rne(a[2], a[3]),
                                               pack_rne(b[0], b[1]), pack_rne(b[2], b[3])));
  const f32x4 ra = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ns.s0, s.hi, a, 0, 0, 0);
  const f32x4 rb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ns.s1, s.hi, b, 0, 0, 0);
  s.lo = __builtin_bit_cast(bf16x8, make_uint4(pack_rne(ra[0], ra[1]), pack_rne(ra[2], ra[3]),
                                               pack_rne(rb[0], rb[1]), pack_rne(rb[2], rb[3])));
  return s;
}

__device__ __forceinline__ bf16x8 cat8(uint2 a, uint2 b) {
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 cat44(s16x4 a, s16x4 b) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Product of two 16x16 fp32 matrices held in accumulator layout:
// xt = accumulator layout of X^T, y = accumulator layout of Y; returns
// acc + X*Y with the three significant hi/lo terms (the lo*lo term is
// below 2^-16 relative).
__device__ __forceinline__ f32x4 mm16_split(f32x4 xt, f32x4 y, f32x4 acc) {
  const Split4 a = split4(xt), b = split4(y);
  const s16x4 z = {0, 0, 0, 0};
  acc = mfma_k32(cat44(a.hi, a.lo), cat44(b.hi, b.hi), acc);  // hi*hi + lo*hi
  acc = mfma_k32(cat44(a.hi, z), cat44(b.lo, z), acc);        // hi*lo
  return acc;
}
__device__ __forceinline__ f32x4 mm16_f32(f32x4 xt, f32x4 y, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = mfma_f32(xt[e], y[e], acc);
  return acc;
}

// GELU and its derivative.  Phi(x) = 1/2 (1 + erf(x / sqrt 2)); erf from
// Abramowitz & Stegun 7.1.26: erf(y) = 1 - (a1 t + .. + a5 t^5) exp(-y^2),
// t = 1 / (1 + p y), y >= 0.  exp(-y^2) = exp(-x^2 / 2) is shared with the
// normal density phi(x) = exp(-x^2 / 2) / sqrt(2 pi) of GELU' = Phi + x phi.
struct GeluOut {
  float g, dg;
};
__device__ __forceinline__ GeluOut gelu_and_grad(float x) {
  const float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
              a4 = -1.453152027f, a5 = 1.061405429f;
  const float y = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, y, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);  // exp(-x^2/2)
  const float q = 0.5f * poly * e;                                         // 1 - Phi(|x|)
  const float phi_cdf = x >= 0.f ? 1.f - q : q;
  return GeluOut{x * phi_cdf, fmaf(x, e * 0.39894228040143268f, phi_cdf)};
}

// Sum over the 16 lanes of a DPP row (row rotations by 8, 4, 2, 1); every
// lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}

// Workgroup barrier for LDS traffic: this wave's LDS reads and writes are
// complete before it arrives (the LDS may reorder requests of different
// waves, and the barrier instruction waits on no counter); no cache or
// vector-memory wait is implied: producers that write LDS with DMA wait on
// their own vector-memory counter before arriving.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), gfx9 encoding
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// A barrier with no counter wait at all (the caller waits on what it needs)
// and no instruction of any kind scheduled across it: keeps a software
// pipeline's stages (reads issued right after the barrier, their use one
// iteration later) in the order they were written.
__device__ __forceinline__ void wg_barrier_pinned() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return
// zeros, which is how partial tiles are padded.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Wave-wide DMA of 16 (or 4) bytes per lane from the buffer into LDS at
// lds_base + 16 * lane (4 * lane).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TTT_LDS void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TTT_LDS void*)lds_base, 4, voff, 0, 0, 0);
}

}  // namespace ttt
