// Learnable inner learning rate ("论文速览 | TTT", §4.6), gfx950:
//   eta[b][h][t] = eta_base * sigmoid(theta_lr[h] . x[b][t])
// for every token of the layer input x [B][T][dx] (bf16) and every head's gate
// vector theta_lr [H][dx] (fp32), written in the scans' eta layout [B][H][T].
//
// It is a skinny product (tokens x dx) . (dx x H) with a sigmoid epilogue,
// bound by the one pass over x.  Workgroup = 16 * TB tokens, four waves that
// split dx (wave w takes the 32-wide steps w, w + 4, ...), all heads in passes
// of 32; the four partial sums meet in LDS, where the epilogue also turns the
// [head][token] tiles into [b][h][t] rows.
//
// Products on the matrix unit: 16x16x32 bf16 MFMA with A = theta (heads x dx),
// B = x^T (dx x tokens).  x is exact in bf16; theta is split into three bf16
// terms hi + mid + lo (fp32 to within 2^-24 relative), so every product is
// exact and the sums are fp32.
//
// 16x16x32 bf16 operand layouts (wave64, lane (c, g), c = lane % 16,
// g = lane / 16): A lane holds A[c][8g .. 8g + 7], B lane holds
// B[8g .. 8g + 7][c], accumulator register r holds C[4g + r][c].
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int GATE_HP = 32;  // heads per pass: two 16-row blocks

struct Theta3 {
  bf16x8 hi, mid, lo;
};

// Eight fp32 values -> three bf16 terms (each the nearest-even rounding of
// what the previous terms leave; the residual subtractions are exact).
__device__ __forceinline__ Theta3 split3(float4 a, float4 b) {
  float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t p[3][4];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[k][e] = pack_rne(r[2 * e], r[2 * e + 1]);
      r[2 * e] -= __builtin_bit_cast(float, p[k][e] << 16);
      r[2 * e + 1] -= __builtin_bit_cast(float, p[k][e] & 0xffff0000u);
    }
  Theta3 t;
  t.hi = __builtin_bit_cast(bf16x8, make_uint4(p[0][0], p[0][1], p[0][2], p[0][3]));
  t.mid = __builtin_bit_cast(bf16x8, make_uint4(p[1][0], p[1][1], p[1][2], p[1][3]));
  t.lo = __builtin_bit_cast(bf16x8, make_uint4(p[2][0], p[2][1], p[2][2], p[2][3]));
  return t;
}

template <int TB>
__global__ void __launch_bounds__(256) lr_gate_kernel(GateArgs a) {
  constexpr int TOK = 16 * TB;
  constexpr int PITCH = TOK + 4;  // words per LDS row: the four lane groups hit distinct banks
  __shared__ float red[4][GATE_HP][PITCH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t ntok = (int64_t)a.B * a.T;
  const int64_t f0 = (int64_t)blockIdx.x * TOK;
  const int ksteps = a.dx >> 5;

  // this lane's x rows (tokens past the end re-read the last token; their
  // sums are never stored)
  const bf16x8* xr[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    int64_t f = f0 + 16 * tb + c;
    if (f >= ntok) f = ntok - 1;
    xr[tb] = (const bf16x8*)((const uint16_t*)a.x + f * a.dx + 8 * g);
  }

  for (int hp = 0; hp < a.H; hp += GATE_HP) {
    const int nhb = a.H - hp > 16 ? 2 : 1;  // head blocks in this pass (wave-uniform)
    const float* th[2];
    bool hv[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = hp + 16 * hb + c;
      hv[hb] = h < a.H;
      th[hb] = a.theta + (size_t)(hv[hb] ? h : 0) * a.dx + 8 * g;
    }
    f32x4 acc[2][TB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[hb][tb] = f32x4{0, 0, 0, 0};

    // one 32-wide step of x and theta in flight ahead of the one in use
    bf16x8 xv[TB];
    float4 tv[2][2];
    auto load = [&](int ks, bf16x8* xd, float4 (*td)[2]) {
      const int k0 = ks * 32;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) xd[tb] = xr[tb][k0 >> 3];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        td[hb][0] = make_float4(0.f, 0.f, 0.f, 0.f);
        td[hb][1] = td[hb][0];
        if (hb < nhb && hv[hb]) {
          td[hb][0] = *(const float4*)(th[hb] + k0);
          td[hb][1] = *(const float4*)(th[hb] + k0 + 4);
        }
      }
    };
    if (wave < ksteps) load(wave, xv, tv);
    for (int ks = wave; ks < ksteps; ks += 4) {
      bf16x8 xn[TB];
      float4 tn[2][2];
      if (ks + 4 < ksteps) load(ks + 4, xn, tn);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (hb < nhb) {
          const Theta3 s = split3(tv[hb][0], tv[hb][1]);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[hb][tb] = mfma_k32(s.hi, xv[tb], acc[hb][tb]);
            acc[hb][tb] = mfma_k32(s.mid, xv[tb], acc[hb][tb]);
            acc[hb][tb] = mfma_k32(s.lo, xv[tb], acc[hb][tb]);
          }
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) xv[tb] = xn[tb];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        tv[hb][0] = tn[hb][0];
        tv[hb][1] = tn[hb][1];
      }
    }
    // register r of acc[hb][tb] = partial sum of head hp + 16 hb + 4g + r, token 16 tb + c
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][16 * hb + 4 * g + r][16 * tb + c] = acc[hb][tb][r];
    __syncthreads();
    // epilogue: thread -> (token i, heads j0, j0 + 256 / TOK, ...)
    const int i = threadIdx.x % TOK;
    const int64_t f = f0 + i;
    if (f < ntok) {
      const int64_t bi = f / a.T, t = f - bi * a.T;
      for (int hl = threadIdx.x / TOK; hl < GATE_HP; hl += 256 / TOK) {
        const int h = hp + hl;
        if (h >= a.H) break;
        const float s = (red[0][hl][i] + red[1][hl][i]) + (red[2][hl][i] + red[3][hl][i]);
        a.eta[((size_t)bi * a.H + h) * a.T + t] = a.eta_base / (1.f + expf(-s));
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_lr_gate(const GateArgs& a, int tokens_per_workgroup, hipStream_t s) {
  const int64_t ntok = (int64_t)a.B * a.T;
  if (ntok == 0 || a.H == 0) return hipSuccess;
  if (tokens_per_workgroup == 0) tokens_per_workgroup = ntok >= 256 * 64 ? 64 : 32;
  switch (tokens_per_workgroup) {
    case 32:
      hipLaunchKernelGGL(lr_gate_kernel<2>, dim3((unsigned)((ntok + 31) / 32)), dim3(256), 0, s, a);
      break;
    case 64:
      hipLaunchKernelGGL(lr_gate_kernel<4>, dim3((unsigned)((ntok + 63) / 64)), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ttt
