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

// ============================================================== backward
// dL/da = dL/deta * eta (1 - eta / eta_base) (= eta_base sigmoid' (a)), from
// the forward's eta, so the logits need not be recomputed;
//   dtheta_lr[h] = sum_{b,t} da[b][h][t] x[b][t],   dx[b][t] = sum_h da[b][h][t] theta_lr[h].
namespace ttt {
namespace {

// da at (batch bi, head h, position t); B * H * T < 2^31 (checked by the ABI)
__device__ __forceinline__ float gate_da_at(const GateBwdArgs& a, int bi, int h, int t,
                                            float inv_base) {
  const int i = (bi * a.H + h) * a.T + t;
  const float e = a.eta[i];
  return a.deta[i] * e * (1.f - e * inv_base);
}
// da of flat token f = bi * T + t (zero past the tokens or the heads)
__device__ __forceinline__ float gate_da(const GateBwdArgs& a, int f, int h, float inv_base) {
  if (f >= a.B * a.T || h >= a.H) return 0.f;
  const int bi = f / a.T;
  return gate_da_at(a, bi, h, f - bi * a.T, inv_base);
}

// Partial sums of dtheta over one chunk of tokens, for 16 * NM columns:
// part[s][h][col].  Products on the matrix unit: x exact in bf16, brought to
// tokens-in-registers by a one-hot selection MFMA (exact), da as hi + lo.
// Four waves take interleaved 16-token blocks and meet in LDS.
template <int NM>
__global__ void __launch_bounds__(256) lr_gate_bwd_dtheta_kernel(GateBwdArgs a, float* part,
                                                                 int chunk) {
  __shared__ f32x4 red[4][2][NM][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t ntok = (int64_t)a.B * a.T;
  const int col0 = blockIdx.x * 16 * NM;
  const int64_t f_begin = (int64_t)blockIdx.y * chunk;
  int64_t f_end = f_begin + chunk;
  if (f_end > ntok) f_end = ntok;
  const float inv_base = a.eta_base != 0.f ? 1.f / a.eta_base : 0.f;
  // one-hot selectors: picks column 16p + c out of a 32-column chunk
  bf16x8 sel[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[p][e] = (bf16)((g == 2 * p + (c >> 3) && e == (c & 7)) ? 1.f : 0.f);

  for (int hp = 0; hp < a.H; hp += 32) {
    f32x4 acc[2][NM];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[hb][m] = f32x4{0, 0, 0, 0};
    for (int64_t f0 = f_begin + 16 * wave; f0 < f_end; f0 += 64) {
      // x rows: token f0 + c, columns col0 + 32 h + 8g .. + 7 (zeros past the chunk)
      const int64_t f = f0 + c;
      const bool ok = f < f_end;
      bf16x8 xr[(NM + 1) / 2];
#pragma unroll
      for (int h = 0; h < (NM + 1) / 2; ++h) {
        xr[h] = bf16x8{};
        if (ok) xr[h] = *(const bf16x8*)((const uint16_t*)a.x + f * a.dx + col0 + 32 * h + 8 * g);
      }
      // tokens in registers: xt[m] register r = x[f0 + 4g + r][col0 + 16 m + c]
      uint2 xt[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 v = mfma_k32(xr[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});
        xt[m] = make_uint2(pack_rne(v[0], v[1]), pack_rne(v[2], v[3]));
      }
      // batch and position of token f0 + 4g (one division per block), then
      // of the next three, stepping into the next batch at each sequence end
      int tb[4], tt[4];
      {
        const int fb = (int)(f0 + 4 * g);
        int bi = fb / a.T, t = fb - bi * a.T;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tb[r] = bi;
          tt[r] = t;
          if (++t == a.T) {
            t = 0;
            ++bi;
          }
        }
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int h = hp + 16 * hb + c;
        f32x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          d[r] = (f0 + 4 * g + r < f_end && h < a.H) ? gate_da_at(a, tb[r], h, tt[r], inv_base) : 0.f;
        const Split4 ds = split4(d);
        const bf16x8 dop = cat44(ds.hi, ds.lo);
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[hb][m] = mfma_k32(dop, cat8(xt[m], xt[m]), acc[hb][m]);
      }
    }
    // register r of acc[hb][m] = sum over this wave's tokens for head
    // hp + 16 hb + 4g + r, column col0 + 16 m + c
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int m = 0; m < NM; ++m) red[wave][hb][m][lane] = acc[hb][m];
    __syncthreads();
    for (int q = wave; q < 2 * NM; q += 4) {
      const int hb = q / NM, m = q % NM;
      const f32x4 s4 = (red[0][hb][m][lane] + red[1][hb][m][lane]) + (red[2][hb][m][lane] + red[3][hb][m][lane]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = hp + 16 * hb + 4 * g + r;
        if (h < a.H) part[((size_t)blockIdx.y * a.H + h) * a.dx + col0 + 16 * m + c] = s4[r];
      }
    }
    __syncthreads();
  }
}

// dtheta[h][col] = sum over the chunks, in chunk order
__global__ void __launch_bounds__(256) lr_gate_bwd_reduce_kernel(GateBwdArgs a, const float* part,
                                                                 int nchunk) {
  const int64_t n = (int64_t)a.H * a.dx;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < nchunk; ++k) s += part[k * n + i];
    a.dtheta[i] = s;
  }
}

// dx[f][col .. col + 3] for 32 tokens f per workgroup, 4 columns per thread,
// 16 heads at a time (their theta rows in registers, da in LDS).
__global__ void __launch_bounds__(256) lr_gate_bwd_dx_kernel(GateBwdArgs a) {
  __shared__ float sda[32][17];
  const int tid = threadIdx.x;
  const int64_t ntok = (int64_t)a.B * a.T;
  const int64_t f0 = (int64_t)blockIdx.x * 32;
  const int col = (blockIdx.y * 256 + tid) * 4;
  const bool cok = col < a.dx;
  const float inv_base = a.eta_base != 0.f ? 1.f / a.eta_base : 0.f;
  float4 acc[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int hc = 0; hc < a.H; hc += 16) {
    // stage da of the 32 tokens x 16 heads: thread -> (head tid / 16, tokens (tid % 16) + 16 j)
    for (int j = 0; j < 2; ++j) {
      const int hl = tid >> 4, tl = (tid & 15) + 16 * j;
      sda[tl][hl] = gate_da(a, (int)f0 + tl, hc + hl, inv_base);
    }
    float4 th[16];
#pragma unroll
    for (int h = 0; h < 16; ++h)
      th[h] = (cok && hc + h < a.H) ? *(const float4*)(a.theta + (size_t)(hc + h) * a.dx + col)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 32; ++t)
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        const float d = sda[t][h];
        acc[t].x = fmaf(d, th[h].x, acc[t].x);
        acc[t].y = fmaf(d, th[h].y, acc[t].y);
        acc[t].z = fmaf(d, th[h].z, acc[t].z);
        acc[t].w = fmaf(d, th[h].w, acc[t].w);
      }
    __syncthreads();
  }
  if (cok)
#pragma unroll
    for (int t = 0; t < 32; ++t)
      if (f0 + t < ntok) *(float4*)(a.dxo + (f0 + t) * a.dx + col) = acc[t];
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

}  // namespace

hipError_t launch_lr_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  const int64_t ntok = (int64_t)a.B * a.T;
  const int64_t nth = (int64_t)a.H * a.dx;
  if (ntok == 0 || a.H == 0) {  // dtheta = 0 (no tokens), dx = 0 (no heads)
    if (nth > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, s, a.dtheta, nth);
    if (ntok > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, a.dxo, ntok * a.dx);
    return hipGetLastError();
  }
  // dtheta: the token range in nchunk chunks whose partial sums go to the
  // start of dx's memory (nchunk * H <= B * T rows of dx) and are summed in
  // chunk order, before dx itself is written; one chunk (fewer than 2 H
  // tokens) writes dtheta directly
  int64_t nchunk = ntok / a.H;
  if (nchunk > 16) nchunk = 16;
  if (nchunk < 1) nchunk = 1;
  const int chunk = (int)((ntok + nchunk - 1) / nchunk);
  float* part = nchunk == 1 ? a.dtheta : a.dxo;
  const dim3 g1(a.dx % 64 == 0 ? a.dx / 64 : a.dx / 32, (unsigned)nchunk);
  if (a.dx % 64 == 0)
    hipLaunchKernelGGL(lr_gate_bwd_dtheta_kernel<4>, g1, dim3(256), 0, s, a, part, chunk);
  else
    hipLaunchKernelGGL(lr_gate_bwd_dtheta_kernel<2>, g1, dim3(256), 0, s, a, part, chunk);
  if (nchunk > 1) {
    const int64_t nb = (nth + 255) / 256;
    hipLaunchKernelGGL(lr_gate_bwd_reduce_kernel, dim3((unsigned)(nb < 1024 ? nb : 1024)), dim3(256), 0,
                       s, a, (const float*)a.dxo, (int)nchunk);
  }
  hipLaunchKernelGGL(lr_gate_bwd_dx_kernel, dim3((unsigned)((ntok + 31) / 32), (unsigned)((a.dx + 1023) / 1024)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
