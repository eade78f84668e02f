// One-token decode steps of the TTT layers, gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): generation processes one token at a time in the
// primal form (§6.11).  Each (batch, head) unit carries its state W and its
// gradient point Wg, the state at the start of the current mini-batch
// (§3.5); a token at position p = pos mod b first sets Wg = W when p = 0,
// then takes its gradient at Wg (per-token eta, §4.6), updates W, and reads
// its output from the updated W (§3.1).  One step is one iteration of the
// scan's primal recurrence.
//
// Work per unit is a few matrix-vector products with a 64 x 64 (or 256 x 64)
// state, so the steps are bound by the state's HBM traffic: read W and Wg,
// write W (and Wg when a mini-batch starts).  No MFMA: a single token gives
// no contraction worth a matrix tile.  fp32 throughout.
//
// Layout of a linear step: one workgroup of 256 threads per unit; thread
// t = 4i + s owns row i of W, columns 16s .. 16s+15 (64 contiguous bytes, so
// a wave moves 4 KB of W per access, coalesced); the four threads of a row
// are adjacent lanes, so row sums are two quad-permute adds.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int STEP_THREADS = 256;

// sum over the 4 adjacent lanes of a quad (row i of W), in every lane
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF,
                                                          0xF, false));  // [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF,
                                                          0xF, false));  // [2,3,0,1]
  return x;
}

// 16 consecutive values of a q/k/v row as fp32
template <bool F32IN>
__device__ __forceinline__ void load16(const void* base, size_t off, float* out) {
  if constexpr (F32IN) {
    const float4* p = (const float4*)((const float*)base + off);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float4 x = p[n];
      out[4 * n] = x.x;
      out[4 * n + 1] = x.y;
      out[4 * n + 2] = x.z;
      out[4 * n + 3] = x.w;
    }
  } else {
    const uint4* p = (const uint4*)((const uint16_t*)base + off);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const uint4 x = p[n];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * n + 2 * e] = __builtin_bit_cast(float, w[e] << 16);
        out[8 * n + 2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xffff0000u);
      }
    }
  }
}
template <bool F32IN>
__device__ __forceinline__ float load1(const void* base, size_t off) {
  if constexpr (F32IN) return ((const float*)base)[off];
  return __builtin_bit_cast(float, ((uint32_t)((const uint16_t*)base)[off]) << 16);
}

__device__ __forceinline__ int minibatch_pos(int pos, int b) {
  const int p = pos % b;
  return p < 0 ? p + b : p;
}

// ------------------------------------------------------------ TTT-Linear
// f(x) = W x, l = ||W k - v||^2:  g = 2 (Wg k - v),  W -= eta g k^T,  z = W q.
template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) linear_step_kernel(StepArgs a) {
  const int unit = blockIdx.x;
  const int t = threadIdx.x, i = t >> 2, s = t & 3;
  const int bi = unit / a.H;
  const size_t vo = (size_t)unit * 64;            // this unit's token vectors
  const size_t wo = (size_t)unit * 4096 + i * 64 + 16 * s;
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;

  float kk[16], qq[16], W[16], G[16];
  load16<F32IN>(a.k, vo + 16 * s, kk);
  load16<F32IN>(a.q, vo + 16 * s, qq);
  const float vi = load1<F32IN>(a.v, vo + i);
  const float eta = a.eta[unit];
  const float4* wp = (const float4*)(a.w + wo);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float4 x = wp[n];
    W[4 * n] = x.x; W[4 * n + 1] = x.y; W[4 * n + 2] = x.z; W[4 * n + 3] = x.w;
  }
  if (start || a.w_gp == nullptr) {
#pragma unroll
    for (int e = 0; e < 16; ++e) G[e] = W[e];
  } else {
    const float4* gp = (const float4*)(a.w_gp + wo);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float4 x = gp[n];
      G[4 * n] = x.x; G[4 * n + 1] = x.y; G[4 * n + 2] = x.z; G[4 * n + 3] = x.w;
    }
  }
  if (start && a.w_gp != nullptr) {  // the gradient point of the new mini-batch
    float4* gp = (float4*)(a.w_gp + wo);
#pragma unroll
    for (int n = 0; n < 4; ++n) gp[n] = make_float4(W[4 * n], W[4 * n + 1], W[4 * n + 2], W[4 * n + 3]);
  }
  float y = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) y = fmaf(G[e], kk[e], y);
  y = quad_sum(y);
  const float ng = -2.f * eta * (y - vi);  // -eta g_i
  float zq = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    W[e] = fmaf(ng, kk[e], W[e]);
    zq = fmaf(W[e], qq[e], zq);
  }
  zq = quad_sum(zq);
  float4* w_out = (float4*)(a.w + wo);
#pragma unroll
  for (int n = 0; n < 4; ++n) w_out[n] = make_float4(W[4 * n], W[4 * n + 1], W[4 * n + 2], W[4 * n + 3]);
  if (s == 0) a.z[vo + i] = zq;
}

// ------------------------------------- TTT-Linear with LayerNorm + residual
// f(x) = x + LN(W x): the LN statistics are sums over the 64 rows, i.e. over
// the whole workgroup (4 waves x 16 rows): a wave sum of the quad leaders
// (DPP) and an LDS exchange of the 4 wave partials.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
// sums over the 64 rows of two per-row values held by the quad leaders;
// every call site passes its own 4-entry LDS buffer, so one barrier suffices
__device__ __forceinline__ float2 rows_sum2(float x, float y, float2* red, int s) {
  x = s == 0 ? x : 0.f;
  y = s == 0 ? y : 0.f;
  x = wave_sum(x);
  y = wave_sum(y);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = make_float2(x, y);
  __syncthreads();
  const float2 r0 = red[0], r1 = red[1], r2 = red[2], r3 = red[3];
  return make_float2((r0.x + r1.x) + (r2.x + r3.x), (r0.y + r1.y) + (r2.y + r3.y));
}

template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) linear_ln_step_kernel(StepArgs a, const float* gamma,
                                                                      const float* beta, float eps) {
  __shared__ float2 red[3][4];
  const int unit = blockIdx.x;
  const int t = threadIdx.x, i = t >> 2, s = t & 3;
  const int bi = unit / a.H, head = unit % a.H;
  const size_t vo = (size_t)unit * 64;
  const size_t wo = (size_t)unit * 4096 + i * 64 + 16 * s;
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;
  const float gi = gamma[head * 64 + i], be = beta[head * 64 + i];

  float kk[16], qq[16], W[16], G[16];
  load16<F32IN>(a.k, vo + 16 * s, kk);
  load16<F32IN>(a.q, vo + 16 * s, qq);
  const float vi = load1<F32IN>(a.v, vo + i), ki = load1<F32IN>(a.k, vo + i),
              qi = load1<F32IN>(a.q, vo + i);
  const float eta = a.eta[unit];
  const float4* wp = (const float4*)(a.w + wo);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float4 x = wp[n];
    W[4 * n] = x.x; W[4 * n + 1] = x.y; W[4 * n + 2] = x.z; W[4 * n + 3] = x.w;
  }
  if (start || a.w_gp == nullptr) {
#pragma unroll
    for (int e = 0; e < 16; ++e) G[e] = W[e];
  } else {
    const float4* gp = (const float4*)(a.w_gp + wo);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float4 x = gp[n];
      G[4 * n] = x.x; G[4 * n + 1] = x.y; G[4 * n + 2] = x.z; G[4 * n + 3] = x.w;
    }
  }
  if (start && a.w_gp != nullptr) {
    float4* gp = (float4*)(a.w_gp + wo);
#pragma unroll
    for (int n = 0; n < 4; ++n) gp[n] = make_float4(W[4 * n], W[4 * n + 1], W[4 * n + 2], W[4 * n + 3]);
  }
  // forward on the training view at the gradient point: y = Wg k, mean and
  // population variance over the 64 rows (one pass: E[y^2] - mu^2, >= 0)
  float y = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) y = fmaf(G[e], kk[e], y);
  y = quad_sum(y);
  const float2 sy = rows_sum2(y, y * y, red[0], s);
  const float mu = sy.x * (1.f / 64);
  const float rs = rsqrtf(fmaxf(fmaf(sy.y, 1.f / 64, -mu * mu), 0.f) + eps);
  const float yh = (y - mu) * rs;
  // dl/dyhat = 2 gamma (k + gamma yhat + beta - v); LayerNorm VJP
  const float gy = 2.f * gi * ((ki + fmaf(gi, yh, be)) - vi);
  const float2 m = rows_sum2(gy, gy * yh, red[1], s);
  const float gr = rs * (gy - m.x * (1.f / 64) - yh * (m.y * (1.f / 64)));
  const float ng = -eta * gr;
  float o = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    W[e] = fmaf(ng, kk[e], W[e]);
    o = fmaf(W[e], qq[e], o);
  }
  o = quad_sum(o);
  float4* w_out = (float4*)(a.w + wo);
#pragma unroll
  for (int n = 0; n < 4; ++n) w_out[n] = make_float4(W[4 * n], W[4 * n + 1], W[4 * n + 2], W[4 * n + 3]);
  // z = q + LN(W q)
  const float2 so = rows_sum2(o, o * o, red[2], s);
  const float mo = so.x * (1.f / 64);
  const float ro = rsqrtf(fmaxf(fmaf(so.y, 1.f / 64, -mo * mo), 0.f) + eps);
  if (s == 0) a.z[vo + i] = qi + fmaf(gi, (o - mo) * ro, be);
}

// ------------------------------------------------------------------ TTT-MLP
// f(x) = W2 GELU(W1 x), hidden width 256 (§4.4).  At the gradient point:
//   a = W1g k, x = GELU(a), e = 2 (W2g x - v), delta = (W2g^T e) * GELU'(a);
// W2 -= eta e x^T, W1 -= eta delta k^T; z = W2 GELU(W1 q).
// Two thread mappings, one workgroup barrier between phases: "hidden"
// (thread h = hidden unit h: row h of W1, column h of W2) and "output"
// (thread t = 4i + s: row i of W2, hidden units 64s .. 64s+63).  A reduction
// over the hidden units thus becomes an in-thread sum plus a quad sum, and
// one over the outputs an in-thread sum.  Within a call W1/W2 are read
// before they are written, by the same thread or across a barrier.
// GELU(x) = x Phi(x) with erf from Abramowitz & Stegun 7.1.26 (|err| <=
// 1.5e-7), the same function as the MLP scan's (gelu_and_grad).
constexpr int MLP_HID = 256;

template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) mlp_step_kernel(StepArgs a) {
  __shared__ float sk[64], sq[64], sx[MLP_HID], se[64], sh[MLP_HID];
  const int unit = blockIdx.x, t = threadIdx.x;
  const int bi = unit / a.H;
  const size_t vo = (size_t)unit * 64;
  const size_t so = (size_t)unit * (MLP_HID * 64);
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;  // always when b == 1
  const bool copy_gp = start && a.w_gp != nullptr;  // gradient points may be NULL for b == 1
  const float eta = a.eta[unit];
  if (t < 64) {
    sk[t] = load1<F32IN>(a.k, vo + t);
    sq[t] = load1<F32IN>(a.q, vo + t);
  }
  __syncthreads();

  // ---- phase 1 (hidden mapping): a_h = W1g[h] . k
  const int h = t;
  float4 w1[16];
  {
    const float4* src = (const float4*)(a.w + so + (size_t)h * 64);
    const float4* gsrc = start ? src : (const float4*)(a.w_gp + so + (size_t)h * 64);
    float4* gdst = copy_gp ? (float4*)(a.w_gp + so + (size_t)h * 64) : nullptr;
#pragma unroll
    for (int n = 0; n < 16; ++n) w1[n] = src[n];
    float ak = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float4 g = start ? w1[n] : gsrc[n];
      if (copy_gp) gdst[n] = g;
      ak = fmaf(g.x, sk[4 * n], ak);
      ak = fmaf(g.y, sk[4 * n + 1], ak);
      ak = fmaf(g.z, sk[4 * n + 2], ak);
      ak = fmaf(g.w, sk[4 * n + 3], ak);
    }
    const GeluOut ga = gelu_and_grad(ak);
    sx[h] = ga.g;
    sh[h] = ga.dg;  // GELU'(a_h), read back by the same thread in phase 3
  }
  __syncthreads();

  // ---- phase 2 (output mapping): y_i = W2g[i] . x, e_i = 2 (y_i - v_i)
  const int i = t >> 2, s = t & 3;
  const size_t r2 = so + (size_t)i * MLP_HID + 64 * s;  // W2[i][64s ..]
  {
    const float4* src = (const float4*)((start ? a.w2 : a.w2_gp) + r2);
    float4* gdst = copy_gp ? (float4*)(a.w2_gp + r2) : nullptr;
    float y = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float4 g = src[n];
      if (copy_gp) gdst[n] = g;
      const int u = 64 * s + 4 * n;
      y = fmaf(g.x, sx[u], y);
      y = fmaf(g.y, sx[u + 1], y);
      y = fmaf(g.z, sx[u + 2], y);
      y = fmaf(g.w, sx[u + 3], y);
    }
    y = quad_sum(y);
    if (s == 0) se[i] = 2.f * (y - load1<F32IN>(a.v, vo + i));
  }
  __syncthreads();

  // ---- phase 3 (hidden mapping): delta_h = (W2g[:, h] . e) GELU'(a_h);
  // W1[h] -= eta delta_h k; hq_h = GELU(W1[h] . q)
  {
    const float* col = (start ? a.w2 : a.w2_gp) + so + h;
    float bp = 0.f;
#pragma unroll 8
    for (int r = 0; r < 64; ++r) bp = fmaf(col[(size_t)r * MLP_HID], se[r], bp);
    const float nd = -eta * bp * sh[h];
    float aq = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      float4 w = w1[n];
      w.x = fmaf(nd, sk[4 * n], w.x);
      w.y = fmaf(nd, sk[4 * n + 1], w.y);
      w.z = fmaf(nd, sk[4 * n + 2], w.z);
      w.w = fmaf(nd, sk[4 * n + 3], w.w);
      w1[n] = w;
      aq = fmaf(w.x, sq[4 * n], aq);
      aq = fmaf(w.y, sq[4 * n + 1], aq);
      aq = fmaf(w.z, sq[4 * n + 2], aq);
      aq = fmaf(w.w, sq[4 * n + 3], aq);
    }
    float4* dst = (float4*)(a.w + so + (size_t)h * 64);
#pragma unroll
    for (int n = 0; n < 16; ++n) dst[n] = w1[n];
    const float hq = gelu_and_grad(aq).g;
    __syncthreads();  // every thread has read its GELU'(a_h) from sh
    sh[h] = hq;
  }
  __syncthreads();

  // ---- phase 4 (output mapping): W2[i] -= eta e_i x; z_i = W2[i] . hq
  {
    float4* row = (float4*)(a.w2 + r2);
    const float ne = -eta * se[i];
    float z = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      float4 w = row[n];
      const int u = 64 * s + 4 * n;
      w.x = fmaf(ne, sx[u], w.x);
      w.y = fmaf(ne, sx[u + 1], w.y);
      w.z = fmaf(ne, sx[u + 2], w.z);
      w.w = fmaf(ne, sx[u + 3], w.w);
      row[n] = w;
      z = fmaf(w.x, sh[u], z);
      z = fmaf(w.y, sh[u + 1], z);
      z = fmaf(w.z, sh[u + 2], z);
      z = fmaf(w.w, sh[u + 3], z);
    }
    z = quad_sum(z);
    if (s == 0) a.z[vo + i] = z;
  }
}

}  // namespace

hipError_t launch_linear_step(const StepArgs& a, bool f32in, hipStream_t s) {
  if (f32in)
    hipLaunchKernelGGL(linear_step_kernel<true>, dim3(a.units), dim3(STEP_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(linear_step_kernel<false>, dim3(a.units), dim3(STEP_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_linear_ln_step(const StepArgs& a, const float* gamma, const float* beta,
                                 float eps, bool f32in, hipStream_t s) {
  if (f32in)
    hipLaunchKernelGGL(linear_ln_step_kernel<true>, dim3(a.units), dim3(STEP_THREADS), 0, s, a,
                       gamma, beta, eps);
  else
    hipLaunchKernelGGL(linear_ln_step_kernel<false>, dim3(a.units), dim3(STEP_THREADS), 0, s, a,
                       gamma, beta, eps);
  return hipGetLastError();
}

hipError_t launch_mlp_step(const StepArgs& a, bool f32in, hipStream_t s) {
  if (f32in)
    hipLaunchKernelGGL(mlp_step_kernel<true>, dim3(a.units), dim3(STEP_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(mlp_step_kernel<false>, dim3(a.units), dim3(STEP_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
