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
// One workgroup of 256 threads per unit.  Every step lays each state row
// across consecutive lanes (16 B per lane), so a wave-wide load or store
// moves 1 KB of consecutive memory; row sums are 16-lane DPP rotation sums.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int STEP_THREADS = 256;

// sum over each group of 16 consecutive lanes, in every lane of the group
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF,
                                                          0xF, false));  // row_ror:8
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF,
                                                          0xF, false));  // row_ror:4
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xF,
                                                          0xF, false));  // row_ror:2
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xF,
                                                          0xF, false));  // row_ror:1
  return x;
}
// sum over the whole wave, the same value in every lane
__device__ __forceinline__ float wave_total(float x) {
  const int s = __builtin_bit_cast(int, row16_sum(x));
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 48)));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
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
// A row of W (64 values, 256 bytes) spans a group of 16 lanes, 4 values per
// lane: wave w, register n, lane l hold row 16 w + 4 n + l / 16, columns
// 4 (l % 16) .. + 3, so every wave-wide state load or store moves 1 KB of
// consecutive memory.  Row dot products are in-lane sums plus a 16-lane DPP
// rotation sum; rows are independent, so no lane exchanges data beyond its
// group.  Each state element is read before it is written, by the same lane.
template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) linear_step_kernel(StepArgs a) {
  const int unit = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, c1 = l & 15;
  const int r0 = 16 * w + (l >> 4);                 // rows r0 + 4 n
  const int bi = unit / a.H;
  const size_t vo = (size_t)unit * 64;              // this unit's token vectors
  const size_t so = (size_t)unit * 4096;
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;
  const float4 k4 = make_float4(load1<F32IN>(a.k, vo + 4 * c1), load1<F32IN>(a.k, vo + 4 * c1 + 1),
                                load1<F32IN>(a.k, vo + 4 * c1 + 2), load1<F32IN>(a.k, vo + 4 * c1 + 3));
  const float4 q4 = make_float4(load1<F32IN>(a.q, vo + 4 * c1), load1<F32IN>(a.q, vo + 4 * c1 + 1),
                                load1<F32IN>(a.q, vo + 4 * c1 + 2), load1<F32IN>(a.q, vo + 4 * c1 + 3));
  const float eta = a.eta[unit];
  float4* wr = (float4*)(a.w + so) + c1;
  float4 W[4], G[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) W[n] = wr[(r0 + 4 * n) * 16];
  if (start || a.w_gp == nullptr) {
#pragma unroll
    for (int n = 0; n < 4; ++n) G[n] = W[n];
  } else {
    const float4* gr = (const float4*)(a.w_gp + so) + c1;
#pragma unroll
    for (int n = 0; n < 4; ++n) G[n] = gr[(r0 + 4 * n) * 16];
  }
  if (start && a.w_gp != nullptr) {  // the gradient point of the new mini-batch
    float4* gr = (float4*)(a.w_gp + so) + c1;
#pragma unroll
    for (int n = 0; n < 4; ++n) gr[(r0 + 4 * n) * 16] = W[n];
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i = r0 + 4 * n;
    const float y = row16_sum(dot4(G[n], k4));
    const float ng = -2.f * eta * (y - load1<F32IN>(a.v, vo + i));  // -eta g_i
    float4 v = W[n];
    v.x = fmaf(ng, k4.x, v.x);
    v.y = fmaf(ng, k4.y, v.y);
    v.z = fmaf(ng, k4.z, v.z);
    v.w = fmaf(ng, k4.w, v.w);
    wr[i * 16] = v;
    const float zq = row16_sum(dot4(v, q4));
    if (c1 == 0) a.z[vo + i] = zq;
  }
}

// ------------------------------------- TTT-Linear with LayerNorm + residual
// f(x) = x + LN(W x), rows laid out as in the TTT-Linear step (16 lanes per
// row, lane group l / 16 of wave w holding rows 16 w + l / 16 + 4 n).  The
// LN statistics are sums over the 64 rows: a lane group sums its 4 rows in
// registers, the wave reads its four groups' sums out of lanes 0, 16, 32,
// 48, and the 4 wave partials meet in LDS.
// Sums over the 64 rows of two values already summed over this lane group's
// rows; every call site passes its own 4-entry LDS buffer, so one barrier
// suffices.
__device__ __forceinline__ float2 rows_total2(float x, float y, float2* red, int w, int l) {
  const int xi = __builtin_bit_cast(int, x), yi = __builtin_bit_cast(int, y);
  auto groups = [](int v) {
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 48)));
  };
  const float xw = groups(xi), yw = groups(yi);
  if (l == 0) red[w] = make_float2(xw, yw);
  __syncthreads();
  const float2 r0 = red[0], r1 = red[1], r2 = red[2], r3 = red[3];
  return make_float2((r0.x + r1.x) + (r2.x + r3.x), (r0.y + r1.y) + (r2.y + r3.y));
}

template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) linear_ln_step_kernel(StepArgs a, const float* gamma,
                                                                      const float* beta, float eps) {
  __shared__ float2 red[3][4];
  const int unit = blockIdx.x;
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, c1 = l & 15;
  const int r0 = 16 * w + (l >> 4);                 // rows r0 + 4 n
  const int bi = unit / a.H, head = unit % a.H;
  const size_t vo = (size_t)unit * 64;
  const size_t so = (size_t)unit * 4096;
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;
  const float4 k4 = make_float4(load1<F32IN>(a.k, vo + 4 * c1), load1<F32IN>(a.k, vo + 4 * c1 + 1),
                                load1<F32IN>(a.k, vo + 4 * c1 + 2), load1<F32IN>(a.k, vo + 4 * c1 + 3));
  const float4 q4 = make_float4(load1<F32IN>(a.q, vo + 4 * c1), load1<F32IN>(a.q, vo + 4 * c1 + 1),
                                load1<F32IN>(a.q, vo + 4 * c1 + 2), load1<F32IN>(a.q, vo + 4 * c1 + 3));
  const float eta = a.eta[unit];
  float gi[4], be[4], ki[4], qi[4], vi[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i = r0 + 4 * n;
    gi[n] = gamma[head * 64 + i];
    be[n] = beta[head * 64 + i];
    ki[n] = load1<F32IN>(a.k, vo + i);
    qi[n] = load1<F32IN>(a.q, vo + i);
    vi[n] = load1<F32IN>(a.v, vo + i);
  }
  float4* wr = (float4*)(a.w + so) + c1;
  float4 W[4], G[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) W[n] = wr[(r0 + 4 * n) * 16];
  if (start || a.w_gp == nullptr) {
#pragma unroll
    for (int n = 0; n < 4; ++n) G[n] = W[n];
  } else {
    const float4* gr = (const float4*)(a.w_gp + so) + c1;
#pragma unroll
    for (int n = 0; n < 4; ++n) G[n] = gr[(r0 + 4 * n) * 16];
  }
  if (start && a.w_gp != nullptr) {
    float4* gr = (float4*)(a.w_gp + so) + c1;
#pragma unroll
    for (int n = 0; n < 4; ++n) gr[(r0 + 4 * n) * 16] = W[n];
  }
  // forward on the training view at the gradient point: y = Wg k, mean and
  // population variance over the 64 rows (one pass: E[y^2] - mu^2, >= 0)
  float y[4], sy1 = 0.f, sy2 = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    y[n] = row16_sum(dot4(G[n], k4));
    sy1 += y[n];
    sy2 = fmaf(y[n], y[n], sy2);
  }
  const float2 sy = rows_total2(sy1, sy2, red[0], w, l);
  const float mu = sy.x * (1.f / 64);
  const float rs = rsqrtf(fmaxf(fmaf(sy.y, 1.f / 64, -mu * mu), 0.f) + eps);
  // dl/dyhat = 2 gamma (k + gamma yhat + beta - v); LayerNorm VJP
  float yh[4], gy[4], sg1 = 0.f, sg2 = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    yh[n] = (y[n] - mu) * rs;
    gy[n] = 2.f * gi[n] * ((ki[n] + fmaf(gi[n], yh[n], be[n])) - vi[n]);
    sg1 += gy[n];
    sg2 = fmaf(gy[n], yh[n], sg2);
  }
  const float2 m = rows_total2(sg1, sg2, red[1], w, l);
  float o[4], so1 = 0.f, so2 = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float gr = rs * (gy[n] - m.x * (1.f / 64) - yh[n] * (m.y * (1.f / 64)));
    const float ng = -eta * gr;
    float4 v = W[n];
    v.x = fmaf(ng, k4.x, v.x);
    v.y = fmaf(ng, k4.y, v.y);
    v.z = fmaf(ng, k4.z, v.z);
    v.w = fmaf(ng, k4.w, v.w);
    wr[(r0 + 4 * n) * 16] = v;
    o[n] = row16_sum(dot4(v, q4));
    so1 += o[n];
    so2 = fmaf(o[n], o[n], so2);
  }
  // z = q + LN(W q)
  const float2 sz = rows_total2(so1, so2, red[2], w, l);
  const float mo = sz.x * (1.f / 64);
  const float ro = rsqrtf(fmaxf(fmaf(sz.y, 1.f / 64, -mo * mo), 0.f) + eps);
  if (c1 == 0) {
#pragma unroll
    for (int n = 0; n < 4; ++n) a.z[vo + r0 + 4 * n] = qi[n] + fmaf(gi[n], (o[n] - mo) * ro, be[n]);
  }
}

// ------------------------------------------------------------------ TTT-MLP
// f(x) = W2 GELU(W1 x), hidden width 256 (§4.4).  At the gradient point:
//   a = W1g k, x = GELU(a), e = 2 (W2g x - v), delta = (W2g^T e) * GELU'(a);
// W2 -= eta e x^T, W1 -= eta delta k^T; z = W2 GELU(W1 q).
// Every state access is a whole-row access across lanes, so each wave-wide
// load or store moves 1 KB of consecutive memory: a W1 row (64 values) is
// spread over a 16-lane group (4 values per lane; wave w, register n, lane l
// hold row 64 w + 4 n + l / 16), a W2 row (256 values) over a whole wave
// (wave w, register n hold row 16 w + n, lane l columns 4 l .. 4 l + 3).
// Row dot products are in-lane sums plus a 16-lane DPP rotation sum (and,
// for W2 rows, the four 16-lane sums read out of lanes 0, 16, 32, 48); the
// sum over W2's rows for delta is in-lane over a wave's 16 rows plus one
// LDS exchange between the four waves.  Every state element is read before
// it is written, by the same lane.
// GELU(x) = x Phi(x) with erf from Abramowitz & Stegun 7.1.26 (|err| <=
// 1.5e-7), the same function as the MLP scan's (gelu_and_grad).
constexpr int MLP_HID = 256;

template <bool F32IN>
__global__ void __launch_bounds__(STEP_THREADS) mlp_step_kernel(StepArgs a) {
  __shared__ float4 sk[16], sq[16], sx[MLP_HID / 4], shq[MLP_HID / 4];
  __shared__ float sg[MLP_HID], sd[MLP_HID], pd[4][MLP_HID];
  const int unit = blockIdx.x, t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int bi = unit / a.H;
  const size_t vo = (size_t)unit * 64;
  const size_t so = (size_t)unit * (MLP_HID * 64);
  const bool start = minibatch_pos(a.pos[bi], a.b) == 0;  // always when b == 1
  const bool copy_gp = start && a.w_gp != nullptr;  // gradient points may be NULL for b == 1
  const float eta = a.eta[unit];
  if (t < 64) {
    ((float*)sk)[t] = load1<F32IN>(a.k, vo + t);
    ((float*)sq)[t] = load1<F32IN>(a.q, vo + t);
  }
  __syncthreads();

  // ---- phase 1: a_h = W1g[h] . k for this lane group's 16 rows
  const int c1 = l & 15;                       // W1: columns 4 c1 .. 4 c1 + 3
  const int h0 = 64 * w + (l >> 4);            // W1: rows h0 + 4 n
  const float4 k4 = sk[c1], q4 = sq[c1];
  float4 w1[16];
  {
    const float4* g1 = (const float4*)((start ? a.w : a.w_gp) + so) + c1;
#pragma unroll
    for (int n = 0; n < 16; ++n) w1[n] = g1[(h0 + 4 * n) * 16];
    if (copy_gp) {
      float4* d1 = (float4*)(a.w_gp + so) + c1;
#pragma unroll
      for (int n = 0; n < 16; ++n) d1[(h0 + 4 * n) * 16] = w1[n];
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float ah = row16_sum(dot4(w1[n], k4));
      const GeluOut ga = gelu_and_grad(ah);
      if (c1 == 0) {
        ((float*)sx)[h0 + 4 * n] = ga.g;
        sg[h0 + 4 * n] = ga.dg;  // GELU'(a_h)
      }
    }
  }
  __syncthreads();

  // ---- phase 2: y_i = W2g[i] . x, e_i = 2 (y_i - v_i) for this wave's 16 rows,
  // then this wave's share of W2g^T e
  const int i0 = 16 * w;
  float4 w2[16];
  float ev[16];
  {
    const float4* g2 = (const float4*)((start ? a.w2 : a.w2_gp) + so) + l;
#pragma unroll
    for (int n = 0; n < 16; ++n) w2[n] = g2[(i0 + n) * 64];
    if (copy_gp) {
      float4* d2 = (float4*)(a.w2_gp + so) + l;
#pragma unroll
      for (int n = 0; n < 16; ++n) d2[(i0 + n) * 64] = w2[n];
    }
    const float4 x4 = sx[l];
    float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float y = wave_total(dot4(w2[n], x4));
      ev[n] = 2.f * (y - load1<F32IN>(a.v, vo + i0 + n));
      part.x = fmaf(w2[n].x, ev[n], part.x);
      part.y = fmaf(w2[n].y, ev[n], part.y);
      part.z = fmaf(w2[n].z, ev[n], part.z);
      part.w = fmaf(w2[n].w, ev[n], part.w);
    }
    *(float4*)&pd[w][4 * l] = part;
  }
  __syncthreads();
  // delta_h = (W2g^T e)_h GELU'(a_h), thread t -> h = t
  sd[t] = ((pd[0][t] + pd[1][t]) + (pd[2][t] + pd[3][t])) * sg[t];
  __syncthreads();

  // ---- phase 3: W1[h] -= eta delta_h k; hq_h = GELU(W1[h] . q)
  {
    float4* r1 = (float4*)(a.w + so) + c1;
    if (!start) {
#pragma unroll
      for (int n = 0; n < 16; ++n) w1[n] = r1[(h0 + 4 * n) * 16];
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float nd = -eta * sd[h0 + 4 * n];
      float4 v = w1[n];
      v.x = fmaf(nd, k4.x, v.x);
      v.y = fmaf(nd, k4.y, v.y);
      v.z = fmaf(nd, k4.z, v.z);
      v.w = fmaf(nd, k4.w, v.w);
      r1[(h0 + 4 * n) * 16] = v;
      const float aq = row16_sum(dot4(v, q4));
      if (c1 == 0) ((float*)shq)[h0 + 4 * n] = gelu_and_grad(aq).g;
    }
  }
  __syncthreads();

  // ---- phase 4: W2[i] -= eta e_i x; z_i = W2[i] . hq
  {
    float4* r2 = (float4*)(a.w2 + so) + l;
    if (!start) {
#pragma unroll
      for (int n = 0; n < 16; ++n) w2[n] = r2[(i0 + n) * 64];
    }
    const float4 x4 = sx[l], hq4 = shq[l];
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const float ne = -eta * ev[n];
      float4 v = w2[n];
      v.x = fmaf(ne, x4.x, v.x);
      v.y = fmaf(ne, x4.y, v.y);
      v.z = fmaf(ne, x4.z, v.z);
      v.w = fmaf(ne, x4.w, v.w);
      r2[(i0 + n) * 64] = v;
      const float z = wave_total(dot4(v, hq4));
      if (l == 0) a.z[vo + i0 + n] = z;
    }
  }
}

}  // namespace

hipError_t launch_linear_step(const StepArgs& a, bool f32in, hipStream_t s) {
  return launch(f32in ? linear_step_kernel<true> : linear_step_kernel<false>, dim3(a.units),
                dim3(STEP_THREADS), s, a);
}

hipError_t launch_linear_ln_step(const StepArgs& a, const float* gamma, const float* beta,
                                 float eps, bool f32in, hipStream_t s) {
  return launch(f32in ? linear_ln_step_kernel<true> : linear_ln_step_kernel<false>, dim3(a.units),
                dim3(STEP_THREADS), s, a, gamma, beta, eps);
}

hipError_t launch_mlp_step(const StepArgs& a, bool f32in, hipStream_t s) {
  return launch(f32in ? mlp_step_kernel<true> : mlp_step_kernel<false>, dim3(a.units),
                dim3(STEP_THREADS), s, a);
}

}  // namespace ttt
