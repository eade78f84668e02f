// TTT-MLP scan in the primal form, one token at a time, in fp32 arithmetic:
// the path for fp32 q/k/v (whose 1e-5 budget wants exact fp32 products) and
// for mini-batches longer than one 16-token tile (b a multiple of 16 above
// 16), where the gradient point must be held across tiles.  The bf16 dual-form
// kernel (ttt_mlp.hip) serves bf16 inputs with b | 16.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): f(x) = W2 GELU(W1 x) (§4.4), loss
// ||f(k_t) - v_t||^2 (§3.3), mini-batch GD with both layers' gradients at the
// state before the mini-batch (§3.5), per-token eta (§4.6), output from the
// updated state (§3.1).  Per token t with gradient point (W1g, W2g):
//   a = W1g k,  x = GELU(a),  e = 2 (W2g x - v),
//   delta = (W2g^T e) * GELU'(a),
//   W2 -= eta e x^T,  W1 -= eta delta k^T,
//   z = W2 GELU(W1 q);
// at the first token of a mini-batch the gradient point is set to the state.
// GELU(x) = x Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, with the device
// library's erff and expf.  The primal form equals the dual form (§3.6/§3.7)
// exactly in real arithmetic; it is the per-token recurrence the dual form
// reorganises.
//
// Work split: one workgroup of 1024 threads (16 waves) per (batch, head) unit.
// Thread (wave v, lane l) owns hidden unit u = 16 v + (l % 16) and the quarter
// j in [16 qd, 16 qd + 16), qd = l / 16, of the 64 input / output components:
// W1[u][j], W2[j][u] and their gradient-point copies in registers.  Sums over
// j (W1 k, W1 q, W2^T e) combine the four quarters with lane swaps; sums over
// u (W2 x, W2 x_q) add the 16 lanes of a DPP row and then the 16 waves'
// partials in LDS.  Tokens are staged in LDS in double-buffered chunks of 16.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int PHID = 256;        // hidden units
constexpr int PCH = 16;          // tokens per staged chunk
constexpr int PTHREADS = 1024;   // 16 waves: 16 hidden units x 4 quarters per wave
constexpr int PSTRIDE = 3 * 64 + 1;  // floats per staged token: k, v, q, eta

__device__ __forceinline__ float gelu_phi(float x) {
  return 0.5f * (1.f + erff(x * 0.70710678118654752f));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}

// Sum over the four quarters (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float quarter_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <bool F32IN>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (F32IN) return ((const float*)p)[i];
  else return bf16_val(((const short*)p)[i]);
}

template <bool F32IN>
__global__ void __launch_bounds__(PTHREADS) mlp_primal_kernel(MlpArgs a) {
  __shared__ float tok[2][PCH * PSTRIDE];  // staged tokens: k[64] v[64] q[64] eta
  __shared__ float red[2][16][64];         // per-wave partial sums over u (y, z)
  __shared__ float ebuf[64];               // e of the current token

  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int qd = l >> 4, ul = l & 15;
  const int u = 16 * wv + ul, j0 = 16 * qd;
  const int unit = blockIdx.x;
  const int head = unit % a.H;
  const int T = a.T, b = a.b;

  const size_t wsel = a.w0_per_batch ? unit : head;
  const float* w1g0 = a.w1_0 + wsel * PHID * 64;
  const float* w2g0 = a.w2_0 + wsel * 64 * PHID;
  float w1[16], w2[16], w1g[16], w2g[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w1[i] = w1g0[u * 64 + j0 + i];
    w2[i] = w2g0[(j0 + i) * PHID + u];
    w1g[i] = w1[i];
    w2g[i] = w2[i];
  }

  const size_t base = (size_t)unit * T * 64;
  // stage tokens [c * PCH, c * PCH + PCH) into buffer c & 1 (zeros past T)
  auto stage = [&](int c) {
    float* dst = tok[c & 1];
    for (int e = t; e < PCH * PSTRIDE; e += PTHREADS) {
      const int s = e / PSTRIDE, f = e % PSTRIDE, tt = c * PCH + s;
      float val = 0.f;
      if (tt < T) {
        if (f < 64) val = load_in<F32IN>(a.k, base + (size_t)tt * 64 + f);
        else if (f < 128) val = load_in<F32IN>(a.v, base + (size_t)tt * 64 + f - 64);
        else if (f < 192) val = load_in<F32IN>(a.q, base + (size_t)tt * 64 + f - 128);
        else val = a.eta[(size_t)unit * T + tt];
      }
      dst[e] = val;
    }
  };
  stage(0);
  __syncthreads();

  float* zu = a.z + base;
  const int nchunks = (T + PCH - 1) / PCH;
  for (int c = 0; c < nchunks; ++c) {
    const float* tc = tok[c & 1];
    const int s_end = min(PCH, T - c * PCH);
    for (int s = 0; s < s_end; ++s) {
      const int tt = c * PCH + s;
      const float* kt = tc + s * PSTRIDE;
      const float* vt = kt + 64;
      const float* qt = kt + 128;
      const float eta = kt[192];
      if (tt % b == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          w1g[i] = w1[i];
          w2g[i] = w2[i];
        }
      }
      // forward at the gradient point
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(w1g[i], kt[j0 + i], acc);
      const float av = quarter_sum(acc);
      const float ph = gelu_phi(av);
      const float x = av * ph;
      const float dg = fmaf(av, expf(-0.5f * av * av) * 0.39894228040143268f, ph);
      // y = W2g x: this lane's 16 components over its hidden unit, summed over
      // the row's 16 units; lane ul keeps component j0 + ul
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float rs = row_sum16(w2g[i] * x);
        if (ul == i) mine = rs;
      }
      red[0][wv][j0 + ul] = mine;
      // the previous token's output: its z partials were written to red[1]
      __syncthreads();  // B1
      if (t < 64) {
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) y += red[0][w][t];
        ebuf[t] = 2.f * (y - vt[t]);
        if (tt > 0) {
          float zs = 0.f;
#pragma unroll
          for (int w = 0; w < 16; ++w) zs += red[1][w][t];
          zu[(size_t)(tt - 1) * 64 + t] = zs;
        }
      }
      __syncthreads();  // B2
      // backward to the first layer, then both updates
      acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(w2g[i], ebuf[j0 + i], acc);
      const float delta = quarter_sum(acc) * dg;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        w2[i] = fmaf(-eta * ebuf[j0 + i], x, w2[i]);
        w1[i] = fmaf(-eta * delta, kt[j0 + i], w1[i]);
      }
      // output from the updated state
      acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(w1[i], qt[j0 + i], acc);
      const float aq = quarter_sum(acc);
      const float xq = aq * gelu_phi(aq);
      mine = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float rs = row_sum16(w2[i] * xq);
        if (ul == i) mine = rs;
      }
      red[1][wv][j0 + ul] = mine;
      // the next chunk is staged once every thread is past this chunk's first
      // B1, i.e. done with the buffer it overwrites (read last by the previous
      // chunk's final token, before that B1)
      if (s == 0 && c + 1 < nchunks) stage(c + 1);
    }
  }
  __syncthreads();
  if (t < 64 && T > 0) {
    float zs = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) zs += red[1][w][t];
    zu[(size_t)(T - 1) * 64 + t] = zs;
  }
  float* w1o = a.w1_out + (size_t)unit * PHID * 64;
  float* w2o = a.w2_out + (size_t)unit * 64 * PHID;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w1o[u * 64 + j0 + i] = w1[i];
    w2o[(j0 + i) * PHID + u] = w2[i];
  }
}

}  // namespace

hipError_t launch_mlp_primal(const MlpArgs& a, bool f32in, hipStream_t s) {
  if (f32in) return launch(mlp_primal_kernel<true>, dim3(a.units), dim3(PTHREADS), s, a);
  return launch(mlp_primal_kernel<false>, dim3(a.units), dim3(PTHREADS), s, a);
}

}  // namespace ttt
