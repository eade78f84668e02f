// TTT-Linear training support in the primal form, one token at a time, in
// fp32 arithmetic: the checkpointing forward and the backward for fp32
// q/k/v, every mini-batch size.  (bf16 q/k/v take the dual-form kernels of
// ttt_linear_bf16.hip / ttt_linear_bwd.hip for every b.)
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): f(x) = W x (§4.4), loss ||W k_t - v_t||^2 (§3.3),
// mini-batch GD with the gradient at the state before the mini-batch (§3.5),
// per-token eta (§4.6), output from the updated state (§3.1):
//   g_t = 2 (Wg k_t - v_t),  W <- W - eta_t g_t k_t^T,  z_t = W q_t,
// Wg the state before token t's mini-batch.  The forward keeps the state at
// every mini-batch start (the kappa = T / b checkpoints of §6.12).  The
// backward walks the mini-batches in reverse.  It replays each forward from
// its checkpoint to its end state, then takes its tokens back (W += eta g k^T)
// while it propagates, with A the adjoint of the state after token t and G
// that of the gradient point:
//   dq = W^T dz,  A += dz q^T,  gb = -eta A k,  deta = -g^T A k,
//   dk = -eta A^T g + 2 Wg^T gb,  dv = -2 gb,  G += 2 gb k^T,
//   at the mini-batch's first token: A += G, G = 0.
//
// Work split: one workgroup of 256 threads per (batch, head) unit.  Thread
// (wave v, lane l) owns row i = 16 v + (l % 16) and the quarter j in
// [16 qd, 16 qd + 16), qd = l / 16, of the columns: W, Wg, A and G in
// registers.  Row sums (W k, W q, A k) combine the four quarters with lane
// swaps; column sums (dq, dk) add the 16 rows of a DPP row and the 4 waves'
// partials in LDS.  The replay needs no barrier (rows are independent).
// Each reverse step needs one barrier.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int LTHREADS = 256;

__device__ __forceinline__ float row16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ float ld(const void* p, size_t i) { return ((const float*)p)[i]; }

// The checkpointing forward: z, the final state, and the state before every
// mini-batch, w_ckpt [units][ceil(T/b)][64][64].
__global__ void __launch_bounds__(LTHREADS) linear_primal_ckpt_kernel(LinearArgs a) {
  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int qd = l >> 4, il = l & 15;
  const int i = 16 * wv + il, j0 = 16 * qd;
  const int unit = blockIdx.x, head = unit % a.H;
  const int T = a.T, b = a.b;
  const int nmb = (T + b - 1) / b;
  const float* w0 = a.w0 + (size_t)(a.w0_per_batch ? unit : head) * 4096;
  float w[16], wg[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) w[c] = w0[i * 64 + j0 + c];
  const size_t base = (size_t)unit * T * 64;
  for (int tt = 0; tt < T; ++tt) {
    if (tt % b == 0) {
      float* ck = a.w_ckpt + ((size_t)unit * nmb + tt / b) * 4096;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        wg[c] = w[c];
        ck[i * 64 + j0 + c] = w[c];
      }
    }
    const size_t o = base + (size_t)tt * 64;
    float p = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) p = fmaf(wg[c], ld(a.k, o + j0 + c), p);
    const float g = 2.f * (quad_sum(p) - ld(a.v, o + i));
    const float eg = -a.eta[(size_t)unit * T + tt] * g;
    float zq = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      w[c] = fmaf(eg, ld(a.k, o + j0 + c), w[c]);
      zq = fmaf(w[c], ld(a.q, o + j0 + c), zq);
    }
    zq = quad_sum(zq);
    if (qd == 0) a.z[o + i] = zq;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) a.w_out[(size_t)unit * 4096 + i * 64 + j0 + c] = w[c];
}

// The backward: per unit, from the checkpoints of the forward above.
__global__ void __launch_bounds__(LTHREADS) linear_primal_bwd_kernel(LinearPrimalBwdArgs a) {
  __shared__ float part[2][4][129];  // [step parity][wave][dq 0..63 | dk 64..127 | deta 128]

  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int qd = l >> 4, il = l & 15;
  const int i = 16 * wv + il, j0 = 16 * qd;
  const int unit = blockIdx.x;
  const int T = a.T, b = a.b;
  const int nmb = (T + b - 1) / b;
  const size_t base = (size_t)unit * T * 64;

  float w[16], wg[16], A[16], G[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    A[c] = a.dw_T ? a.dw_T[(size_t)unit * 4096 + i * 64 + j0 + c] : 0.f;
    G[c] = 0.f;
  }
  int n = 0;  // reverse steps taken (selects the LDS partial buffer)
  for (int m = nmb - 1; m >= 0; --m) {
    const int m0 = m * b, m1 = min(T, m0 + b);
    const float* ck = a.w_ckpt + ((size_t)unit * nmb + m) * 4096;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      wg[c] = ck[i * 64 + j0 + c];
      w[c] = wg[c];
    }
    // replay the mini-batch to its end state
    for (int tt = m0; tt < m1; ++tt) {
      const size_t o = base + (size_t)tt * 64;
      float p = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) p = fmaf(wg[c], ld(a.k, o + j0 + c), p);
      const float g = 2.f * (quad_sum(p) - ld(a.v, o + i));
      const float eg = -a.eta[(size_t)unit * T + tt] * g;
#pragma unroll
      for (int c = 0; c < 16; ++c) w[c] = fmaf(eg, ld(a.k, o + j0 + c), w[c]);
    }
    // take its tokens back
    for (int tt = m1 - 1; tt >= m0; --tt, ++n) {
      const size_t o = base + (size_t)tt * 64;
      const float eta = a.eta[(size_t)unit * T + tt];
      float kv[16], qv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        kv[c] = ld(a.k, o + j0 + c);
        qv[c] = ld(a.q, o + j0 + c);
      }
      const float dzi = a.dz[o + i];
      float p = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) p = fmaf(wg[c], kv[c], p);
      const float g = 2.f * (quad_sum(p) - ld(a.v, o + i));
      // dq (column sums of W dz over the rows); then the output's adjoint
      float dqm = 0.f, ak = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float rs = row16(w[c] * dzi);
        if (il == c) dqm = rs;
        A[c] = fmaf(dzi, qv[c], A[c]);
        ak = fmaf(A[c], kv[c], ak);
      }
      ak = quad_sum(ak);
      const float gb = -eta * ak;
      float dkm = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float rs = row16(fmaf(-eta * A[c], g, 2.f * wg[c] * gb));
        if (il == c) dkm = rs;
      }
      const float de = row16(qd == 0 ? -g * ak : 0.f);
      float* pp = part[n & 1][wv];
      pp[j0 + il] = dqm;
      pp[64 + j0 + il] = dkm;
      if (l == 0) pp[128] = de;
      if (qd == 0) a.dv[o + i] = -2.f * gb;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        G[c] = fmaf(2.f * gb, kv[c], G[c]);
        w[c] = fmaf(eta * g, kv[c], w[c]);  // the state before token tt
      }
      if (tt == m0) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          A[c] += G[c];
          G[c] = 0.f;
        }
      }
      __syncthreads();
      if (t < 128) {
        const float* q4 = &part[n & 1][0][0];
        const float s = q4[t] + q4[129 + t] + q4[258 + t] + q4[387 + t];
        (t < 64 ? a.dq : a.dk)[o + (t & 63)] = s;
      } else if (t == 128) {
        const float* q4 = &part[n & 1][0][0];
        a.deta[(size_t)unit * T + tt] = q4[128] + q4[257] + q4[386] + q4[515];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) a.dw0[(size_t)unit * 4096 + i * 64 + j0 + c] = A[c];
}

}  // namespace

hipError_t launch_linear_primal_ckpt(const LinearArgs& a, hipStream_t s) {
  return launch(linear_primal_ckpt_kernel, dim3(a.units), dim3(LTHREADS), s, a);
}

hipError_t launch_linear_primal_bwd(const LinearPrimalBwdArgs& a, hipStream_t s) {
  return launch(linear_primal_bwd_kernel, dim3(a.units), dim3(LTHREADS), s, a);
}

}  // namespace ttt
