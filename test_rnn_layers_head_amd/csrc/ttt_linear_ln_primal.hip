// TTT-Linear with the LayerNorm + residual inner model in the primal form,
// one token at a time, in fp32 arithmetic: the forward for every mini-batch
// size and fp32 q/k/v (optionally keeping the state before every mini-batch),
// and the backward from those checkpoints.  (bf16 q/k/v with 16 | b take the
// dual-form forward of ttt_linear_ln.hip.)
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): f(x) = x + LN(W x) (§4.4) with
// LN(y) = gamma (y - mean y) / sqrt(var y + eps) + beta over the 64 output
// components (population variance), loss ||f(k) - v||^2 (§3.3) differentiated
// through the LayerNorm at the state before the mini-batch (§3.5), per-token
// eta (§4.6), output from the updated state (§3.1).  Per token, at the
// gradient point Wg:
//   y = Wg k, c = y - mean y, rs = (mean c^2 + eps)^-1/2, yh = c rs,
//   g = 2 gamma (k + gamma yh + beta - v),
//   dy = rs (g - mean g - yh mean(g yh)),   W <- W - eta dy k^T,
//   z = q + gamma LNhat(W q) + beta.
// The backward (§6.12) replays each mini-batch from its checkpoint, then
// takes its tokens back, applying every forward operation's adjoint in
// reverse order.  A is the adjoint of the state after the token and Ag that
// of the gradient point (added to A at the mini-batch's first token).
// dgamma and dbeta are summed over the tokens, per unit.
//
// Work split: one workgroup of 256 threads per (batch, head) unit.  Thread
// (wave v, lane l) owns row i = 16 v + (l % 16) and the quarter j in
// [16 qd, 16 qd + 16), qd = l / 16, of the columns of W (and of Wg, A, Ag).
// Row sums (W k, W q, A k) combine the four quarters with lane swaps.  Sums
// over the 64 rows (the LayerNorm statistics and their adjoints) add the 16
// rows of a DPP row and the 4 waves' partials through a rotating set of LDS
// slots, one barrier per sum; column sums (dq, dk) likewise.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int NTHR = 256;
constexpr int NSLOT = 3;  // rotating LDS slots for the sums over rows
constexpr int SLOTW = 8;  // values per slot and wave

__device__ __forceinline__ float rowsum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}
__device__ __forceinline__ float qsum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
template <bool F32IN>
__device__ __forceinline__ float ldx(const void* p, size_t i) {
  if constexpr (F32IN) return ((const float*)p)[i];
  else return bf16_val(((const short*)p)[i]);
}

// Sums over the 64 rows of N per-row values (held by every lane of a row);
// every thread gets the totals.  `ctr` counts the sums taken (selects the slot).
template <int N>
__device__ __forceinline__ void rows_sum(float (&v)[N], float (*slots)[4][SLOTW], int& ctr, int wv,
                                         int l) {
  static_assert(N <= SLOTW, "slot width");
  float r[N];
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = rowsum16(v[n]);  // DPP row 0..3 each hold 16 rows' sum
  float* s = slots[ctr % NSLOT][wv];
  if (l == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) s[n] = r[n];
  }
  __syncthreads();
  const float* t = slots[ctr % NSLOT][0];
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = t[n] + t[SLOTW + n] + t[2 * SLOTW + n] + t[3 * SLOTW + n];
  ++ctr;
}

// The token's LayerNorm statistics of y (per row i): c = y - mean, rs.
__device__ __forceinline__ void ln_stats(float y, float eps, float (*slots)[4][SLOTW], int& ctr,
                                         int wv, int l, float& c, float& rs) {
  float s1[1] = {y};
  rows_sum<1>(s1, slots, ctr, wv, l);
  c = y - s1[0] * (1.f / 64.f);
  float s2[1] = {c * c};
  rows_sum<1>(s2, slots, ctr, wv, l);
  rs = 1.f / sqrtf(s2[0] * (1.f / 64.f) + eps);
}

template <bool F32IN, bool CKPT>
__global__ void __launch_bounds__(NTHR) linear_ln_primal_fwd_kernel(LinearLnArgs a) {
  __shared__ float slots[NSLOT][4][SLOTW];
  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int qd = l >> 4, il = l & 15;
  const int i = 16 * wv + il, j0 = 16 * qd;
  const LinearArgs& s = a.s;
  const int unit = blockIdx.x, head = unit % s.H;
  const int T = s.T, b = s.b;
  const int nmb = (T + b - 1) / b;
  const float gam = a.gamma[head * 64 + i], bet = a.beta[head * 64 + i], eps = a.eps;
  const float* w0 = s.w0 + (size_t)(s.w0_per_batch ? unit : head) * 4096;
  float w[16], wg[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) w[c] = w0[i * 64 + j0 + c];
  const size_t base = (size_t)unit * T * 64;
  int ctr = 0;
  for (int tt = 0; tt < T; ++tt) {
    if (tt % b == 0) {
#pragma unroll
      for (int c = 0; c < 16; ++c) wg[c] = w[c];
      if constexpr (CKPT) {
        float* ck = s.w_ckpt + ((size_t)unit * nmb + tt / b) * 4096;
#pragma unroll
        for (int c = 0; c < 16; ++c) ck[i * 64 + j0 + c] = w[c];
      }
    }
    const size_t o = base + (size_t)tt * 64;
    const float eta = s.eta[(size_t)unit * T + tt];
    float kv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) kv[c] = ldx<F32IN>(s.k, o + j0 + c);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc = fmaf(wg[c], kv[c], acc);
    float cc, rs;
    ln_stats(qsum(acc), eps, slots, ctr, wv, l, cc, rs);
    const float yh = cc * rs;
    const float g = 2.f * gam * (ldx<F32IN>(s.k, o + i) + gam * yh + bet - ldx<F32IN>(s.v, o + i));
    float gm[2] = {g, g * yh};
    rows_sum<2>(gm, slots, ctr, wv, l);
    const float dy = rs * (g - gm[0] * (1.f / 64.f) - yh * gm[1] * (1.f / 64.f));
    acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      w[c] = fmaf(-eta * dy, kv[c], w[c]);
      acc = fmaf(w[c], ldx<F32IN>(s.q, o + j0 + c), acc);
    }
    float cq, rsq;
    ln_stats(qsum(acc), eps, slots, ctr, wv, l, cq, rsq);
    if (qd == 0) s.z[o + i] = ldx<F32IN>(s.q, o + i) + gam * cq * rsq + bet;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) s.w_out[(size_t)unit * 4096 + i * 64 + j0 + c] = w[c];
}

// Adjoint of yh = LNhat(y) given dyh and an extra adjoint drs0 of rs
// (per row i): returns dy.
__device__ __forceinline__ float ln_hat_adjoint(float c, float rs, float dyh, float drs0,
                                                float (*slots)[4][SLOTW], int& ctr, int wv,
                                                int l) {
  float s1[1] = {c * dyh};
  rows_sum<1>(s1, slots, ctr, wv, l);
  const float drs = drs0 + s1[0];
  const float dvar = -0.5f * rs * rs * rs * drs;
  const float dc = fmaf(2.f / 64.f * c, dvar, rs * dyh);
  float s2[1] = {dc};
  rows_sum<1>(s2, slots, ctr, wv, l);
  return dc - s2[0] * (1.f / 64.f);
}

template <bool F32IN>
__global__ void __launch_bounds__(NTHR) linear_ln_primal_bwd_kernel(LinearLnBwdArgs a) {
  __shared__ float slots[NSLOT][4][SLOTW];
  __shared__ float colp[2][4][129];  // column partials [parity][wave][dq | dk | -] and dr per row
  __shared__ float drow[2][64];       // dr of each row: the k_i term of dk

  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int qd = l >> 4, il = l & 15;
  const int i = 16 * wv + il, j0 = 16 * qd;
  const int unit = blockIdx.x, head = unit % a.H;
  const int T = a.T, b = a.b;
  const int nmb = (T + b - 1) / b;
  const float gam = a.gamma[head * 64 + i], bet = a.beta[head * 64 + i], eps = a.eps;
  const size_t base = (size_t)unit * T * 64;

  float w[16], wg[16], A[16], Ag[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    A[c] = a.dw_T ? a.dw_T[(size_t)unit * 4096 + i * 64 + j0 + c] : 0.f;
    Ag[c] = 0.f;
  }
  float dgam = 0.f, dbet = 0.f;
  int ctr = 0, n = 0;

  // the token's gradient quantities at the gradient point
  auto grad_point = [&](size_t o, const float (&kv)[16], float& cc, float& rs, float& yh, float& r,
                        float& g, float& gbar, float& m, float& dy) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc = fmaf(wg[c], kv[c], acc);
    ln_stats(qsum(acc), eps, slots, ctr, wv, l, cc, rs);
    yh = cc * rs;
    r = ldx<F32IN>(a.k, o + i) + gam * yh + bet - ldx<F32IN>(a.v, o + i);
    g = 2.f * gam * r;
    float gm[2] = {g, g * yh};
    rows_sum<2>(gm, slots, ctr, wv, l);
    gbar = gm[0] * (1.f / 64.f);
    m = gm[1] * (1.f / 64.f);
    dy = rs * (g - gbar - yh * m);
  };

  for (int mb = nmb - 1; mb >= 0; --mb) {
    const int m0 = mb * b, m1 = min(T, m0 + b);
    const float* ck = a.w_ckpt + ((size_t)unit * nmb + mb) * 4096;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      wg[c] = ck[i * 64 + j0 + c];
      w[c] = wg[c];
    }
    for (int tt = m0; tt < m1; ++tt) {  // replay to the mini-batch's end state
      const size_t o = base + (size_t)tt * 64;
      float kv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) kv[c] = ldx<F32IN>(a.k, o + j0 + c);
      float cc, rs, yh, r, g, gbar, m, dy;
      grad_point(o, kv, cc, rs, yh, r, g, gbar, m, dy);
      const float eta = a.eta[(size_t)unit * T + tt];
#pragma unroll
      for (int c = 0; c < 16; ++c) w[c] = fmaf(-eta * dy, kv[c], w[c]);
    }
    for (int tt = m1 - 1; tt >= m0; --tt, ++n) {
      const size_t o = base + (size_t)tt * 64;
      const float eta = a.eta[(size_t)unit * T + tt];
      float kv[16], qv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        kv[c] = ldx<F32IN>(a.k, o + j0 + c);
        qv[c] = ldx<F32IN>(a.q, o + j0 + c);
      }
      float cc, rs, yh, r, g, gbar, m, dy;
      grad_point(o, kv, cc, rs, yh, r, g, gbar, m, dy);
      // output z = q + gamma LNhat(W q) + beta, W the state after the token
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = fmaf(w[c], qv[c], acc);
      float cq, rsq;
      ln_stats(qsum(acc), eps, slots, ctr, wv, l, cq, rsq);
      const float dzi = a.dz[o + i];
      dgam = fmaf(cq * rsq, dzi, dgam);
      dbet += dzi;
      const float dyq = ln_hat_adjoint(cq, rsq, gam * dzi, 0.f, slots, ctr, wv, l);
      // dq: column sums of W^T dyq (plus the residual, added at the store)
      float dqm = 0.f, ak = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float rs16 = rowsum16(w[c] * dyq);
        if (il == c) dqm = rs16;
        A[c] = fmaf(dyq, qv[c], A[c]);
        ak = fmaf(A[c], kv[c], ak);
      }
      ak = qsum(ak);
      // the update W_after = W_before - eta dy k^T
      const float ddy = -eta * ak;
      // the LayerNorm VJP dy = rs (g - gbar - yh m): its three sums and deta
      float sv[4] = {ddy * (g - gbar - yh * m), ddy, ddy * yh, -dy * ak};
      rows_sum<4>(sv, slots, ctr, wv, l);
      const float drs = sv[0], dgbar = -rs * sv[1], dm = -rs * sv[2];
      const float dg = rs * ddy + dm * (1.f / 64.f) * yh + dgbar * (1.f / 64.f);
      float dyh = -rs * m * ddy + dm * (1.f / 64.f) * g;
      // g = 2 gamma r, r = k + gamma yh + beta - v
      const float dr = 2.f * gam * dg;
      dgam += 2.f * r * dg + yh * dr;
      dbet += dr;
      dyh = fmaf(gam, dr, dyh);
      if (qd == 0) a.dv[o + i] = -dr;
      const float dyv = ln_hat_adjoint(cc, rs, dyh, drs, slots, ctr, wv, l);
      // dk: column sums of -eta A^T dy + Wg^T dyv (the k_i term dr is added at the store)
      float dkm = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float rs16 = rowsum16(fmaf(-eta * A[c], dy, wg[c] * dyv));
        if (il == c) dkm = rs16;
        Ag[c] = fmaf(dyv, kv[c], Ag[c]);
        w[c] = fmaf(eta * dy, kv[c], w[c]);  // the state before the token
      }
      float* cp = colp[n & 1][wv];
      cp[j0 + il] = dqm;
      cp[64 + j0 + il] = dkm;
      if (qd == 0) drow[n & 1][i] = dr;
      if (tt == m0) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          A[c] += Ag[c];
          Ag[c] = 0.f;
        }
      }
      __syncthreads();
      if (t < 64) {
        const float* p4 = &colp[n & 1][0][0];
        a.dq[o + t] = a.dz[o + t] + p4[t] + p4[129 + t] + p4[258 + t] + p4[387 + t];
        a.dk[o + t] = drow[n & 1][t] + p4[64 + t] + p4[193 + t] + p4[322 + t] + p4[451 + t];
      } else if (t == 64) {
        a.deta[(size_t)unit * T + tt] = sv[3];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) a.dw0[(size_t)unit * 4096 + i * 64 + j0 + c] = A[c];
  if (qd == 0) {
    a.dgamma[(size_t)unit * 64 + i] = dgam;
    a.dbeta[(size_t)unit * 64 + i] = dbet;
  }
}

}  // namespace

hipError_t launch_linear_ln_primal(const LinearLnArgs& a, bool f32in, hipStream_t s) {
  const dim3 g(a.s.units), blk(NTHR);
  if (a.s.w_ckpt)
    return f32in ? launch(linear_ln_primal_fwd_kernel<true, true>, g, blk, s, a)
                 : launch(linear_ln_primal_fwd_kernel<false, true>, g, blk, s, a);
  return f32in ? launch(linear_ln_primal_fwd_kernel<true, false>, g, blk, s, a)
               : launch(linear_ln_primal_fwd_kernel<false, false>, g, blk, s, a);
}

hipError_t launch_linear_ln_primal_bwd(const LinearLnBwdArgs& a, bool f32in, hipStream_t s) {
  if (f32in) return launch(linear_ln_primal_bwd_kernel<true>, dim3(a.units), dim3(NTHR), s, a);
  return launch(linear_ln_primal_bwd_kernel<false>, dim3(a.units), dim3(NTHR), s, a);
}

}  // namespace ttt
