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
// With the LayerNorm + residual wrapper (§4.4), f(x) = x + LN(y) with
// y = W2 GELU(W1 x) and LN(y) = gamma (y - mean y) / sqrt(var y + eps) + beta
// over the 64 components: e = 2 (y - v) becomes the LayerNorm's VJP of
// g = 2 gamma (k + LN(y) - v), and the output is q + LN(W2_t GELU(W1_t q)).
// The 64 components of y live in wave 0, one per lane, so the LayerNorm's
// sums are wave reductions.
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

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_total(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
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

template <bool F32IN, bool LN>
__global__ void __launch_bounds__(PTHREADS) mlp_primal_kernel(MlpLnArgs la) {
  const MlpArgs& a = la.s;
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
  // LayerNorm (wave 0, lane = component): scale, shift, and the previous
  // token's q for its output
  float lg = 0.f, lb = 0.f, qprev = 0.f;
  if (LN && t < 64) {
    lg = la.gamma[(size_t)head * 64 + t];
    lb = la.beta[(size_t)head * 64 + t];
  }
  // (y - mean) / sqrt(var + eps) over the wave's 64 lanes (two passes); rs out
  auto lnhat = [&](float y, float& rs) {
    const float dev = y - wave_total(y) * (1.f / 64);
    rs = 1.f / sqrtf(wave_total(dev * dev) * (1.f / 64) + la.eps);
    return dev * rs;
  };
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
        if (a.w1_ckpt) {  // the state before mini-batch tt / b
          const size_t co = ((size_t)unit * ((T + b - 1) / b) + tt / b) * PHID * 64;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a.w1_ckpt[co + u * 64 + j0 + i] = w1[i];
            a.w2_ckpt[co + (j0 + i) * PHID + u] = w2[i];
          }
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
        if constexpr (LN) {
          // g = 2 gamma (k + gamma yhat + beta - v), then the LayerNorm VJP
          float rs;
          const float yh = lnhat(y, rs);
          const float gv = 2.f * lg * (kt[t] + lg * yh + lb - vt[t]);
          const float m1 = wave_total(gv) * (1.f / 64), m2 = wave_total(gv * yh) * (1.f / 64);
          ebuf[t] = rs * (gv - m1 - yh * m2);
        } else {
          ebuf[t] = 2.f * (y - vt[t]);
        }
        if (tt > 0) {
          float zs = 0.f;
#pragma unroll
          for (int w = 0; w < 16; ++w) zs += red[1][w][t];
          if constexpr (LN) {
            float rs;
            zs = qprev + lg * lnhat(zs, rs) + lb;
          }
          zu[(size_t)(tt - 1) * 64 + t] = zs;
        }
        if constexpr (LN) qprev = qt[t];
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
    if constexpr (LN) {
      float rs;
      zs = qprev + lg * lnhat(zs, rs) + lb;
    }
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

// ---------------------------------------------------------------------------
// Backward ("论文速览 | TTT" §6.12: the outer loop differentiates through the
// inner loop; the forward keeps the state at every mini-batch start).  The
// mini-batches are walked in reverse.  For mini-batch m the kernel loads its
// checkpoint (the gradient point of all its tokens), replays its tokens
// forward to the state at its end, then walks its tokens backwards; each step
// takes back its token's update exactly as the forward made it, to recover
// the state before the token.  Per token t (reverse), with A1, A2 the
// adjoints of the state after t and G1, G2 those of the gradient point:
//   output:  aq = W1 q, xq = GELU(aq), A2 += dz xq^T,
//            daq = (W2^T dz) * GELU'(aq), A1 += daq q^T, dq = W1^T daq;
//   update:  ddelta = -eta A1 k, dk = -eta A1^T delta, de = -eta A2 x,
//            dx = -eta A2^T e, deta = -delta^T A1 k - e^T A2 x;
//   delta = s * GELU'(a): ds = ddelta GELU'(a), da = ddelta s GELU''(a);
//   s = W2g^T e: G2 += e ds^T, de += W2g ds;
//   e = 2 (W2g x - v): dv = -2 de, G2 += 2 de x^T, dx += 2 W2g^T de;
//   x = GELU(a), a = W1g k: da += dx GELU'(a), G1 += da k^T, dk += W1g^T da;
//   at the mini-batch's first token: A += G, G = 0.
// Thread layout: 512 threads (8 waves); thread (wave v, lane l) owns hidden
// unit u = 32 v + (l % 32) and the half j in [32 hf, 32 hf + 32), hf = l / 32,
// of the 64 components, for the state, its adjoint and the gradient-point
// adjoint (96 registers); the gradient point sits in LDS, each thread's 64
// values in a private, bank-conflict-free slot.
constexpr int BTHREADS = 512;
constexpr int BSTRIDE = 4 * 64 + 1;  // floats per staged token: k, v, q, dz, eta

// Sum over the 32 lanes of a half wave (two DPP rows).
__device__ __forceinline__ float half_sum32(float v) { return row_sum16(v) + __shfl_xor(row_sum16(v), 16); }

template <bool F32IN>
__global__ void __launch_bounds__(BTHREADS) mlp_primal_bwd_kernel(MlpBwdArgs a) {
  __shared__ f32x4 wg1s[8][8][64];   // gradient point W1g[u][j0 + 4c + r] at [wave][c][lane]
  __shared__ f32x4 wg2s[8][8][64];   // W2g[j0 + 4c + r][u]
  __shared__ float tok[2][BSTRIDE];  // the current and the next step's token
  __shared__ float red_y[8][64], red_q[8][64], red_e[8][64], red_k[8][64];
  __shared__ float red_eta[8];
  __shared__ float ebuf[64], debuf[64];

  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  const int hf = l >> 5, ul = l & 31;
  const int u = 32 * wv + ul, j0 = 32 * hf;
  const int unit = blockIdx.x;
  const int T = a.T, b = a.b;
  const int nmb = (T + b - 1) / b;
  const int nsteps = 2 * T;
  const int llast = T - (nmb - 1) * b;  // tokens of the last mini-batch
  const size_t base = (size_t)unit * T * 64;
  const size_t nst = (size_t)PHID * 64;

  // step n of the walk: mini-batches from the last; in each, its tokens
  // forward (the replay), then backward
  auto step_token = [&](int n, bool& fwd, int& m) {
    int r;
    if (n < 2 * llast) {
      m = nmb - 1;
      r = n;
    } else {
      const int n2 = n - 2 * llast;
      m = nmb - 2 - n2 / (2 * b);
      r = n2 % (2 * b);
    }
    const int len = min(b, T - m * b);
    fwd = r < len;
    return m * b + (fwd ? r : 2 * len - 1 - r);
  };
  // element e of step n's staged token (threads e < BSTRIDE)
  auto token_value = [&](int n, int e) {
    bool fwd;
    int m;
    const int tt = step_token(n, fwd, m);
    const size_t o = base + (size_t)tt * 64;
    if (e < 64) return load_in<F32IN>(a.k, o + e);
    if (e < 128) return load_in<F32IN>(a.v, o + e - 64);
    if (e < 192) return load_in<F32IN>(a.q, o + e - 128);
    if (e < 256) return a.dz[o + e - 192];
    return a.eta[(size_t)unit * T + tt];
  };
  // the gradient point's values, read from LDS where they are used
  auto wg1 = [&](int i) { return wg1s[wv][i >> 2][l][i & 3]; };
  auto wg2 = [&](int i) { return wg2s[wv][i >> 2][l][i & 3]; };

  float w1[32], w2[32], a1[32], a2[32], g1[32], g2[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    a1[i] = a.dw1_T ? a.dw1_T[(size_t)unit * nst + u * 64 + j0 + i] : 0.f;
    a2[i] = a.dw2_T ? a.dw2_T[(size_t)unit * nst + (j0 + i) * PHID + u] : 0.f;
    g1[i] = 0.f;
    g2[i] = 0.f;
    w1[i] = 0.f;
    w2[i] = 0.f;
  }
  float pre = 0.f;  // step n + 1's staged value, held by thread t < BSTRIDE
  if (nsteps > 0 && t < BSTRIDE) {
    tok[0][t] = token_value(0, t);
    if (nsteps > 1) pre = token_value(1, t);
  }
  __syncthreads();

  int pend_t = -1;  // token whose dk partials wait in red_k
  for (int n = 0; n < nsteps; ++n) {
    bool fwd;
    int m;
    const int tt = step_token(n, fwd, m);
    const float* kt = tok[n & 1];
    const float* vt = kt + 64;
    const float* qt = kt + 128;
    const float* dzt = kt + 192;
    const float eta = kt[256];
    if (fwd && tt == m * b) {  // a mini-batch starts: its checkpoint
      const size_t co = ((size_t)unit * nmb + m) * nst;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f32x4 x1, x2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x1[r] = a.w1_ckpt[co + u * 64 + j0 + 4 * c + r];
          x2[r] = a.w2_ckpt[co + (j0 + 4 * c + r) * PHID + u];
          w1[4 * c + r] = x1[r];
          w2[4 * c + r] = x2[r];
        }
        wg1s[wv][c][l] = x1;
        wg2s[wv][c][l] = x2;
      }
    }
    // the token's forward quantities at the gradient point
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc = fmaf(wg1(i), kt[j0 + i], acc);
    const float av = acc + __shfl_xor(acc, 32);
    const float ph = gelu_phi(av);
    const float dens = expf(-0.5f * av * av) * 0.39894228040143268f;  // phi(a)
    const float x = av * ph;
    const float gp = fmaf(av, dens, ph);                  // GELU'(a)
    const float gpp = dens * (2.f - av * av);             // GELU''(a)
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float rs = half_sum32(wg2(i) * x);
      if (ul == i) mine = rs;
    }
    red_y[wv][j0 + ul] = mine;
    if (!fwd) {
      // output of token t from the state after it (w1, w2)
      acc = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(w1[i], qt[j0 + i], acc);
      const float aq = acc + __shfl_xor(acc, 32);
      const float phq = gelu_phi(aq);
      const float xq = aq * phq;
      const float gq = fmaf(aq, expf(-0.5f * aq * aq) * 0.39894228040143268f, phq);
      acc = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(w2[i], dzt[j0 + i], acc);
      const float daq = (acc + __shfl_xor(acc, 32)) * gq;
      mine = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        a2[i] = fmaf(dzt[j0 + i], xq, a2[i]);
        a1[i] = fmaf(daq, qt[j0 + i], a1[i]);
        const float rs = half_sum32(w1[i] * daq);
        if (ul == i) mine = rs;
      }
      red_q[wv][j0 + ul] = mine;
    }
    __syncthreads();  // B1
    if (n + 1 < nsteps && t < BSTRIDE) {
      tok[(n + 1) & 1][t] = pre;
      if (n + 2 < nsteps) pre = token_value(n + 2, t);
    }
    if (t < 64) {
      if (pend_t >= 0) {
        float sm = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sm += red_k[w][t];
        a.dk[base + (size_t)pend_t * 64 + t] = sm;
      }
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) y += red_y[w][t];
      ebuf[t] = 2.f * (y - vt[t]);
      if (!fwd) {
        float sm = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sm += red_q[w][t];
        a.dq[base + (size_t)tt * 64 + t] = sm;
      }
    }
    pend_t = -1;
    __syncthreads();  // B2
    acc = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc = fmaf(wg2(i), ebuf[j0 + i], acc);
    const float sv = acc + __shfl_xor(acc, 32);
    const float delta = sv * gp;
    if (fwd) {  // replay: the token's update
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        w2[i] = fmaf(-eta * ebuf[j0 + i], x, w2[i]);
        w1[i] = fmaf(-eta * delta, kt[j0 + i], w1[i]);
      }
      continue;
    }
    // adjoints through the update, then through the gradient
    float ak = 0.f, ae = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      ak = fmaf(a1[i], kt[j0 + i], ak);
      ae = fmaf(a2[i], ebuf[j0 + i], ae);
    }
    ak += __shfl_xor(ak, 32);
    ae += __shfl_xor(ae, 32);
    const float ddl = -eta * ak;
    float dx = -eta * ae;
    const float pe = half_sum32(hf == 0 ? -(delta * ak + x * ae) : 0.f);
    if (l == 0) red_eta[wv] = pe;
    const float ds = ddl * gp;
    float da = ddl * sv * gpp;
    mine = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      g2[i] = fmaf(ebuf[j0 + i], ds, g2[i]);
      const float rs = half_sum32(fmaf(-eta * a2[i], x, wg2(i) * ds));
      if (ul == i) mine = rs;
    }
    red_e[wv][j0 + ul] = mine;
    __syncthreads();  // B3
    if (t < 64) {
      float de = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) de += red_e[w][t];
      debuf[t] = de;
      a.dv[base + (size_t)tt * 64 + t] = -2.f * de;
      if (t == 0) {
        float sm = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sm += red_eta[w];
        a.deta[(size_t)unit * T + tt] = sm;
      }
    }
    __syncthreads();  // B4
    acc = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc = fmaf(wg2(i), debuf[j0 + i], acc);
    dx = fmaf(2.f, acc + __shfl_xor(acc, 32), dx);
    da = fmaf(dx, gp, da);
    mine = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      g2[i] = fmaf(2.f * debuf[j0 + i], x, g2[i]);
      g1[i] = fmaf(da, kt[j0 + i], g1[i]);
      const float rs = half_sum32(fmaf(-eta * a1[i], delta, wg1(i) * da));
      if (ul == i) mine = rs;
      // the state before token t
      w1[i] = fmaf(eta * delta, kt[j0 + i], w1[i]);
      w2[i] = fmaf(eta * ebuf[j0 + i], x, w2[i]);
    }
    red_k[wv][j0 + ul] = mine;
    pend_t = tt;
    if (tt == m * b) {  // the gradient point is the state before this token
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        a1[i] += g1[i];
        a2[i] += g2[i];
        g1[i] = 0.f;
        g2[i] = 0.f;
      }
    }
  }
  __syncthreads();
  if (t < 64 && pend_t >= 0) {
    float sm = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sm += red_k[w][t];
    a.dk[base + (size_t)pend_t * 64 + t] = sm;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    a.dw1_0[(size_t)unit * nst + u * 64 + j0 + i] = a1[i];
    a.dw2_0[(size_t)unit * nst + (j0 + i) * PHID + u] = a2[i];
  }
}

}  // namespace

hipError_t launch_mlp_bwd_primal(const MlpBwdArgs& a, bool f32in, hipStream_t s) {
  if (f32in) return launch(mlp_primal_bwd_kernel<true>, dim3(a.units), dim3(BTHREADS), s, a);
  return launch(mlp_primal_bwd_kernel<false>, dim3(a.units), dim3(BTHREADS), s, a);
}

hipError_t launch_mlp_primal(const MlpArgs& a, bool f32in, hipStream_t s) {
  const MlpLnArgs la{a, nullptr, nullptr, 0.f};
  if (f32in) return launch(mlp_primal_kernel<true, false>, dim3(a.units), dim3(PTHREADS), s, la);
  return launch(mlp_primal_kernel<false, false>, dim3(a.units), dim3(PTHREADS), s, la);
}

hipError_t launch_mlp_ln_primal(const MlpLnArgs& a, bool f32in, hipStream_t s) {
  if (f32in) return launch(mlp_primal_kernel<true, true>, dim3(a.s.units), dim3(PTHREADS), s, a);
  return launch(mlp_primal_kernel<false, true>, dim3(a.s.units), dim3(PTHREADS), s, a);
}

}  // namespace ttt
