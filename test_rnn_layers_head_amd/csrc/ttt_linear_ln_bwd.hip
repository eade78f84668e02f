// Backward of the TTT-Linear scan with the LayerNorm + residual inner model,
// in dual form: bf16 Q/K/V, b = 16, gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): f(x) = x + gamma LNhat(W x) + beta (§4.4), loss
// ||f(k) - v||^2 (§3.3) at the state before the mini-batch (§3.5),
// per-token eta (§4.6); the backward walks the mini-batches in reverse, each
// from its checkpoint (§6.12).  Per 16-token tile (columns are tokens,
// D = diag eta, Gn = -G the negative gradient, A = triu(K^T Q), sums and
// means over the 64 rows per token):
//   Y = W K, C = Y - mean Y, rs = (mean C^2 + eps)^-1/2, Yh = C rs,
//   R = K + gamma Yh + beta - V, Gh = 2 gamma R,
//   P = Gh - mean Gh - Yh mean(Gh Yh), GY = rs P, Gn = -GY D,
//   Zp = W Q + Gn A, Z = Q + gamma LNhat(Zp) + beta, W' = W + Gn K^T,
// and, given Zb = dL/dZ and the adjoint Wb' of W', every product taken back
// in reverse (the order of tests/dual_form.py: linear_ln_bwd_unit):
//   Zpb = LNhat'(gamma Zb),  Ab = triu(Gn^T Zpb),  Gnb = Zpb A^T + Wb' K,
//   GYb = -Gnb D,  deta = -sum_i Gnb GY,
//   Pb = rs GYb, rsb = sum_i GYb P,  Ghb, Yhb from P's means,
//   Rb = 2 gamma Ghb,  Yhb += gamma Rb,  Yb = LNhat'(Yhb) (with rsb),
//   dQ = Zb + W^T Zpb + K Ab,  dK = Q Ab^T + Wb'^T Gn + Rb + W^T Yb,
//   dV = -Rb,  Wb = Wb' + Zpb Q^T + Yb K^T,
//   dgamma += sum_t (Zb LNhat(Zp) + 2 R Ghb + Yh Rb),  dbeta += sum_t (Zb + Rb),
// where LNhat'(H) = C' - mean C', C' = rs H + (2/64) C varb,
// varb = -rs^3 (rsb0 + sum_i C H) / 2 is LNhat's adjoint.
//
// Work split: one workgroup of four waves per (batch, head) unit; wave w
// owns column block j in [16 w, 16 w + 16) of the state and of its adjoint,
// kept as W[i][j] at [16 w + 4g + r][16 ib + c] (rows j; all 64 rows i).
// Tiles are "transposed" (tokens on the accumulator rows): lane (c, g)
// register r holds X[token 4g + r][16 ib + c] for the four row blocks ib.
// The three contractions over j (Y = W K, W Q and Wb' K) leave per-wave
// partials in LDS, summed in a fixed order after one barrier; everything
// else over the 64 rows is repeated in every wave, so each LayerNorm sum is
// four in-lane adds and a DPP row sum; the contractions over i (dQ, dK's
// terms) and the adjoint's update need only the wave's own column block, from
// the transposed blocks (an MFMA against the identity, exact for the hi + lo
// halves).  The checkpoint's column block of each tile is read from HBM; K,
// Q, V, dZ and eta arrive by LDS DMA one tile ahead.  Two barriers per tile.
//
// Precision: fp32 factors enter the bf16 MFMA as hi + lo halves, three
// products kept (~2^-16 relative per product); K, Q, V are exact bf16; the
// LayerNorm statistics use the one-pass variance E[Y^2] - mean^2 (clamped
// at 0), as the forward scan does.
#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_mlp_ops.h"

namespace ttt {
namespace {

typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

// one staged tile: K, Q (swizzled), V, dZ (fp32), eta
constexpr int T_K = 0, T_Q = 2048, T_V = 4096, T_DZ = 6144, T_ETA = 10240;
constexpr int RAWB = T_ETA + 64;
// per-wave partials of the contractions over j: [set][wave][ib][lane] f32x4,
// sets Y = W K, W Q, Wb' K
constexpr int L_PART = 2 * RAWB;
constexpr int L_TOTAL = L_PART + 3 * 4 * 4 * 1024;

// [x0 x1 x2 x3 x0 x1 x2 x3]: the bf16 rows 4g .. 4g + 3 of column col of a
// swizzled tile, seen by both the hi and the lo slots of the other operand
__device__ __forceinline__ bf16x8 rows_twice(const char* tile, int g, int col) {
  short x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = *(const short*)(tile + swz_chunk(4 * g + r, col >> 3) + (col & 7) * 2);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {x[0], x[1], x[2], x[3], x[0], x[1], x[2], x[3]};
  return __builtin_bit_cast(bf16x8, v);
}
// Operand over the 64 rows i from two column blocks (2 kb, 2 kb + 1) of a
// transposed tile: lane (c, g) slot 8g + e holds X[token c][32 kb + 16 (e/4)
// + 4g + e % 4] - an A operand over (token, i) or a B operand over (i, token).
__device__ __forceinline__ Split8 i_operand(f32x4 x0, f32x4 x1, bf16x8 itr, const NegSel& ns) {
  return split8_mfma(transpose16(x0, itr), transpose16(x1, itr), ns);
}

// PAD: b < 16, each b-token mini-batch alone in a tile whose rows b..15 read
// as zero tokens (eta = 0: they change neither the state nor the other
// tokens' outputs) and drop their outputs (token T: past every descriptor).
template <bool PAD>
__global__ void __launch_bounds__(256) linear_ln_bwd_kernel(LinearLnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[L_TOTAL];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int bt = PAD ? a.b : 16;  // tokens per tile
  const int ntiles = PAD ? (T + bt - 1) / bt : (T + 15) >> 4;
  auto tk = [&](int j, int r) {
    if constexpr (PAD)
      return r < bt ? j * bt + r : T;
    else
      return 16 * j + r;
  };
  const float eps = a.eps;

  bf16x8 itr, negI;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    itr[e] = (bf16)((4 * g + (e & 3) == c) ? 1.f : 0.f);
    negI[e] = (bf16)((g < 2 && 8 * g + e == c) ? -1.f : 0.f);
  }
  const NegSel ns = make_negsel(c, g);
  float gam[4], bet[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    gam[ib] = a.gamma[head * 64 + 16 * ib + c];
    bet[ib] = a.beta[head * 64 + 16 * ib + c];
  }

  // per-token sums over the 64 rows (every lane of row group g gets those of
  // tokens 4g .. 4g + 3)
  auto tsum = [&](const f32x4* x) {
    f32x4 s;
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = row_sum16((x[0][r] + x[1][r]) + (x[2][r] + x[3][r]));
    return s;
  };
  auto tdot = [&](const f32x4* x, const f32x4* y) {
    f32x4 s;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s[r] = row_sum16(fmaf(x[0][r], y[0][r], x[1][r] * y[1][r]) + fmaf(x[2][r], y[2][r], x[3][r] * y[3][r]));
    return s;
  };

  // this wave's column block of the state's adjoint, W[i][j] at [16 w + 4g + r][16 ib + c]
  f32x4 Wb[4];
  {
    const float* d0 = a.dw_T ? a.dw_T + (size_t)unit * 4096 : nullptr;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
      Wb[ib] = d0 ? *(const f32x4*)(d0 + (16 * ib + c) * 64 + 16 * w + 4 * g) : f32x4{0, 0, 0, 0};
  }
  auto part_at = [&](int set, int v, int ib) {
    return (f32x4*)(smem + L_PART + ((set * 4 + v) * 4 + ib) * 1024 + lane * 16);
  };
  f32x4 dgam = {0, 0, 0, 0}, dbet = {0, 0, 0, 0};  // [ib]: partial sums over this lane's tokens

  // ------------------------------------------------------- input staging
  const size_t uoff = (size_t)unit * T * 64;
  // Tile j is loaded into registers one tile ahead and written to slot
  // j & 1 at the end of the tile before it (register staging: the compiler
  // then waits for exactly these loads, and only where they are written).
  // Wave 0 loads K (and eta), wave 1 Q, wave 2 V, wave 3 dZ, with the same
  // instructions: four 1 KB pieces, those a wave does not need aimed past its
  // buffer's end (the hardware returns zeros without a memory access), so no
  // loaded register is merged across branches.  K and Q rows get chunk p of
  // row r at position p ^ (r & 7), linear in the staged tile.
  const char* const src = w == 0 ? (const char*)a.k : w == 1 ? (const char*)a.q
                        : w == 2 ? (const char*)a.v : (const char*)a.dz;
  const uint32_t srow = w == 3 ? 256u : 128u;  // bytes per token
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(src + uoff / 64 * srow, (uint32_t)T * srow);
  const __amdgpu_buffer_rsrc_t reta = make_rsrc(a.eta + (size_t)unit * T, w == 0 ? (uint32_t)T * 4 : 0u);
  const int npiece = w == 3 ? 4 : 2;
  uint32_t pofs[4];  // piece n's offset within the tile (PAD: within its token row)
  int prow[4];       // PAD: the token row of piece n
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 8 * n + (lane >> 3), kp = lane & 7;
    pofs[n] = w < 2 ? (uint32_t)(r * 128 + ((kp ^ (r & 7)) << 4)) : (uint32_t)(n * 1024 + lane * 16);
    prow[n] = w == 3 ? 4 * n + (lane >> 4) : r;
    if constexpr (PAD) pofs[n] = w < 2 ? (uint32_t)((kp ^ (r & 7)) << 4) : (uint32_t)((lane * 16) % srow);
  }
  uint4v pf[4];
  float pfe;
  auto fetch = [&](int j) {
    const uint32_t tb = (uint32_t)j * 16 * srow;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t off = PAD ? (uint32_t)tk(j, prow[n]) * srow + pofs[n] : tb + pofs[n];
      pf[n] = __builtin_amdgcn_raw_buffer_load_b128(rin, n < npiece ? off : 0x80000000u, 0, 0);
    }
    pfe = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(reta, (uint32_t)tk(j, lane & 15) * 4, 0, 0));
  };
  auto stash = [&](int j) {
    char* dst = smem + (j & 1) * RAWB + w * 2048 + lane * 16;  // T_K, T_Q, T_V, T_DZ = 2048 w
#pragma unroll
    for (int n = 0; n < 4; ++n)
      if (n < npiece) *(uint4v*)(dst + n * 1024) = pf[n];
    if (w == 0 && lane < 16) *(float*)(smem + (j & 1) * RAWB + T_ETA + lane * 4) = pfe;
  };
  const __amdgpu_buffer_rsrc_t oq = make_rsrc(a.dq + uoff, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t ok = make_rsrc(a.dk + uoff, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t ov = make_rsrc(a.dv + uoff, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t odeta = make_rsrc(a.deta + (size_t)unit * T, (uint32_t)T * 4);
  // lane (c, g) stores [row 4g + r of tile j][col]; stores past T fall outside
  auto store_tile = [&](__amdgpu_buffer_rsrc_t r, int j, int col, f32x4 x) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[k]), r,
                                            (uint32_t)((tk(j, 4 * g + k) * 64 + col) * 4), 0, 0);
  };

  // this wave's column block of the checkpoint of tile t
  auto load_w = [&](int t, f32x4* x) {
    const float* wc = a.w_ckpt + ((size_t)unit * ntiles + t) * 4096;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) x[ib] = *(const f32x4*)(wc + (16 * ib + c) * 64 + 16 * w + 4 * g);
  };
  f32x4 W[4], Wn[4];
  if (ntiles > 0) {
    load_w(ntiles - 1, W);
    fetch(ntiles - 1);
    stash(ntiles - 1);
  }
  wg_barrier();

  for (int j = ntiles - 1; j >= 0; --j) {
    const char* raw = smem + (j & 1) * RAWB;
    const char* Kt = raw + T_K;
    const char* Qt = raw + T_Q;
    const char* Vt = raw + T_V;
    const float* dZt = (const float*)(raw + T_DZ);
    const f32x4 eta4 = *(const f32x4*)(raw + T_ETA + 16 * g);

    // the next tile's checkpoint block and inputs, into registers
    if (j > 0) {
      load_w(j - 1, Wn);
      fetch(j - 1);
    }

    // K, Q rows as A operands over j: slots 8g + e of half h are columns
    // 32 h + 16 (e/4) + 4g + e % 4 (two 8-byte reads)
    auto rowop = [&](const char* tile, int h) {
      const uint2 lo = *(const uint2*)(tile + swz_chunk(c, 4 * h + (g >> 1)) + (g & 1) * 8);
      const uint2 hi = *(const uint2*)(tile + swz_chunk(c, 4 * h + 2 + (g >> 1)) + (g & 1) * 8);
      return cat8(lo, hi);
    };
    bf16x8 kop[2], qop[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kop[h] = rowop(Kt, h);
      qop[h] = rowop(Qt, h);
    }
    f32x4 Am = {0, 0, 0, 0}, AmT = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Am = mfma_k32(kop[h], qop[h], Am);    // [s = 4g + r][t = c] = sum_j K[s][j] Q[t][j]
      AmT = mfma_k32(qop[h], kop[h], AmT);  // [t = 4g + r][s = c]
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * g + r > c) Am[r] = 0.f;
      if (c > 4 * g + r) AmT[r] = 0.f;
    }
    const Split4 ams = split4(Am), amts = split4(AmT);
    const bf16x8 aop = cat44(ams.hi, ams.lo);    // A = Am^T: rows t, slots s
    const bf16x8 aTop = cat44(amts.hi, amts.lo); // A = Am: rows s, slots t

    // ============================================== forward of the tile
    // partials over this wave's 16 columns j of W K, W Q and Wb' K: A = the
    // K / Q row's 4 columns 16 w + 4g .. + 3 twice, B = [hi | lo] of the block
    {
      const int kcol = swz_chunk(c, 2 * w + (g >> 1)) + (g & 1) * 8;
      const uint2 kx = *(const uint2*)(Kt + kcol), qx = *(const uint2*)(Qt + kcol);
      const bf16x8 kw = cat8(kx, kx), qw = cat8(qx, qx);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const Split4 ws = split4(W[ib]), bs = split4(Wb[ib]);
        const bf16x8 wop = cat44(ws.hi, ws.lo), bop = cat44(bs.hi, bs.lo);
        *part_at(0, w, ib) = mfma_k32(kw, wop, f32x4{0, 0, 0, 0});
        *part_at(1, w, ib) = mfma_k32(qw, wop, f32x4{0, 0, 0, 0});
        *part_at(2, w, ib) = mfma_k32(kw, bop, f32x4{0, 0, 0, 0});
      }
    }
    wg_barrier();  // the partials of the three contractions over j
    f32x4 Y[4], Zp[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 y = {0, 0, 0, 0}, zq = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        y += *part_at(0, v, ib);
        zq += *part_at(1, v, ib);
      }
      Y[ib] = y;
      Zp[ib] = zq;  // W Q; the Gn A term is added below
    }
    f32x4 mu, rs;
    {
      const f32x4 s1 = tsum(Y), s2 = tdot(Y, Y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mu[r] = s1[r] * (1.f / 64);
        rs[r] = rsqrtf(fmaxf(fmaf(s2[r], 1.f / 64, -mu[r] * mu[r]), 0.f) + eps);
      }
    }
    f32x4 C[4], R[4], GY[4], Gn[4];  // Y - mean, K + gamma Yh + beta - V, rs P, -eta rs P
    f32x4 gbar, m;
    {
      f32x4 Gh[4], Yh[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 kv = mfma_k32(*(const bf16x8*)(Kt + swz_chunk(c, 2 * ib + (g & 1))), negI, f32x4{0, 0, 0, 0});
#pragma unroll
        for (int r = 0; r < 4; ++r) kv[r] = -kv[r];
        kv = mfma_k32(*(const bf16x8*)(Vt + c * 128 + (16 * ib + 8 * (g & 1)) * 2), negI, kv);  // K - V
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          C[ib][r] = Y[ib][r] - mu[r];
          Yh[ib][r] = C[ib][r] * rs[r];
          R[ib][r] = kv[r] + fmaf(gam[ib], Yh[ib][r], bet[ib]);
          Gh[ib][r] = 2.f * gam[ib] * R[ib][r];
        }
      }
      const f32x4 sg = tsum(Gh), sgy = tdot(Gh, Yh);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gbar[r] = sg[r] * (1.f / 64);
        m[r] = sgy[r] * (1.f / 64);
      }
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          GY[ib][r] = rs[r] * (Gh[ib][r] - gbar[r] - Yh[ib][r] * m[r]);
          Gn[ib][r] = -eta4[r] * GY[ib][r];
        }
    }
    // Zp = W Q + Gn A, its statistics and normalised form
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) Zp[ib] = mm_pre(aop, yops(split4(Gn[ib])), Zp[ib]);
    f32x4 rsq;
    {
      const f32x4 s1 = tsum(Zp), s2 = tdot(Zp, Zp);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mq = s1[r] * (1.f / 64);
        rsq[r] = rsqrtf(fmaxf(fmaf(s2[r], 1.f / 64, -mq * mq), 0.f) + eps);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) Zp[ib][r] -= mq;  // Zp now holds Zp - mean
      }
    }

    // ============================================== the output's adjoint
    f32x4 Zb[4], Zpb[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) Zb[ib][r] = dZt[(4 * g + r) * 64 + 16 * ib + c];
    {
      f32x4 Hb[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dgam[ib] = fmaf(Zb[ib][r], Zp[ib][r] * rsq[r], dgam[ib]);
          dbet[ib] += Zb[ib][r];
          Hb[ib][r] = gam[ib] * Zb[ib][r];
        }
      // LNhat's adjoint: C' = rsq Hb + (2/64) Cq varb, Zpb = C' - mean C'
      const f32x4 sch = tdot(Zp, Hb);
      f32x4 vq;
#pragma unroll
      for (int r = 0; r < 4; ++r) vq[r] = (2.f / 64) * (-0.5f * rsq[r] * rsq[r] * rsq[r] * sch[r]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Zpb[ib][r] = fmaf(rsq[r], Hb[ib][r], Zp[ib][r] * vq[r]);
      const f32x4 sc = tsum(Zpb);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Zpb[ib][r] -= sc[r] * (1.f / 64);
    }
    Split4 zpbs[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) zpbs[ib] = split4(Zpb[ib]);

    // Gnb^T[s][i] = sum_t Am[s][t] Zpb^T[t][i] + sum_j K[s][j] Wb'[i][j] (the partials)
    f32x4 Gnb[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; ++v) acc += *part_at(2, v, ib);
      Gnb[ib] = mm_pre(aTop, yops(zpbs[ib]), acc);
    }

    // ============================================== the gradient's adjoint
    f32x4 Rb[4], Yb[4];
    {
      f32x4 Pb[4], Yh[4];
      f32x4 de, rsb, spb, spy;
      {
        f32x4 gyb[4], P[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gyb[ib][r] = -eta4[r] * Gnb[ib][r];
            Yh[ib][r] = C[ib][r] * rs[r];
            P[ib][r] = fmaf(-Yh[ib][r], m[r], fmaf(2.f * gam[ib], R[ib][r], -gbar[r]));  // GY = rs P
            Pb[ib][r] = rs[r] * gyb[ib][r];
          }
        de = tdot(Gnb, GY);
        rsb = tdot(gyb, P);
        spb = tsum(Pb);
        spy = tdot(Pb, Yh);
      }
      if (w == 0 && c == 0) {  // tokens past T fall outside the descriptor
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-de[r]), odeta,
                                                (uint32_t)tk(j, 4 * g + r) * 4, 0, 0);
      }
      f32x4 Yhb[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ghb = Pb[ib][r] - spb[r] * (1.f / 64) - Yh[ib][r] * spy[r] * (1.f / 64);
          const float gh = 2.f * gam[ib] * R[ib][r];
          const float yhb = -Pb[ib][r] * m[r] - gh * spy[r] * (1.f / 64);
          const float rb = 2.f * gam[ib] * ghb;
          dgam[ib] = fmaf(2.f * R[ib][r], ghb, fmaf(Yh[ib][r], rb, dgam[ib]));
          dbet[ib] += rb;
          Rb[ib][r] = rb;
          Yhb[ib][r] = fmaf(gam[ib], rb, yhb);
        }
      // Yb = LNhat'(Yhb) with the extra adjoint rsb of rs
      const f32x4 scy = tdot(C, Yhb);
      f32x4 vy;
#pragma unroll
      for (int r = 0; r < 4; ++r) vy[r] = (2.f / 64) * (-0.5f * rs[r] * rs[r] * rs[r] * (rsb[r] + scy[r]));
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Yb[ib][r] = fmaf(rs[r], Yhb[ib][r], C[ib][r] * vy[r]);
      const f32x4 sc = tsum(Yb);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Yb[ib][r] -= sc[r] * (1.f / 64);
    }

    // Ab [s][t] = triu(sum_i Gn[i][s] Zpb[i][t]) and its transpose
    Split8 gno[2], zpbo[2], ybo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      gno[kb] = i_operand(Gn[2 * kb], Gn[2 * kb + 1], itr, ns);
      zpbo[kb] = i_operand(Zpb[2 * kb], Zpb[2 * kb + 1], itr, ns);
      ybo[kb] = i_operand(Yb[2 * kb], Yb[2 * kb + 1], itr, ns);
    }
    f32x4 Ab = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ab = mm3(gno[kb], zpbo[kb], Ab);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > c) Ab[r] = 0.f;
    const Split4 abs_ = split4(Ab), abts = split4(transpose16(Ab, itr));
    const bf16x8 abop = cat44(abs_.hi, abs_.lo);     // A = Ab^T: rows t, slots s
    const bf16x8 abTop = cat44(abts.hi, abts.lo);   // A = Ab: rows s, slots t

    // ============================================== dQ, dK, dV of column block w
    {
      // the residual's dz and dk's direct Rb of column block w (selects, no indexing)
      f32x4 dq = Zb[0], dk = Rb[0];
#pragma unroll
      for (int jb = 1; jb < 4; ++jb)
        if (w == jb) {
          dq = Zb[jb];
          dk = Rb[jb];
        }
      f32x4 dv;
#pragma unroll
      for (int r = 0; r < 4; ++r) dv[r] = -dk[r];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // W and Wb' with i on the rows (transposed blocks)
        const Split8 w2 = split8_mfma(transpose16(W[2 * kb], itr), transpose16(W[2 * kb + 1], itr), ns);
        const Split8 b2 = split8_mfma(transpose16(Wb[2 * kb], itr), transpose16(Wb[2 * kb + 1], itr), ns);
        dq = mm3(zpbo[kb], w2, dq);  // W^T Zpb
        dk = mm3(ybo[kb], w2, dk);   // W^T Yb
        dk = mm3(gno[kb], b2, dk);   // Wb'^T Gn
      }
      dq = mfma_k32(abop, rows_twice(Kt, g, 16 * w + c), dq);   // + K Ab
      dk = mfma_k32(abTop, rows_twice(Qt, g, 16 * w + c), dk);  // + Q Ab^T
      store_tile(oq, j, 16 * w + c, dq);
      store_tile(ok, j, 16 * w + c, dk);
      store_tile(ov, j, 16 * w + c, dv);
    }

    // ============================================== Wb = Wb' + Zpb Q^T + Yb K^T
    Split4 ybs[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) ybs[ib] = split4(Yb[ib]);
    {
      const bf16x8 qj = rows_twice(Qt, g, 16 * w + c), kj = rows_twice(Kt, g, 16 * w + c);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        Wb[ib] = mfma_k32(qj, cat44(zpbs[ib].hi, zpbs[ib].lo), Wb[ib]);
        Wb[ib] = mfma_k32(kj, cat44(ybs[ib].hi, ybs[ib].lo), Wb[ib]);
      }
    }
    if (j > 0) stash(j - 1);  // into the slot tile j + 1 used
    wg_barrier();             // the next tile's inputs; the partial areas free again
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) W[ib] = Wn[ib];
  }

  // the adjoint of the initial state and of the LayerNorm parameters
  float* d0 = a.dw0 + (size_t)unit * 4096;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) *(f32x4*)(d0 + (16 * ib + c) * 64 + 16 * w + 4 * g) = Wb[ib];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    float sg = dgam[ib], sb = dbet[ib];
    sg += __shfl_xor(sg, 16);
    sg += __shfl_xor(sg, 32);
    sb += __shfl_xor(sb, 16);
    sb += __shfl_xor(sb, 32);
    if (w == 0 && g == 0) {
      a.dgamma[(size_t)unit * 64 + 16 * ib + c] = sg;
      a.dbeta[(size_t)unit * 64 + 16 * ib + c] = sb;
    }
  }
}

}  // namespace

hipError_t launch_linear_ln_bwd(const LinearLnBwdArgs& a, bool f32in, hipStream_t s) {
  if (f32in || a.b > 16) return launch_linear_ln_primal_bwd(a, f32in, s);
  if (a.b < 16) return launch(linear_ln_bwd_kernel<true>, dim3(a.units), dim3(256), s, a);
  return launch(linear_ln_bwd_kernel<false>, dim3(a.units), dim3(256), s, a);
}

}  // namespace ttt
