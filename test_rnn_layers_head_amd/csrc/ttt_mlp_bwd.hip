// Backward of the TTT-MLP scan in dual form, bf16 Q/K/V, b | 16, gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): the outer loop differentiates through the inner
// one (§6.12); the forward keeps the state at the start of every
// mini-batch, and the backward walks the mini-batches in reverse, each from
// its checkpoint.  Per 16-token tile (columns are tokens, D = diag eta,
// Gn = -G the negative gradients, GELU' and GELU'' of Z1 written P1, P2):
//   Z1 = W1 K, X2 = GELU(Z1), Y = W2 X2, E = Y - V, Gn2 = -2 E D,
//   Sn = W2^T Gn2, Gn1 = Sn * P1, A = triu(K^T Q), Z1q = W1 Q + Gn1 A,
//   X2q = GELU(Z1q), B2 = triu(X2^T X2q), Z = W2 X2q + Gn2 B2,
//   W1' = W1 + Gn1 K^T, W2' = W2 + Gn2 X2^T            (§3.7 dual form)
// and, given Zb = dL/dZ and the adjoints A1', A2' of W1', W2', every
// product taken back in reverse (the order of tests/dual_form.py):
//   Mb = triu(Gn2^T Zb),  X2qb = W2^T Zb + X2 Mb,  Z1qb = X2qb * GELU'(Z1q),
//   Gn1b = A1' K + Z1qb A^T,  Ab = triu(Gn1^T Z1qb),
//   Snb = Gn1b * P1,  Z1b = Gn1b * Sn * P2,
//   Gn2b = Zb B2^T + A2' X2 + W2 Snb,  Yb = -2 Gn2b D,  dV = -Yb,
//   deta_t = -2 sum_i Gn2b[i,t] E[i,t],
//   X2b = X2q Mb^T + A2'^T Gn2 + W2^T Yb,  Z1b += X2b * P1,
//   dQ = W1^T Z1qb + K Ab,  dK = A1'^T Gn1 + Q Ab^T + W1^T Z1b,
//   A1 = A1' + Z1qb Q^T + Z1b K^T,  A2 = A2' + Zb X2q^T + Gn2 Snb^T + Yb X2^T.
// A mini-batch of b < 16 tokens takes a tile of its own whose rows b..15
// read as zero tokens (eta = 0: they change neither the state nor the other
// tokens' outputs) and drop their outputs.
//
// Work split: one workgroup of 8 waves per (batch, head) unit; wave w owns
// the hidden units u in [32 w, 32 w + 32) (two 16-blocks): its rows of W1 and
// A1 and its columns of W2 and A2, the adjoints resident in registers for
// the whole sequence.  Products over the hidden units (Y, the Gn2 adjoint,
// dQ, dK, B2, Ab) leave per-wave partials in LDS that the first four waves
// (one 16-column block of d each) or every wave (16 x 16) sum in a fixed
// order; dK's partials reuse each wave's W2N area once its last read of the
// tile is done.  Tokens sit on the accumulator rows ("transposed" tiles, X^T[t][.]).
//
// Layouts per wave (lane c + 16 g, register r; u0 = 32 w):
//   W1, A1   [n][m]: [u0 + 16 n + c][sigma(m, 4g + r)], sigma(m, 4g + r) =
//            32 (m/2) + 8 g + 4 (m%2) + r: the K reduction slots of W1 K
//            are 8 consecutive columns, one 16-byte chunk of a K row;
//   W2, A2   [nu][mi]: W2[16 mi + c][u0 + 16 nu + 4g + r] (u on the rows);
//   W2N      [mi][nu]: W2[16 mi + 4g + r][u0 + 16 nu + c] (i on the rows),
//            loaded from the checkpoint into the wave's own LDS area;
//   W1T      [nu][m]: W1[u0 + 16 nu + 4g + r][sigma(m, c)], loaded late;
//   A1T, A2N the same transposes of the resident adjoints, formed per tile
//            by an MFMA against the identity (exact for the hi + lo halves).
// dQ and dK are formed with their columns in the sigma order of W1, and
// stored there.
//
// Precision: every fp32 factor enters the bf16 MFMA as hi + lo halves, three
// products kept (~2^-16 relative per product); K, Q, V are exact bf16.
#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_mlp_ops.h"

namespace ttt {
namespace {

constexpr int BWV = 8;                  // waves
constexpr int BHID = 256;               // hidden units
// one staged tile: K (swizzled), Q (swizzled), V, dZ (fp32), eta
constexpr int T_K = 0, T_Q = 2048, T_V = 4096, T_DZ = 6144, T_ETA = 10240;
constexpr int RAWB = T_ETA + 64;
// LDS map (bytes)
constexpr int L_RAW = 0;                          // 2 tile slots
constexpr int L_P = L_RAW + 2 * RAWB;             // [wave][blk][lane] f32x4 d-space partials
constexpr int L_SB = L_P + BWV * 4 * 1024;        // [wave][lane] f32x4 B2^T partials
constexpr int L_SA = L_SB + BWV * 1024;           // [wave][lane] f32x4 Ab partials
constexpr int L_G2A = L_SA + BWV * 1024;          // [mi][lane] hi|lo of Gn2^T (t x i)
constexpr int L_G2B = L_G2A + 4 * 1024;           // [mi][lane] hi|lo of Gn2 (i x t)
constexpr int L_YBA = L_G2B + 4 * 1024;           // [mi][lane] hi|lo of Yb^T
constexpr int L_YBB = L_YBA + 4 * 1024;           // [mi][lane] hi|lo of Yb
constexpr int L_ETA = L_YBB + 4 * 1024;           // [mi][16] deta partial sums
constexpr int L_W2N = L_ETA + 256;                // [wave][mi][nu][lane] f32x4
constexpr int L_TOTAL = L_W2N + BWV * 8 * 1024;
static_assert(L_TOTAL <= 160 * 1024, "LDS budget");

// Operand over the wave's 32 hidden units from the splits of two
// accumulator tiles X[n] (rows tokens, columns u0 + 16 n + c): lane (c, g)
// slot 8g + e holds X[token c][u0 + 16 (e/4) + 4g + e%4], an A operand over
// (token, u) or a B operand over (u, token).
__device__ __forceinline__ Split8 u_operand(const Split4& x0, const Split4& x1, bf16x8 itr,
                                            const NegSel& ns) {
  const f32x4 t0 = mfma_k32(cat44(x0.hi, x0.lo), itr, f32x4{0, 0, 0, 0});
  const f32x4 t1 = mfma_k32(cat44(x1.hi, x1.lo), itr, f32x4{0, 0, 0, 0});
  return split8_mfma(t0, t1, ns);
}
// GELU, GELU' and GELU'' = phi(x) (2 - x^2) at one point
struct Gelu3 {
  float g, dg, ddg;
};
__device__ __forceinline__ Gelu3 gelu3(float x) {
  const GeluOut o = gelu_and_grad(x);
  const float phi = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f) * 0.39894228040143268f;
  return Gelu3{o.g, o.dg, phi * (2.f - x * x)};
}
// bf16 element (row r, column i) of a swizzled K / Q tile
__device__ __forceinline__ short tile_elem(const char* tile, int r, int i) {
  return *(const short*)(tile + swz_chunk(r, i >> 3) + (i & 7) * 2);
}
// [x0 x1 x2 x3 x0 x1 x2 x3]: a B operand whose hi and lo slots see the same
// exact bf16 rows 4g .. 4g + 3 (column col) of a swizzled tile
__device__ __forceinline__ bf16x8 rows_twice(const char* tile, int g, int col) {
  const short x0 = tile_elem(tile, 4 * g, col), x1 = tile_elem(tile, 4 * g + 1, col);
  const short x2 = tile_elem(tile, 4 * g + 2, col), x3 = tile_elem(tile, 4 * g + 3, col);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {x0, x1, x2, x3, x0, x1, x2, x3};
  return __builtin_bit_cast(bf16x8, v);
}

template <bool PAD>  // PAD: b < 16, one mini-batch per tile
__global__ void __launch_bounds__(BWV * 64) mlp_bwd_kernel(MlpBwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[L_TOTAL];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  if (unit >= a.units) return;
  const int T = a.T;
  // tokens per tile: 16, or b < 16 with each mini-batch alone in a tile
  // whose rows b..15 read as zero tokens (eta = 0: they change nothing) and
  // drop their outputs (token T: just past every descriptor)
  const int bt = PAD ? a.b : 16;
  const int ntiles = PAD ? (T + bt - 1) / bt : (T + 15) >> 4;
  auto tk = [&](int j, int r) {
    if constexpr (PAD)
      return r < bt ? j * bt + r : T;
    else
      return 16 * j + r;
  };
  const int u0 = 32 * w;
  const size_t nst = (size_t)BHID * 64;

  // ------------------------------------------------------------ constants
  bf16x8 sel[2], itr, negI;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sel[0][e] = (bf16)((g == (c >> 2) && e == (c & 3)) ? 1.f : 0.f);
    sel[1][e] = (bf16)((g == (c >> 2) && e == 4 + (c & 3)) ? 1.f : 0.f);
    itr[e] = (bf16)((4 * g + (e & 3) == c) ? 1.f : 0.f);
    negI[e] = (bf16)((g < 2 && 8 * g + e == c) ? -1.f : 0.f);
  }
  const NegSel ns = make_negsel(c, g);
  // sigma(m, c): the column of W1 that lane column c stands for in block m
  auto sigc = [&](int m) { return 32 * (m >> 1) + 8 * (c >> 2) + 4 * (m & 1) + (c & 3); };

  // ---------------------------------------------------- adjoints of the state
  f32x4 A1[2][4], A2[2][4];
  {
    const float* d1 = a.dw1_T ? a.dw1_T + (size_t)unit * nst : nullptr;
    const float* d2 = a.dw2_T ? a.dw2_T + (size_t)unit * nst : nullptr;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        A1[n][m] = d1 ? *(const f32x4*)(d1 + (u0 + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1))
                      : f32x4{0, 0, 0, 0};
        A2[n][m] = d2 ? *(const f32x4*)(d2 + (16 * m + c) * BHID + u0 + 16 * n + 4 * g)
                      : f32x4{0, 0, 0, 0};
      }
  }

  // ------------------------------------------------------- input staging
  // Tile j goes into slot j & 1 by LDS DMA, one 1 KiB block per wave and
  // instruction: waves 0..5 the two halves of K, Q, V (K, Q with chunk p of
  // row r at position p ^ (r & 7), set by the source addresses), waves 6, 7
  // two blocks of dZ each, wave 0 also eta.  Loads past T return zeros.
  const size_t uoff = (size_t)unit * T * 64;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const __amdgpu_buffer_rsrc_t rin =
      wu < 2 ? make_rsrc((const short*)a.k + uoff, (uint32_t)T * 128)
             : (wu < 4 ? make_rsrc((const short*)a.q + uoff, (uint32_t)T * 128)
                       : (wu < 6 ? make_rsrc((const short*)a.v + uoff, (uint32_t)T * 128)
                                 : make_rsrc(a.dz + uoff, (uint32_t)T * 256)));
  const __amdgpu_buffer_rsrc_t reta = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
  auto issue = [&](int j) {
    char* slot = smem + L_RAW + (j & 1) * RAWB;
    if (wu < 6) {
      const int n = wu & 1, r = 8 * n + (lane >> 3), kp = lane & 7;
      const uint32_t tb = (uint32_t)j * 2048;
      const uint32_t off = PAD ? (uint32_t)tk(j, r) * 128 + ((wu < 4 ? kp ^ (r & 7) : kp) << 4)
                               : (wu < 4 ? tb + r * 128 + ((kp ^ (r & 7)) << 4) : tb + n * 1024 + lane * 16);
      dma16(rin, slot + (wu >> 1) * 2048 + n * 1024, off);
    } else {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int blk = 2 * (wu - 6) + n;
        dma16(rin, slot + T_DZ + blk * 1024,
              PAD ? (uint32_t)tk(j, 4 * blk + (lane >> 4)) * 256 + (lane & 15) * 16
                  : (uint32_t)j * 4096 + blk * 1024 + lane * 16);
      }
    }
    if (wu == 0 && lane < 16) dma4(reta, slot + T_ETA, (uint32_t)tk(j, lane) * 4);
  };

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.dq + uoff, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.dk + uoff, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.dv + uoff, (uint32_t)T * 256);
  // store of a d-space tile: lane (c, g) holds [token 4g + r][column col]
  auto store_tile = [&](__amdgpu_buffer_rsrc_t r, int j, int col, f32x4 x) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[k]), r,
                                            (uint32_t)((tk(j, 4 * g + k) * 64 + col) * 4), 0, 0);
  };

  char* const w2n = smem + L_W2N + w * 8192 + lane * 16;
  auto w2n_at = [&](int mi, int nu) { return (f32x4*)(w2n + (mi * 2 + nu) * 1024); };
  auto part_at = [&](int v, int blk) { return (f32x4*)(smem + L_P + (v * 4 + blk) * 1024 + lane * 16); };
  // dK partials of wave v, block m: the first 4 KiB of the wave's W2N area
  auto dk_at = [&](int v, int m) { return (f32x4*)(smem + L_W2N + v * 8192 + m * 1024 + lane * 16); };

  if (ntiles > 0) issue(ntiles - 1);
  wait_vmcnt<0>();
  wg_barrier();

  for (int j = ntiles - 1; j >= 0; --j) {
    const char* raw = smem + L_RAW + (j & 1) * RAWB;
    const char* Kt = raw + T_K;
    const char* Qt = raw + T_Q;
    const char* Vt = raw + T_V;
    const float* dZt = (const float*)(raw + T_DZ);
    const float* Et = (const float*)(raw + T_ETA);

    // ------------------------------------------------ checkpoint of tile j
    const size_t co = ((size_t)unit * ntiles + j) * nst;
    const float* w1c = a.w1_ckpt + co;
    const float* w2c = a.w2_ckpt + co;
    // W2 with u on the rows, block (nu, mi), and W1 with u on the rows and
    // columns sigma(m, c), block (nu, m): read where they are used
    auto w2t = [&](int nu, int mi) { return *(const f32x4*)(w2c + (16 * mi + c) * BHID + u0 + 16 * nu + 4 * g); };
    auto w2t_op = [&](int mi) { return split8_mfma(w2t(0, mi), w2t(1, mi), ns); };
    // W1^T block (nu, m) = the transpose of W1's block (nu, m): rows u, columns
    // sigma(m, c) - the hi + lo halves of W1, which split again into the same halves
    auto w1blk = [&](int n, int m) {
      return *(const f32x4*)(w1c + (u0 + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1));
    };
    auto w1t_op = [&](int m) {
      return split8_mfma(transpose16(w1blk(0, m), itr), transpose16(w1blk(1, m), itr), ns);
    };
    // W2N = the transposes of the W2^T blocks (their hi + lo halves, which
    // split again into the same halves as W2 itself)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int nu = 0; nu < 2; ++nu) *w2n_at(mi, nu) = transpose16(w2t(nu, mi), itr);  // this wave only
    auto w2n_op = [&](int kb, int nu) { return split8_mfma(*w2n_at(2 * kb, nu), *w2n_at(2 * kb + 1, nu), ns); };

    // ------------------------------------------- per-tile K, Q operands
    bf16x8 kop[2], qop[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kop[h] = row_chunk(Kt, c, h, g);
      qop[h] = row_chunk(Qt, c, h, g);
    }
    f32x4 Am = {0, 0, 0, 0}, AmT = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Am = mfma_k32(kop[h], qop[h], Am);    // [s = 4g + r][t = c] = sum_i K[s][i] Q[t][i]
      AmT = mfma_k32(qop[h], kop[h], AmT);  // [t = 4g + r][s = c]
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * g + r > c) Am[r] = 0.f;
      if (c > 4 * g + r) AmT[r] = 0.f;
    }
    const Split4 ams = split4(Am), amts = split4(AmT);
    const bf16x8 aop = cat44(ams.hi, ams.lo);    // A = Am^T (rows t, slots s)
    const bf16x8 aTop = cat44(amts.hi, amts.lo); // A = Am (rows s, slots t)
    const f32x4 eta4 = *(const f32x4*)(Et + 4 * g);
    // the next tile's inputs, into the slot tile j + 1 used: issued after the
    // tile's first LDS reads, since the compiler makes the next LDS read wait
    // for every DMA in flight
    __builtin_amdgcn_sched_barrier(0);
    if (j > 0) issue(j - 1);
    f32x4 e2;
#pragma unroll
    for (int r = 0; r < 4; ++r) e2[r] = 2.f * eta4[r];

    // ================================== forward of the tile at its checkpoint
    f32x4 ZQ[2], D[2], Z1bp[2];
    Split4 x2ts[2];
    {
      f32x4 X2t[2], D2[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const Split8 s0 = split8_mfma(w1blk(n, 0), w1blk(n, 1), ns), s1 = split8_mfma(w1blk(n, 2), w1blk(n, 3), ns);
        f32x4 z = {0, 0, 0, 0}, zq = {0, 0, 0, 0};
        z = mfma_k32(kop[0], s0.hi, z);
        z = mfma_k32(kop[0], s0.lo, z);
        z = mfma_k32(kop[1], s1.hi, z);
        z = mfma_k32(kop[1], s1.lo, z);
        zq = mfma_k32(qop[0], s0.hi, zq);
        zq = mfma_k32(qop[0], s0.lo, zq);
        zq = mfma_k32(qop[1], s1.hi, zq);
        zq = mfma_k32(qop[1], s1.lo, zq);
        ZQ[n] = zq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const Gelu3 o = gelu3(z[r]);
          X2t[n][r] = o.g;   // X2^T[t][u]
          D[n][r] = o.dg;
          D2[n][r] = o.ddg;
        }
        x2ts[n] = split4(X2t[n]);
      }
      Z1bp[0] = D2[0];  // GELU'' kept until the adjoint of GELU' is known
      Z1bp[1] = D2[1];
    }
    const Split8 x2o = u_operand(x2ts[0], x2ts[1], itr, ns);
    // Y partial over this wave's units: [t][i] per block mi
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      *part_at(w, mi) = mm3(x2o, w2t_op(mi), f32x4{0, 0, 0, 0});
    wg_barrier();  // B1: Y partials

    // ================================== E, Gn2 (block mi = w)
    f32x4 Eb = {0, 0, 0, 0};
    if (w < 4) {
      const int mi = w;
      f32x4 Y = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < BWV; ++v) Y += *part_at(v, mi);
      Eb = mfma_k32(*(const bf16x8*)(Vt + c * 128 + (16 * mi + 8 * (g & 1)) * 2), negI, Y);  // Y - V
      f32x4 Gv;
#pragma unroll
      for (int r = 0; r < 4; ++r) Gv[r] = -e2[r] * Eb[r];
      const Split4 gs = split4(Gv);
      *(uint4*)(smem + L_G2A + mi * 1024 + lane * 16) = pack_split(gs);
      const f32x4 GT = mfma_k32(cat44(gs.hi, gs.lo), itr, f32x4{0, 0, 0, 0});  // Gn2[i][t]
      *(uint4*)(smem + L_G2B + mi * 1024 + lane * 16) = pack_split(split4(GT));
    }
    wg_barrier();  // B2: Gn2

    // Gn2^T as A operand over i (rows t): ga[kb] covers i in [32 kb, 32 kb + 32)
    auto load_ga = [&](int area, Split8* out) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Split4 t0 = unpack_split(*(const uint4*)(smem + area + (2 * kb) * 1024 + lane * 16));
        const Split4 t1 = unpack_split(*(const uint4*)(smem + area + (2 * kb + 1) * 1024 + lane * 16));
        out[kb] = Split8{cat44(t0.hi, t1.hi), cat44(t0.lo, t1.lo)};
      }
    };
    // dZ of the tile, as an operand over i with the token on the lane column:
    // lane (c, g) slot 8g + e holds dZ[token c][32 kb + 16 (e/4) + 4g + e%4]
    Split8 dzb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      dzb[kb] = split8(*(const f32x4*)(dZt + c * 64 + 32 * kb + 4 * g),
                       *(const f32x4*)(dZt + c * 64 + 32 * kb + 16 + 4 * g));
    // dZ^T block mi in accumulator layout: [token 4g + r][16 mi + c]
    auto dz_acc = [&](int mi) {
      f32x4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = dZt[(4 * g + r) * 64 + 16 * mi + c];
      return x;
    };

    // ================================== Sn, Gn1, Z1q, X2q; Mb; adjoints in u
    Split4 g1s[2], x2qs[2], z1qbs[2], snbs[2];
    f32x4 Sn[2], Dq[2], Gn1b[2];
    Split8 x2qo;
    bf16x8 mbop, mbtop;
    {
      Split8 ga[2];
      load_ga(L_G2B, ga);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mm3(ga[kb], w2n_op(kb, n), acc);
        Sn[n] = acc;
        f32x4 g1;
#pragma unroll
        for (int r = 0; r < 4; ++r) g1[r] = acc[r] * D[n][r];
        g1s[n] = split4(g1);
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const f32x4 z1q = mm_pre(aop, yops(g1s[n]), ZQ[n]);
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const GeluOut o = gelu_and_grad(z1q[r]);
          x[r] = o.g;
          Dq[n][r] = o.dg;
        }
        x2qs[n] = split4(x);
      }
      x2qo = u_operand(x2qs[0], x2qs[1], itr, ns);
      // B2^T partial: [t][s] = sum_u X2q[u][t] X2[u][s]
      *(f32x4*)(smem + L_SB + w * 1024 + lane * 16) = mm3(x2qo, x2o, f32x4{0, 0, 0, 0});
      // Mb [s][t] = triu(Gn2^T Zb) and its transpose [t][s]
      f32x4 Mb = {0, 0, 0, 0}, MbT = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Mb = mm3(ga[kb], dzb[kb], Mb);
        MbT = mm3(dzb[kb], ga[kb], MbT);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r > c) Mb[r] = 0.f;
        if (c > 4 * g + r) MbT[r] = 0.f;
      }
      const Split4 mbs = split4(Mb), mbts = split4(MbT);
      mbop = cat44(mbs.hi, mbs.lo);     // A = Mb^T (rows t, slots s)
      mbtop = cat44(mbts.hi, mbts.lo);  // A = Mb (rows s, slots t)
      // X2qb^T[t][u] = sum_i Zb^T[t][i] W2[i][u] + sum_s Mb[s][t] X2^T[s][u]; Z1qb; Gn1b
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mm3(dzb[kb], w2n_op(kb, n), acc);
        acc = mm_pre(mbop, yops(x2ts[n]), acc);
        f32x4 z1qb;
#pragma unroll
        for (int r = 0; r < 4; ++r) z1qb[r] = acc[r] * Dq[n][r];
        z1qbs[n] = split4(z1qb);
        // Gn1b^T[s][u] = sum_i K[s][i] A1[u][i] + sum_t Am[s][t] Z1qb^T[t][u]
        const Split8 s0 = split8_mfma(A1[n][0], A1[n][1], ns), s1 = split8_mfma(A1[n][2], A1[n][3], ns);
        f32x4 gb = {0, 0, 0, 0};
        const bf16x8 k0 = row_chunk(Kt, c, 0, g), k1 = row_chunk(Kt, c, 1, g);  // re-read
        gb = mfma_k32(k0, s0.hi, gb);
        gb = mfma_k32(k0, s0.lo, gb);
        gb = mfma_k32(k1, s1.hi, gb);
        gb = mfma_k32(k1, s1.lo, gb);
        Gn1b[n] = mm_pre(aTop, yops(z1qbs[n]), gb);
      }
    }
    // Snb = Gn1b * P1, Z1b (part) = Gn1b * Sn * P2
    Split8 g1o;
    {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 snb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          snb[r] = Gn1b[n][r] * D[n][r];
          Z1bp[n][r] = Gn1b[n][r] * Sn[n][r] * Z1bp[n][r];
        }
        snbs[n] = split4(snb);
      }
      g1o = u_operand(g1s[0], g1s[1], itr, ns);
      const Split8 z1qbo = u_operand(z1qbs[0], z1qbs[1], itr, ns);
      const Split8 snbo = u_operand(snbs[0], snbs[1], itr, ns);
      // Ab partial: [s][t] = sum_u Gn1[u][s] Z1qb[u][t]
      *(f32x4*)(smem + L_SA + w * 1024 + lane * 16) = mm3(g1o, z1qbo, f32x4{0, 0, 0, 0});
      // Gn2b^T partial: [s][i] = sum_u X2^T[s][u] A2[i][u] + Snb^T[s][u] W2[i][u]
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        f32x4 acc = mm3(x2o, split8_mfma(A2[0][mi], A2[1][mi], ns), f32x4{0, 0, 0, 0});
        *part_at(w, mi) = mm3(snbo, w2t_op(mi), acc);
      }
    }
    wg_barrier();  // B3: Gn2b, B2^T and Ab partials

    // Ab [s][t] (every wave) and its transpose
    f32x4 Ab = {0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < BWV; ++v) Ab += *(const f32x4*)(smem + L_SA + v * 1024 + lane * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > c) Ab[r] = 0.f;
    const f32x4 AbT = transpose16(Ab, itr);
    // ================================== Gn2b, Yb, dV, deta (block mi = w)
    if (w < 4) {
      const int mi = w;
      f32x4 B2T = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < BWV; ++v) B2T += *(const f32x4*)(smem + L_SB + v * 1024 + lane * 16);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (c > 4 * g + r) B2T[r] = 0.f;
      const Split4 b2s = split4(B2T);
      f32x4 G2b = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < BWV; ++v) G2b += *part_at(v, mi);
      G2b = mm_pre(cat44(b2s.hi, b2s.lo), yops(split4(dz_acc(mi))), G2b);  // + B2 Zb^T
      f32x4 Yb, dv, ep;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Yb[r] = -e2[r] * G2b[r];
        dv[r] = -Yb[r];
        ep[r] = row_sum16(G2b[r] * Eb[r]);
      }
      if (tk(j, 4 * g) < T) store_tile(rv, j, 16 * mi + c, dv);
      if (c == 0) *(f32x4*)(smem + L_ETA + (mi * 16 + 4 * g) * 4) = ep;
      const Split4 ys = split4(Yb);
      *(uint4*)(smem + L_YBA + mi * 1024 + lane * 16) = pack_split(ys);
      const f32x4 YT = mfma_k32(cat44(ys.hi, ys.lo), itr, f32x4{0, 0, 0, 0});
      *(uint4*)(smem + L_YBB + mi * 1024 + lane * 16) = pack_split(split4(YT));
    }
    wg_barrier();  // B4: Yb

    if (w == 4 && lane < 16 && tk(j, lane) < T) {
      float s = 0.f;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) s += *(const float*)(smem + L_ETA + (mi * 16 + lane) * 4);
      a.deta[(size_t)unit * T + tk(j, lane)] = -2.f * s;
    }
    // ================================== X2b, Z1b
    {
      Split8 z1bo;
      Split8 ga[2], yba[2];
      load_ga(L_G2B, ga);
      load_ga(L_YBB, yba);
      Split4 z1bs[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 acc = mm_pre(mbtop, yops(x2qs[n]), f32x4{0, 0, 0, 0});  // X2q Mb^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // A2 with i on the rows (the W2N layout), transposed from the resident layout
          acc = mm3(ga[kb], split8_mfma(transpose16(A2[n][2 * kb], itr), transpose16(A2[n][2 * kb + 1], itr), ns), acc);
          acc = mm3(yba[kb], w2n_op(kb, n), acc);
        }
        f32x4 z1b;
#pragma unroll
        for (int r = 0; r < 4; ++r) z1b[r] = fmaf(acc[r], D[n][r], Z1bp[n][r]);
        z1bs[n] = split4(z1b);
      }
      z1bo = u_operand(z1bs[0], z1bs[1], itr, ns);
      // dQ partial: [t][sigma(m, c)] = sum_u Z1qb^T[t][u] W1[u][sigma]
      {
        const Split8 z1qbo = u_operand(z1qbs[0], z1qbs[1], itr, ns);
#pragma unroll
        for (int m = 0; m < 4; ++m) *part_at(w, m) = mm3(z1qbo, w1t_op(m), f32x4{0, 0, 0, 0});
      }
      // dK partial: [s][sigma] = sum_u Gn1^T[s][u] A1[u][sigma] + Z1b^T[s][u] W1[u][sigma],
      // into this wave's W2N area (its last read was X2b above)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 a1t0 = transpose16(A1[0][m], itr), a1t1 = transpose16(A1[1][m], itr);
        f32x4 acc = mm3(g1o, split8_mfma(a1t0, a1t1, ns), f32x4{0, 0, 0, 0});
        *dk_at(w, m) = mm3(z1bo, w1t_op(m), acc);
      }
      wg_barrier();  // B5: dQ and dK partials
      if (w < 4) {
        const int m = w;
        f32x4 dq = {0, 0, 0, 0}, dk = {0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < BWV; ++v) {
          dq += *part_at(v, m);
          dk += *dk_at(v, m);
        }
        const Split4 abs_ = split4(Ab), abts = split4(AbT);
        dq = mfma_k32(cat44(abs_.hi, abs_.lo), rows_twice(Kt, g, sigc(m)), dq);   // + K Ab
        dk = mfma_k32(cat44(abts.hi, abts.lo), rows_twice(Qt, g, sigc(m)), dk);  // + Q Ab^T
        if (tk(j, 4 * g) < T) {
          store_tile(rq, j, sigc(m), dq);
          store_tile(rk, j, sigc(m), dk);
        }
      }
      // ============================== adjoint updates
      // A1 += Z1qb Q^T + Z1b K^T (accumulator [sigma][u])
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 xq = mfma_k32(row_chunk(Qt, c, m >> 1, g), sel[m & 1], f32x4{0, 0, 0, 0});  // Q[t][sigma(m, c)]
        const f32x4 xk = mfma_k32(row_chunk(Kt, c, m >> 1, g), sel[m & 1], f32x4{0, 0, 0, 0});
        const uint32_t q0 = pack_rne(xq[0], xq[1]), q1 = pack_rne(xq[2], xq[3]);
        const uint32_t k0 = pack_rne(xk[0], xk[1]), k1 = pack_rne(xk[2], xk[3]);
        const bf16x8 qt2 = __builtin_bit_cast(bf16x8, make_uint4(q0, q1, q0, q1));
        const bf16x8 kt2 = __builtin_bit_cast(bf16x8, make_uint4(k0, k1, k0, k1));
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          A1[n][m] = mfma_k32(qt2, cat44(z1qbs[n].hi, z1qbs[n].lo), A1[n][m]);
          A1[n][m] = mfma_k32(kt2, cat44(z1bs[n].hi, z1bs[n].lo), A1[n][m]);
        }
      }
    }
    // A2 += Zb X2q^T + Gn2 Snb^T + Yb X2^T (accumulator [u][i])
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const YOps zy = yops(split4(dz_acc(mi)));
      const YOps gy = yops(unpack_split(*(const uint4*)(smem + L_G2A + mi * 1024 + lane * 16)));
      const YOps yy = yops(unpack_split(*(const uint4*)(smem + L_YBA + mi * 1024 + lane * 16)));
#pragma unroll
      for (int nu = 0; nu < 2; ++nu) {
        f32x4 acc = A2[nu][mi];
        acc = mm_pre(cat44(x2qs[nu].hi, x2qs[nu].lo), zy, acc);
        acc = mm_pre(cat44(snbs[nu].hi, snbs[nu].lo), gy, acc);
        acc = mm_pre(cat44(x2ts[nu].hi, x2ts[nu].lo), yy, acc);
        A2[nu][mi] = acc;
      }
    }

    wait_vmcnt<0>();  // the next tile's inputs have landed
    wg_barrier();     // B0: the next tile's inputs; partial areas free
  }

  // the adjoint of the initial state
  float* d1 = a.dw1_0 + (size_t)unit * nst;
  float* d2 = a.dw2_0 + (size_t)unit * nst;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      *(f32x4*)(d1 + (u0 + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) = A1[n][m];
      *(f32x4*)(d2 + (16 * m + c) * BHID + u0 + 16 * n + 4 * g) = A2[n][m];
    }
}

}  // namespace

hipError_t launch_mlp_bwd(const MlpBwdArgs& a, bool f32in, hipStream_t s) {
  if (f32in || a.b > 16) return launch_mlp_bwd_primal(a, f32in, s);
  if (a.b < 16) return launch(mlp_bwd_kernel<true>, dim3(a.units), dim3(BWV * 64), s, a);
  return launch(mlp_bwd_kernel<false>, dim3(a.units), dim3(BWV * 64), s, a);
}

}  // namespace ttt
