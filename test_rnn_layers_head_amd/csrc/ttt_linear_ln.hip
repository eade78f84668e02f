// TTT-Linear with the LayerNorm + residual inner model, bf16 Q/K/V, gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): the inner model of §4.4 wrapped in a LayerNorm and
// a residual, f(x) = x + LN(W x), LN(y) = gamma (y - mean y) / sqrt(var y +
// eps) + beta over the d = 64 output components of one token; trained by
// mini-batch GD with every gradient of a mini-batch taken at the state W0
// before it (§3.5), per-token eta (§4.6), loss ||f(k) - v||^2 (§3.3), and the
// output read from the updated state (§3.1).  Per 16-token tile (columns are
// tokens, U = K + beta - V):
//   Y = W0 K,  rs = 1 / sqrt(var + eps),  Yhat = (Y - mu) rs
//   g = 2 gamma (U + gamma Yhat)                   (dl / dYhat)
//   dY = rs (g - mean(g) - Yhat mean(g Yhat))     (LayerNorm VJP)
//   Gn = -dY diag(eta),  W <- W0 + Gn K^T
//   z = q + LN(W0 Q + Gn triu(K^T Q))              (dual form, §3.6)
// mean, var and the two means of the VJP are sums over the 64 rows of W.
//
// Workgroup = one (batch, head) unit, all 64 rows of W:
//   waves 0..3  compute waves, 16 rows each, W resident in accumulators;
//   waves 4, 5  helpers: per-tile operands that depend only on K, Q, eta
//               (triu(K^T Q), K_{j-1}^T K_j, 2 eta, the update operand), two
//               tiles ahead, into a three-slot "prepared" LDS area;
//   wave 6      loader: buffer->LDS DMA of K/Q/V/eta tiles into a ring.
// One workgroup barrier per tile.  Before barrier j+1 every compute wave
// leaves in LDS its partial sums over its 16 rows of the statistics of tile
// j+1 (of Y_{j+1} = W0 K_{j+1}) and of the outputs of tile j; after it, every
// wave finishes the reduction and computes the gradient of tile j+1 and the
// outputs of tile j.  The output normalisation thus runs one tile behind the
// recurrence and off its serial chain; the normalised outputs pass through
// an LDS staging tile, from which helpers 1 and 2 store whole 256-byte rows
// one tile later.
//
// Layouts.  The statistics and the gradient are formed transposed ("layout
// T": lane (c, g) register r holds row 4g+r of the wave's 16 rows for token
// c), where a token's sums over rows are in-lane adds plus two cross-lane
// steps (permlane32/permlane16 swaps) and all per-token scalars are per lane.
// The rank-16 update needs the gradient with tokens in the MFMA reduction
// slots ("layout A": lane (c, g) register r holds row c, token 4g+r).  The
// bf16 hi and lo halves of the layout-T gradient are carried over to layout A
// exactly by two MFMAs against one-hot selections.
//
// The lookahead of the plain scan carries over (Y is linear in W):
//   Y_{j+1} = W_j K_{j+1} + Gn_j (K_j^T K_{j+1})
// so W_j K_{j+1} is formed from the split of W_j before Gn_j is known.
//
// Precision: K, Q, V are exact bf16; every sum and scalar is fp32.  fp32
// operands enter bf16 MFMA as sums of bf16 terms.  The LayerNorm makes the
// recurrence more sensitive to rounding than the plain scan (its loss is
// blind to a common shift of W's rows and, up to eps, to W's scale, so
// errors along those directions are never pulled back), so the products that
// carry the recurrence take their fp32 factor in three terms (~2^-24
// relative): W in W K, the gradient in the update W += Gn K^T, and both
// factors of the lookahead correction Gn (K^T K).  The outputs W Q and
// Gn triu(K^T Q) use two (~2^-16).  The variance
// uses the one-pass form E[y^2] - mu^2 (clamped at 0).
#include <type_traits>

#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_linear_ops.h"

namespace ttt {
namespace {

struct LnGeom {
  static constexpr int NCW = 4;                 // compute waves
  static constexpr int KB = 16 * 64 * 2;        // K or Q tile (bf16)
  static constexpr int VB = 16 * 64 * 2;        // V tile
  static constexpr int RAW = 2 * KB + VB + 64;  // + eta (16 fp32)
  static constexpr int NI = 4 + 2 + 1;          // DMA ops per tile
  static constexpr int D = 9;                   // loader lookahead (D - 1 tiles in flight)
  static constexpr int NST = D + 3;             // raw ring slots
  static constexpr int P_NE = 0;                // -eta_t, 16 fp32
  static constexpr int P_SGU = 64;              // sums of gamma (k + beta - v) over rows 0..31,
  static constexpr int P_SGU2 = 128;            //   and over rows 32..63, 16 fp32 each
  static constexpr int P_A = 192;               // triu(K^T Q), hi | lo
  static constexpr int P_MKK = P_A + 1024;      // K_{j-1}^T K_j, hi | mid
  static constexpr int P_MKL = P_MKK + 1024;    // K_{j-1}^T K_j, lo (8 bytes per lane)
  static constexpr int P_KT = P_MKL + 512;      // update operand, x4
  static constexpr int P_GU = P_KT + 4096;      // 2 gamma (k + beta - v), layout T, x4 waves
  static constexpr int P_QB = P_GU + 4096;      // q + beta, layout T, x4 waves
  static constexpr int PREP = P_QB + 4096;
  static constexpr int NPREP = 4;
  static constexpr int XST = 8 * 16 * 4;        // floats: [stat 8][token 16][wave 4]
  static constexpr int ZROW = 68 * 4;           // bytes per token of a Z staging tile (64 + 4 pad)
  static constexpr int ZT = 16 * ZROW;          // one Z staging tile (16 tokens)
  static constexpr int LDS = NST * RAW + NPREP * PREP + 2 * XST * 4 + 2 * ZT;
  // waves 0..3 compute, 4 and 5 helpers, 6 loader, 7 helper: wave i shares
  // a SIMD with wave i + 4, so every SIMD holds one compute wave and one
  // wave of preparation work
  static constexpr int W_H0 = 4, W_H1 = 5, W_LOAD = 6, W_H2 = 7;
  static constexpr int THREADS = 8 * 64;
};
static_assert(63 / LnGeom::NI >= LnGeom::D, "DMA lookahead exceeds the vmcnt range");
static_assert(LnGeom::NPREP == 4, "prepared slots are indexed with a mask");

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float x) { return __builtin_bit_cast(uint32_t, x); }

// [p summed over lanes l and l^32 on lanes 0..31 | q summed likewise on 32..63]
__device__ __forceinline__ float fold32(float p, float q) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(p), f_bits(q), false, false);
  return bits_f(r[0]) + bits_f(r[1]);
}
// Rows (16 lanes) 0..3 of the result: p0 + p1, q0 + q1, p2 + p3, q2 + q3,
// where pi / qi are rows of p / q.
__device__ __forceinline__ float fold16(float p, float q) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(p), f_bits(q), false, false);
  return bits_f(r[0]) + bits_f(r[1]);
}
// x has row i = value X_i (16-lane rows); returns {X_0, X_1} broadcast to
// every row for x = [X_0, X_1, X_0, X_1], i.e. after a 32-lane swap.
__device__ __forceinline__ void bcast16(float x, float& x0, float& x1) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x0 = bits_f(r[0]);
  x1 = bits_f(r[1]);
}
__device__ __forceinline__ void bcast32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  lo = bits_f(r[0]);
  hi = bits_f(r[1]);
}

// Three-term bf16 split of two accumulator blocks, x = hi + mid + lo with
// |x - hi - mid - lo| <~ 2^-25 |x|: the residuals x - hi and x - hi - mid are
// formed exactly on the matrix unit (one-hot -I times the bf16 term, added to
// the fp32 value), as in split8_mfma.
struct Split8x3 {
  bf16x8 hi, mid, lo;
};
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_rne(a[0], a[1]), pack_rne(a[2], a[3]),
                                               pack_rne(b[0], b[1]), pack_rne(b[2], b[3])));
}
__device__ __forceinline__ Split8x3 split8x3(f32x4 a, f32x4 b, const NegSel& ns) {
  Split8x3 s;
  s.hi = pack8(a, b);
  const f32x4 ra = mfma_k32(ns.s0, s.hi, a), rb = mfma_k32(ns.s1, s.hi, b);
  s.mid = pack8(ra, rb);
  const f32x4 sa = mfma_k32(ns.s0, s.mid, ra), sb = mfma_k32(ns.s1, s.mid, rb);
  s.lo = pack8(sa, sb);
  return s;
}
// The same for one accumulator block, on the vector unit.
struct Split4x3 {
  s16x4 hi, mid, lo;
};
__device__ __forceinline__ Split4x3 split4x3(f32x4 x) {
  Split4x3 s;
  f32x4 r = x;
  uint2 p[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    p[k] = make_uint2(pack_rne(r[0], r[1]), pack_rne(r[2], r[3]));
    r[0] -= __builtin_bit_cast(float, p[k].x << 16);
    r[1] -= __builtin_bit_cast(float, p[k].x & 0xffff0000u);
    r[2] -= __builtin_bit_cast(float, p[k].y << 16);
    r[3] -= __builtin_bit_cast(float, p[k].y & 0xffff0000u);
  }
  s.hi = u2s(p[0]);
  s.mid = u2s(p[1]);
  s.lo = u2s(p[2]);
  return s;
}

// four bf16 (two packed words) -> fp32
__device__ __forceinline__ f32x4 bf4(uint2 u) {
  return f32x4{bits_f(u.x << 16), bits_f(u.x & 0xffff0000u), bits_f(u.y << 16),
               bits_f(u.y & 0xffff0000u)};
}

// TPM: tiles per mini-batch when fixed at compile time (b = 16, 32, 64),
// 0 = read from the arguments (other multiples of 16).  CKPT: also store
// the state before every mini-batch (the checkpoints the backward reads),
// straight from the compute waves' accumulators.
// PAD (b < 16, TPM = 1): each b-token mini-batch takes a tile of its own whose
// rows b..15 read as zero tokens (eta = 0: they change neither the state nor
// the other tokens' outputs) and drop their outputs (token T: past every
// descriptor): the b = 16 arithmetic at 16 / b times the tiles.
template <int TPM, bool CKPT = false, bool PAD = false>
__global__ void __launch_bounds__(LnGeom::THREADS) linear_ln_scan_kernel(LinearLnArgs la) {
  using G = LnGeom;
  const LinearArgs& a = la.s;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];
  char* const raw = smem;
  char* const prep = smem + G::NST * G::RAW;
  float* const xst = (float*)(smem + G::NST * G::RAW + G::NPREP * G::PREP);
  char* const zst = smem + G::NST * G::RAW + G::NPREP * G::PREP + 2 * G::XST * 4;  // 2 Z tiles

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int bt = PAD ? a.b : 16;  // tokens per tile
  const int ntiles = PAD ? (T + bt - 1) / bt : (T + 15) >> 4;
  // token of row r of tile t
  auto tokrow = [&](int t, int r) {
    if constexpr (PAD)
      return r < bt ? t * bt + r : T;
    else
      return t * 16 + r;
  };

  // Z through a range-checked buffer (rows past T are dropped).  A token's
  // 256-byte row spans the four compute waves (16 rows each), so they stage
  // their parts in an LDS tile (two, alternating) and helpers 1 and 2 store
  // whole rows from it one tile later: 1 KB of consecutive memory per store.
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.z + (size_t)unit * T * 64, (uint32_t)T * 256);
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  // tokens tok0 + 4 k + g (k = 0, 1) of staged tile t to HBM, lane chunk c
  auto flush_z = [&](int t, int tok0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tk = tok0 + 4 * k + g;
      const f32x4 Z = *(const f32x4*)(zst + (t & 1) * G::ZT + tk * G::ZROW + c * 16);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Z), rz,
                                             (uint32_t)(tokrow(t, tk) * 256 + c * 16), 0, 2);
    }
  };

  // ================================================================ loader
  // Barriers B_-2, B_-1, B_0 .. B_ntiles.  At B_j raw tiles <= j+2 have
  // landed.  Raw tile t is read up to compute iteration t (its Q rows; the
  // iteration between B_t and B_{t+1}), so after B_{j-1} the loader reuses
  // the slot of tile j-2 for tile j+D+1: NST = D + 3 slots, D - 1 tiles in
  // flight at each barrier.
  if (wave == G::W_LOAD) {
    const uint32_t ubytes = (uint32_t)T * 128;
    const size_t uoff = (size_t)unit * T * 64;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const short*)a.k + uoff, ubytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const short*)a.q + uoff, ubytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const short*)a.v + uoff, ubytes);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    const int krow = lane >> 3, kpos = lane & 7;
    auto issue = [&](int j) {
      char* st = raw + (j % G::NST) * G::RAW;
      const uint32_t tb = (uint32_t)j * 2048;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = 8 * n + krow;
        const uint32_t off = PAD ? (uint32_t)tokrow(j, r) * 128 + ((kpos ^ (r & 7)) << 4)
                                 : tb + r * 128 + ((kpos ^ (r & 7)) << 4);
        dma16(rk, st + n * 1024, off);
        dma16(rq, st + G::KB + n * 1024, off);
        dma16(rv, st + 2 * G::KB + n * 1024,  // V unswizzled
              PAD ? (uint32_t)tokrow(j, r) * 128 + kpos * 16 : tb + n * 1024 + lane * 16);
      }
      if (lane < 16) dma4(re, st + 2 * G::KB + G::VB, (uint32_t)tokrow(j, lane) * 4);
    };
    const int pro = ntiles < G::D + 1 ? ntiles : G::D + 1;
    for (int j = 0; j < pro; ++j) issue(j);
    if (pro == G::D + 1) wait_vmcnt<G::NI * (G::D - 1)>();  // tiles 0, 1 landed
    else wait_vmcnt<0>();
    wg_barrier_pinned();  // B_{-2}
    wg_barrier_pinned();  // B_{-1}
    for (int j = 0; j < ntiles; ++j) {
      if (j + G::D + 1 < ntiles) {
        issue(j + G::D + 1);
        wait_vmcnt<G::NI * (G::D - 1)>();  // tiles <= j+2 landed
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier_pinned();  // B_j
    }
    wg_barrier_pinned();  // B_ntiles
    return;
  }

  // ================================================================ helper
  // Iteration j (between B_j and B_{j+1}, j = -2 .. ntiles-2) prepares tile
  // j+2 into prepared slot (j+2) % 4; compute iteration j reads the slots of
  // tiles j and j+1 in the same interval.  Helper 0 forms the products of
  // the plain scan (triu(K^T Q), K_{j-1}^T K_j, -eta, the update operand);
  // helpers 1 and 2 the LayerNorm terms that do not depend on W, in layout T
  // for compute waves 0, 1 and 2, 3 (lane (c, g), wave block w: rows
  // 16w + 4g .. +3 of token c): 2 gamma (k + beta - v), its sums over their
  // 32 rows per token, and q + beta.
  if (wave != G::W_LOAD && wave >= G::NCW) {
    const int role = wave == G::W_H0 ? 0 : wave == G::W_H1 ? 1 : 2;
    const float* gm = la.gamma + (size_t)head * 64;
    const float* bt = la.beta + (size_t)head * 64;
    const int wb = role == 2 ? 2 : 0;  // first compute-wave block of helpers 1, 2
    f32x4 hg[2], hb[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      hg[w] = *(const f32x4*)(gm + 16 * (wb + w) + 4 * g);
      hb[w] = *(const f32x4*)(bt + 16 * (wb + w) + 4 * g);
    }
    bf16x8 kprev[2], sel[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      for (int e = 0; e < 8; ++e) {
        kprev[h][e] = (bf16)0.f;
        sel[h][e] = (bf16)((g == (c >> 2) && e == 4 * h + (c & 3)) ? 1.f : 0.f);
      }
    const int ztok0 = role == 1 ? 0 : 8;  // the staged tokens this helper stores
    wg_barrier_pinned();  // B_{-2}
    for (int j = -2; j < ntiles - 1; ++j) {
      const int tn = j + 2;
      // tile j-2's outputs, staged by the compute waves before B_j
      if (role != 0 && j >= 2) flush_z(j - 2, ztok0);
      if (tn >= ntiles) {
        wait_lgkm0();
        wg_barrier_pinned();  // B_{j+1}
        continue;
      }
      const char* st = raw + (tn % G::NST) * G::RAW;
      const char* Kt = st;
      char* pp = prep + (tn % G::NPREP) * G::PREP;
      if (role == 0) {
        const char* Qt = st + G::KB;
        const float* Et = (const float*)(st + 2 * G::KB + G::VB);
        bf16x8 kop[2], qop[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          kop[h] = row_chunk(Kt, c, h, g);
          qop[h] = row_chunk(Qt, c, h, g);
        }
        f32x4 A = {0, 0, 0, 0}, Mkk = {0, 0, 0, 0}, KS[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          A = mfma_k32(kop[h], qop[h], A);        // A[s = 4g+r][t = c] = k_s . q_t
          Mkk = mfma_k32(kprev[h], kop[h], Mkk);  // k^{prev}_s . k_t
        }
        // update operand kt[m][e] = K[t = 4g+e][sigma(m, c)] (exact selection)
#pragma unroll
        for (int m = 0; m < 4; ++m) KS[m] = mfma_k32(kop[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > c) A[r] = 0.f;
        put_split(pp + G::P_A, lane, A);
        const Split4x3 m3 = split4x3(Mkk);
        const uint2 mh = s4u(m3.hi), mm = s4u(m3.mid);
        *(uint4*)(pp + G::P_MKK + lane * 16) = make_uint4(mh.x, mh.y, mm.x, mm.y);
        *(uint2*)(pp + G::P_MKL + lane * 8) = s4u(m3.lo);
        if (lane < 16) ((float*)(pp + G::P_NE))[lane] = -Et[lane];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t p0 = pack_rne(KS[m][0], KS[m][1]), p1 = pack_rne(KS[m][2], KS[m][3]);
          *(uint4*)(pp + G::P_KT + m * 1024 + lane * 16) = make_uint4(p0, p1, p0, p1);
        }
        kprev[0] = kop[0];
        kprev[1] = kop[1];
      } else {
        float su = 0.f;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int rb = 16 * (wb + w) + 4 * g;
          const f32x4 kf = bf4(*(const uint2*)(Kt + swz(c, rb)));
          const f32x4 vf = bf4(*(const uint2*)(st + 2 * G::KB + c * 128 + rb * 2));
          f32x4 gu;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gu[r] = hg[w][r] * ((kf[r] + hb[w][r]) - vf[r]);
            su += gu[r];
          }
          *(f32x4*)(pp + G::P_GU + (wb + w) * 1024 + lane * 16) = gu + gu;
          const f32x4 qf = bf4(*(const uint2*)(st + G::KB + swz(c, rb)));
          *(f32x4*)(pp + G::P_QB + (wb + w) * 1024 + lane * 16) = qf + hb[w];
        }
        const float t = fold32(su, su);
        su = fold16(t, t);
        if (lane < 16) ((float*)(pp + (role == 1 ? G::P_SGU : G::P_SGU2)))[lane] = su;
      }
      wait_lgkm0();
      wg_barrier_pinned();  // B_{j+1}
    }
    wg_barrier_pinned();  // B_ntiles
    // the last two staged tiles (tile ntiles-1 goes out from the compute waves)
    if (role != 0) {
      if (ntiles >= 3) flush_z(ntiles - 3, ztok0);
      if (ntiles >= 2) flush_z(ntiles - 2, ztok0);
    }
    return;
  }

  // =============================================================== compute
  __builtin_amdgcn_s_setprio(3);
  const int rbase = wave * 16;
  const float* w0 = a.w0 + (size_t)(a.w0_per_batch ? unit : head) * 4096;
  f32x4 W[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    W[m] = *(const f32x4*)(w0 + (rbase + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1));
  // LayerNorm scale of this lane's rows (layout T: rows rbase + 4g + r)
  const float* gm = la.gamma + (size_t)head * 64;
  const f32x4 gam = *(const f32x4*)(gm + rbase + 4 * g);
  f32x4 gsq, tg;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    gsq[r] = gam[r] * gam[r];
    tg[r] = 2.f * gsq[r];
  }
  float G2 = 0.f;  // sum over all 64 rows of gamma^2
  for (int i = 0; i < 64; ++i) G2 = fmaf(gm[i], gm[i], G2);
  const float eps = la.eps;
  const int tpm = TPM > 0 ? TPM : (a.b >> 4);  // tiles per mini-batch
  const int nmb = (T + a.b - 1) / a.b;           // mini-batches (checkpoints)

  const NegSel ns = make_negsel(c, g);
  // one-hot selections that carry the hi (slots 0..3) or lo (4..7) half of a
  // layout-T operand to layout A
  bf16x8 selH, selL;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    selH[e] = (bf16)((e < 4 && 4 * g + e == c) ? 1.f : 0.f);
    selL[e] = (bf16)((e >= 4 && 4 * g + e - 4 == c) ? 1.f : 0.f);
  }
  // statistic slots: after the in-wave fold, row g of u0 holds statistic
  // s0[g], of u1 statistic s0[g] + 4
  const int s0g = (g == 0) ? 0 : (g == 1) ? 2 : (g == 2) ? 1 : 3;
  const int lane16 = lane * 16, wblk = wave * 1024;
  // per-lane byte offsets inside the exchange buffers and the raw tiles
  const int xw0 = ((s0g * 16 + c) * 4 + wave) * 4, xw1 = xw0 + 4 * 16 * 4 * 4;
  const int xr0 = (s0g * 16 + c) * 16, xr1 = xr0 + 4 * 16 * 4 * 4;
  const int kc0 = c * 128 + (((0 + g) ^ (c & 7)) << 4), kc1 = c * 128 + (((4 + g) ^ (c & 7)) << 4);

  // Partial sums over this wave's rows of the per-token statistics
  //   0 sum y, 1 sum y^2, 2 sum gamma^2 y, 3 sum gamma^2 y^2, 4 sum 2 gu y,
  //   6 sum o, 7 sum o^2   (y = W0 k, gu = gamma (k + beta - v), o = pre-LN
  // output; slot 5 is unused), folded over the 4 lane rows and written to
  // exchange buffer xs.
  auto publish = [&](char* xs, const f32x4& Y, const f32x4& GU2, const f32x4& O) {
    float p[8];
    f32x4 gy2;
#pragma unroll
    for (int r = 0; r < 4; ++r) gy2[r] = gsq[r] * Y[r];
    p[0] = (Y[0] + Y[1]) + (Y[2] + Y[3]);
    p[1] = fmaf(Y[3], Y[3], fmaf(Y[2], Y[2], fmaf(Y[1], Y[1], Y[0] * Y[0])));
    p[2] = (gy2[0] + gy2[1]) + (gy2[2] + gy2[3]);
    p[3] = fmaf(gy2[3], Y[3], fmaf(gy2[2], Y[2], fmaf(gy2[1], Y[1], gy2[0] * Y[0])));
    p[4] = fmaf(GU2[3], Y[3], fmaf(GU2[2], Y[2], fmaf(GU2[1], Y[1], GU2[0] * Y[0])));
    p[5] = 0.f;
    p[6] = (O[0] + O[1]) + (O[2] + O[3]);
    p[7] = fmaf(O[3], O[3], fmaf(O[2], O[2], fmaf(O[1], O[1], O[0] * O[0])));
    const float t0 = fold32(p[0], p[1]), t1 = fold32(p[2], p[3]);
    const float t2 = fold32(p[4], p[5]), t3 = fold32(p[6], p[7]);
    *(float*)(xs + xw0) = fold16(t0, t1);
    *(float*)(xs + xw1) = fold16(t2, t3);
  };
  // Totals of the 8 statistics for token c, in every lane, from the partial
  // sums of the four waves.
  auto gather = [&](const f32x4& v0, const f32x4& v1, float S[8]) {
    const float a0 = (v0[0] + v0[1]) + (v0[2] + v0[3]);
    const float a1 = (v1[0] + v1[1]) + (v1[2] + v1[3]);
    float lo, hi;
    bcast32(a0, lo, hi);  // rows: lo = [S0, S2, S0, S2], hi = [S1, S3, S1, S3]
    bcast16(lo, S[0], S[2]);
    bcast16(hi, S[1], S[3]);
    bcast32(a1, lo, hi);
    bcast16(lo, S[4], S[6]);
    bcast16(hi, S[5], S[7]);
  };

  // Lane (c, g) of a compute wave holds rows rbase + 4g .. +3 of token c.
  const uint32_t zlane = (uint32_t)((c * 64 + rbase + 4 * g) * 4);
  // z = q + beta + gamma (o - mu_o) rs_o, from the output statistics S6, S7
  auto z_of = [&](const float S[8], const f32x4& O, const f32x4& QB) {
    const float mo = S[6] * (1.f / 64);
    const float vo = fmaxf(fmaf(S[7], 1.f / 64, -mo * mo), 0.f);
    const float ro = rsqrtf(vo + eps);
    f32x4 Z;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rg = ro * gam[r];
      Z[r] = fmaf(O[r], rg, fmaf(-mo, rg, QB[r]));
    }
    return Z;
  };
  // tile t's part of this lane into the staging tile of t's parity
  auto stage_z = [&](int t, const float S[8], const f32x4& O, const f32x4& QB) {
    *(f32x4*)(zst + (t & 1) * G::ZT + c * G::ZROW + (rbase + 4 * g) * 4) = z_of(S, O, QB);
  };
  // the last tile directly (no barrier follows it)
  auto store_z = [&](int t, const float S[8], const f32x4& O, const f32x4& QB) {
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(u32x4, z_of(S, O, QB)), rz,
        PAD ? (uint32_t)((tokrow(t, c) * 64 + rbase + 4 * g) * 4) : zlane + (uint32_t)t * (16 * 64 * 4), 0, 2);
  };

  wg_barrier_pinned();  // B_{-2}: raw tiles 0 and 1 are in LDS
  Split8x3 wg[2];       // split of the gradient point (b > 16)
  f32x4 Y;              // W0 K of the current tile (layout T)
  {
    const Split8x3 ws[2] = {split8x3(W[0], W[1], ns), split8x3(W[2], W[3], ns)};
    wg[0] = ws[0];
    wg[1] = ws[1];
    Y = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 k = row_chunk(raw, c, h, g);
      Y = mfma_k32(ws[h].hi, k, Y);
      Y = mfma_k32(ws[h].mid, k, Y);
      Y = mfma_k32(ws[h].lo, k, Y);
    }
  }
  wg_barrier_pinned();  // B_{-1}: prepared tile 0 is in LDS
  f32x4 GU2 = *(const f32x4*)(prep + G::P_GU + wblk + lane16);  // 2 gamma U, tile 0
  publish((char*)xst, Y, GU2, f32x4{0, 0, 0, 0});
  wait_lgkm0();
  wg_barrier_pinned();  // B_0: statistics of tile 0 and prepared tiles 0, 1 ready
  f32x4 O = {0, 0, 0, 0}, QB = {0, 0, 0, 0};  // pre-LN outputs of the previous tile, q + beta

  // One tile.  POS = the tile's position in its mini-batch when fixed at
  // compile time (std::integral_constant), -1 otherwise.
  auto tile = [&](const int j, auto POS) {
    constexpr int pos = decltype(POS)::value;
    const bool new_mb = TPM == 1 || (pos >= 0 ? pos == 0 : (j % tpm) == 0);
    const bool next_new = TPM == 1 || (pos >= 0 ? (pos + 1) % (TPM > 0 ? TPM : 1) == 0
                                                : ((j + 1) % tpm) == 0);
    const char* pj = prep + (j & (G::NPREP - 1)) * G::PREP;
    const char* pj1 = prep + ((j + 1) & (G::NPREP - 1)) * G::PREP;
    const char* tj = raw + (j % G::NST) * G::RAW;
    const char* tj1 = raw + ((j + 1) % G::NST) * G::RAW;
    const char* xs = (const char*)xst + (j & 1) * (G::XST * 4);
    char* xsn = (char*)xst + ((j + 1) & 1) * (G::XST * 4);

    // The body is cut into phases that the compiler may not interleave
    // (sched_barrier): left to itself it spreads the off-chain products
    // through the serial chain, which in-order issue then waits behind.
    //   1. LDS reads, the split of W_j and its products (off the chain);
    //   2. statistics -> gradient; 3. transposition MFMAs;
    //   4. outputs of tile j-1, the correction of Y_{j+1}, W_j Q_j's
    //      correction, the update; then the statistics of tile j+1.
    // ---- reads: the statistics first (they start the serial chain)
    const f32x4 v0 = *(const f32x4*)(xs + xr0), v1 = *(const f32x4*)(xs + xr1);
    const float ne = ((const float*)(pj + G::P_NE))[c];  // -eta_t
    const float sgu = ((const float*)(pj + G::P_SGU))[c] + ((const float*)(pj + G::P_SGU2))[c];
    const bf16x8 k1a = *(const bf16x8*)(tj1 + kc0), k1b = *(const bf16x8*)(tj1 + kc1);
    const bf16x8 q0a = *(const bf16x8*)(tj + G::KB + kc0), q0b = *(const bf16x8*)(tj + G::KB + kc1);
    const uint4 mkk1 = *(const uint4*)(pj1 + G::P_MKK + lane16);  // [hi | mid]
    const uint2 mkl1 = *(const uint2*)(pj1 + G::P_MKL + lane * 8);  // lo
    const bf16x8 att = get8(pj + G::P_A, lane);
    bf16x8 kt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kt[m] = get8(pj + G::P_KT + m * 1024, lane);
    const f32x4 qb = *(const f32x4*)(pj + G::P_QB + wblk + lane16);
    const f32x4 gu2n = *(const f32x4*)(pj1 + G::P_GU + wblk + lane16);
    const bf16x8 k1[2] = {k1a, k1b}, q0[2] = {q0a, q0b};

    if constexpr (CKPT) {  // W_j is the state before mini-batch j / tpm
      if (new_mb) {  // nontemporal: read back only by the backward
        typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w_ckpt + ((size_t)unit * nmb + j / tpm) * 4096, 4096u * 4u);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4c, W[m]), rc,
                                                 (uint32_t)(((rbase + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) * 4),
                                                 0, 2);
      }
    }
    // ---- products with W_j that do not wait for the gradient: its split,
    // W_j K_{j+1} (or the gradient point's), W_j Q_j
    const Split8x3 ws[2] = {split8x3(W[0], W[1], ns), split8x3(W[2], W[3], ns)};
    if (TPM != 1 && new_mb) {
      wg[0] = ws[0];
      wg[1] = ws[1];
    }
    f32x4 Yn = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const Split8x3& wy = next_new ? ws[h] : wg[h];
      Yn = mfma_k32(wy.hi, k1[h], Yn);
      Yn = mfma_k32(wy.mid, k1[h], Yn);
      Yn = mfma_k32(wy.lo, k1[h], Yn);
    }
    f32x4 R = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      R = mfma_k32(ws[h].hi, q0[h], R);
      R = mfma_k32(ws[h].mid, q0[h], R);
    }

    // ---- gradient of tile j (layout T), token c:
    //   Gn_r = -eta [rs (2 gu_r - m1) + rs^2 (2 gamma_r^2 - m2)(y_r - mu)]
    __builtin_amdgcn_sched_barrier(0);
    float S[8];
    gather(v0, v1, S);
    const float mu = S[0] * (1.f / 64);
    const float var = fmaxf(fmaf(S[1], 1.f / 64, -mu * mu), 0.f);
    const float rs = rsqrtf(var + eps);
    const float m1 = (2.f / 64) * fmaf(rs, fmaf(-mu, G2, S[2]), sgu);
    const float c3 = fmaf(mu, fmaf(mu, G2, -2.f * S[2]), S[3]);  // sum gamma^2 (y - mu)^2
    const float m2 = (2.f / 64) * rs * fmaf(rs, c3, fmaf(-mu, sgu, 0.5f * S[4]));  // S4 = sum 2 gu y
    const float a0 = ne * rs, a1 = a0 * rs;
    const float na0m1 = -a0 * m1, nm2a1 = -m2 * a1;
    f32x4 GnT;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      GnT[r] = fmaf(fmaf(tg[r], a1, nm2a1), Y[r] - mu, fmaf(a0, GU2[r], na0m1));

    __builtin_amdgcn_sched_barrier(0);
    // ---- gradient to layout A: its three bf16 terms moved exactly
    const Split4x3 gT = split4x3(GnT);
    const bf16x8 gat = cat44(gT.hi, gT.mid);
    const bf16x8 gal = cat44(gT.lo, s16x4{0, 0, 0, 0});
    const f32x4 CH = mfma_k32(gat, selH, f32x4{0, 0, 0, 0});
    const f32x4 CM = mfma_k32(gat, selL, f32x4{0, 0, 0, 0});
    const f32x4 CL = mfma_k32(gal, selH, f32x4{0, 0, 0, 0});

    __builtin_amdgcn_sched_barrier(0);
    // ---- outputs of tile j-1 (off the chain, while the MFMAs run), staged
    // in LDS for the helpers
    if (j > 0) stage_z(j - 1, S, O, QB);

    Split4 gs;  // hi, mid: the operands of the products with K^T K and K^T Q
    gs.hi = u2s(make_uint2(pack_rne(CH[0], CH[1]), pack_rne(CH[2], CH[3])));
    gs.lo = u2s(make_uint2(pack_rne(CM[0], CM[1]), pack_rne(CM[2], CM[3])));
    const s16x4 glo = u2s(make_uint2(pack_rne(CL[0], CL[1]), pack_rne(CL[2], CL[3])));
    const YOps gy = yops(gs);

    // ---- Y_{j+1} += Gn_j (K_j^T K_{j+1}) at a new mini-batch, both factors in
    // three terms; the six products above 2^-24 in three MFMAs:
    // hi.[hi|mid] + [mid|lo].hi + [hi|mid].[lo|mid]
    const bf16x8 g2 = cat44(gs.hi, gs.lo);            // [hi | mid]
    const bf16x8 g3 = cat44(glo, s16x4{0, 0, 0, 0});  // [lo | 0]
    if (next_new) {
      const bf16x8 x1 = __builtin_bit_cast(bf16x8, mkk1);
      const bf16x8 x2 = __builtin_bit_cast(bf16x8, make_uint4(mkk1.x, mkk1.y, mkk1.x, mkk1.y));
      const bf16x8 x3 = __builtin_bit_cast(bf16x8, make_uint4(mkl1.x, mkl1.y, mkk1.z, mkk1.w));
      Yn = mfma_k32(gy.hh, x1, Yn);
      Yn = mfma_k32(cat44(gs.lo, glo), x2, Yn);
      Yn = mfma_k32(g2, x3, Yn);
    }

    // ---- pre-LN outputs of tile j: W_j Q_j + Gn_j triu(K_j^T Q_j)
    R = mm_pre_t(gy, att, R);

    __builtin_amdgcn_sched_barrier(0);
    // ---- rank-16 update W_{j+1} = W_j + Gn_j K_j^T
#pragma unroll
    for (int m = 0; m < 4; ++m) W[m] = mfma_k32(kt[m], g3, mfma_k32(kt[m], g2, W[m]));

    // ---- hand over to tile j+1: publish its statistics
    publish(xsn, Yn, gu2n, R);

    GU2 = gu2n;
    QB = qb;
    O = R;
    Y = Yn;
    wait_lgkm0();
    wg_barrier_pinned();  // B_{j+1}
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using PN = std::integral_constant<int, -1>;
  int j = 0;
  if constexpr (TPM == 1) {
    for (; j < ntiles; ++j) tile(j, P0{});
  } else if constexpr (TPM == 2) {
    for (; j + 1 < ntiles; j += 2) {
      tile(j, P0{});
      tile(j + 1, P1{});
    }
    if (j < ntiles) tile(j, P0{});
  } else if constexpr (TPM == 4) {
    for (; j + 3 < ntiles; j += 4) {
      tile(j, P0{});
      tile(j + 1, P1{});
      tile(j + 2, P2{});
      tile(j + 3, P3{});
    }
    if (j < ntiles) tile(j, P0{});
    if (j + 1 < ntiles) tile(j + 1, P1{});
    if (j + 2 < ntiles) tile(j + 2, P2{});
  } else {
    for (; j < ntiles; ++j) tile(j, PN{});
  }
  {
    const char* xs = (const char*)xst + (ntiles & 1) * (G::XST * 4);
    float S[8];
    gather(*(const f32x4*)(xs + xr0), *(const f32x4*)(xs + xr1), S);
    store_z(ntiles - 1, S, O, QB);
  }

  float* wo = a.w_out + (size_t)unit * 4096;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    *(f32x4*)(wo + (rbase + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) = W[m];
}

}  // namespace

hipError_t launch_linear_ln(const LinearLnArgs& a, hipStream_t s) {
  const dim3 grid(a.s.units), block(LnGeom::THREADS);
  if (a.s.b < 16)  // one mini-batch per zero-padded tile
    return a.s.w_ckpt ? launch(linear_ln_scan_kernel<1, true, true>, grid, block, s, a)
                      : launch(linear_ln_scan_kernel<1, false, true>, grid, block, s, a);
  if (a.s.w_ckpt) {
    switch (a.s.b) {
      case 16: return launch(linear_ln_scan_kernel<1, true>, grid, block, s, a);
      case 32: return launch(linear_ln_scan_kernel<2, true>, grid, block, s, a);
      case 64: return launch(linear_ln_scan_kernel<4, true>, grid, block, s, a);
      default: return launch(linear_ln_scan_kernel<0, true>, grid, block, s, a);
    }
  }
  switch (a.s.b) {
    case 16: return launch(linear_ln_scan_kernel<1>, grid, block, s, a);
    case 32: return launch(linear_ln_scan_kernel<2>, grid, block, s, a);
    case 64: return launch(linear_ln_scan_kernel<4>, grid, block, s, a);
    default: return launch(linear_ln_scan_kernel<0>, grid, block, s, a);
  }
}

}  // namespace ttt
