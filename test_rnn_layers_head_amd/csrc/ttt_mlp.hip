// TTT-MLP forward scan for gfx950: f(x) = W2 GELU(W1 x), hidden = 256, d = 64.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): mini-batch GD of the reconstruction loss
// ||f(k_t) - v_t||^2 with both layers' gradients taken at the state before
// the mini-batch (§3.5), per-token eta (§4.6), evaluated per tile in the MLP
// dual form of §3.7 / App. A:
//   Z1 = W1 K, X2 = GELU(Z1), Z2 = W2 X2,
//   G2 = 2 (Z2 - V) diag(eta),  G1 = (W2^T G2) * GELU'(Z1),
//   Z1q = W1 Q - G1 triu(K^T Q),  X2q = GELU(Z1q),
//   Z = W2 X2q - G2 triu(X2^T X2q),
//   W1 <- W1 - G1 K^T,  W2 <- W2 - G2 X2^T.
// Columns are tokens; the causal mask keeps s <= t (token t's output sees its
// own update, §3.1).  The kernel carries Gn = -G.  GELU is x Phi(x) with the
// error function from Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7).
//
// Work split: one workgroup per (batch, head) unit, 8 waves.  Wave w owns the
// hidden units u in [32w, 32w + 32) (two 16-blocks): its rows of W1 and its
// columns of W2, all in fp32 registers for the whole sequence.  W2 enters
// contractions over u (forward) and over i (backward), so each wave keeps
// its W2 block in both accumulator layouts (W2T: lane holds i = c and 4
// consecutive u; W2N: lane holds u = c and 4 consecutive i) and updates both
// on MFMA.  The two cross-wave sums per tile (Z2 and Z over hidden units)
// go through LDS: every wave writes its partial, waves 0..3 each reduce one
// 16-column block.  Transposes of 16x16 fp32 blocks use an MFMA with the
// identity as the other operand (exact for hi + lo bf16 halves).
//
// Inputs are register-staged one tile ahead by the waves themselves (each
// lane moves one 16-byte chunk of K, Q, V or one eta), so no wave issues
// LDS-DMA and no wave is idle.  Mini-batches b < 16 (b | 16) run each
// sub-batch of a tile as its own pass with eta masked to that sub-batch.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int NW = 8;          // waves per workgroup
constexpr int HID = 256;       // hidden units
constexpr int RAWB = 2048 * 3 + 64;  // K (swizzled), Q (swizzled), V, eta
// LDS map (bytes)
constexpr int L_RAW = 0;                         // 2 raw tile slots
constexpr int L_Z2P = L_RAW + 2 * RAWB;          // [wave][mi][lane] f32x4 partial Z2^T
constexpr int L_ZP = L_Z2P + NW * 4 * 1024;      // [wave][mi][lane] f32x4 partial Z^T
constexpr int L_A2P = L_ZP + NW * 4 * 1024;      // [wave][lane] f32x4 partial X2^T X2q
constexpr int L_G2A = L_A2P + NW * 1024;         // [mi][lane] hi|lo of Gn2^T (t x i layout)
constexpr int L_G2B = L_G2A + 4 * 1024;          // [mi][lane] hi|lo of Gn2   (i x t layout)
constexpr int L_TOTAL = L_G2B + 4 * 1024;

__device__ __forceinline__ int swz_chunk(int r, int p) { return r * 128 + ((p ^ (r & 7)) << 4); }
__device__ __forceinline__ bf16x8 row_chunk(const char* tile, int r, int h, int g) {
  return *(const bf16x8*)(tile + swz_chunk(r, 4 * h + g));
}

// GELU and its derivative.  Phi(x) = 1/2 (1 + erf(x / sqrt 2)); erf from
// Abramowitz & Stegun 7.1.26: erf(y) = 1 - (a1 t + .. + a5 t^5) exp(-y^2),
// t = 1 / (1 + p y), y >= 0.  exp(-y^2) = exp(-x^2 / 2) is shared with the
// normal density phi(x) = exp(-x^2 / 2) / sqrt(2 pi) of GELU' = Phi + x phi.
struct GeluOut {
  float g, dg;
};
__device__ __forceinline__ GeluOut gelu_and_grad(float x) {
  const float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
              a4 = -1.453152027f, a5 = 1.061405429f;
  const float y = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, y, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);  // exp(-x^2/2)
  const float q = 0.5f * poly * e;                                         // 1 - Phi(|x|)
  const float phi_cdf = x >= 0.f ? 1.f - q : q;
  return GeluOut{x * phi_cdf, fmaf(x, e * 0.39894228040143268f, phi_cdf)};
}

struct YOps {
  bf16x8 hh, l0;
};
__device__ __forceinline__ YOps yops(const Split4& y) {
  const s16x4 z = {0, 0, 0, 0};
  return YOps{cat44(y.hi, y.hi), cat44(y.lo, z)};
}
// acc + X*Y, X as [Xhi | Xlo] of the accumulator layout of X^T (three terms)
__device__ __forceinline__ f32x4 mm_pre(bf16x8 x, const YOps& y, f32x4 acc) {
  acc = mfma_k32(x, y.hh, acc);
  acc = mfma_k32(x, y.l0, acc);
  return acc;
}
// acc + A*B for 8-slot operands split into hi/lo (three terms)
__device__ __forceinline__ f32x4 mm3(const Split8& a, const Split8& b, f32x4 acc) {
  acc = mfma_k32(a.hi, b.hi, acc);
  acc = mfma_k32(a.hi, b.lo, acc);
  acc = mfma_k32(a.lo, b.hi, acc);
  return acc;
}
__device__ __forceinline__ uint4 pack_split(const Split4& s) {
  const uint2 h = __builtin_bit_cast(uint2, s.hi), l = __builtin_bit_cast(uint2, s.lo);
  return make_uint4(h.x, h.y, l.x, l.y);
}
__device__ __forceinline__ Split4 unpack_split(uint4 v) {
  return Split4{__builtin_bit_cast(s16x4, make_uint2(v.x, v.y)),
                __builtin_bit_cast(s16x4, make_uint2(v.z, v.w))};
}

template <bool SUB>
__global__ void __launch_bounds__(NW * 64) mlp_scan_kernel(MlpArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[L_TOTAL];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int ntiles = (T + 15) >> 4;
  const int bsub = SUB ? a.b : 16;
  const int npass = 16 / bsub;

  // ------------------------------------------------------------ constants
  bf16x8 sel[2], itr, negI;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // one-hot selection of column sigma(m, c) within a 32-column block (m % 2 = h)
    sel[0][e] = (bf16)((g == (c >> 2) && e == (c & 3)) ? 1.f : 0.f);
    sel[1][e] = (bf16)((g == (c >> 2) && e == 4 + (c & 3)) ? 1.f : 0.f);
    // [hi | lo] of 4 indices 4g..4g+3 -> identity: transposes a 16x16 block
    itr[e] = (bf16)((4 * g + (e & 3) == c) ? 1.f : 0.f);
    // -I on 16 V columns (slots 16..31 unused)
    negI[e] = (bf16)((g < 2 && 8 * g + e == c) ? -1.f : 0.f);
  }

  // ---------------------------------------------------------------- state
  const size_t wsel = a.w0_per_batch ? unit : head;
  const float* w1g = a.w1_0 + wsel * HID * 64;
  const float* w2g = a.w2_0 + wsel * 64 * HID;
  f32x4 W1[2][4];   // [n][m]: W1[u = 32w + 16n + c][sigma(m, 4g + r)]
  f32x4 W2T[2][4];  // [nu][mi]: W2[i = 16mi + c][u = 32w + 16nu + 4g + r]
  f32x4 W2N[4][2];  // [mi][nu]: W2[i = 16mi + 4g + r][u = 32w + 16nu + c]
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      W1[n][m] = *(const f32x4*)(w1g + (32 * w + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1));
#pragma unroll
  for (int nu = 0; nu < 2; ++nu)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      W2T[nu][mi] = *(const f32x4*)(w2g + (16 * mi + c) * HID + 32 * w + 16 * nu + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) W2N[mi][nu][r] = w2g[(16 * mi + 4 * g + r) * HID + 32 * w + 16 * nu + c];
    }

  // ------------------------------------------------------- input staging
  // flat lane q = 64 w + lane moves: q < 128 a K chunk, q < 256 a Q chunk,
  // q < 384 a V chunk, q < 400 one eta; zero past T (buffer range check).
  const int q = w * 64 + lane;
  const size_t uoff = (size_t)unit * T * 64;
  __amdgpu_buffer_rsrc_t rsrc;
  int ldst = -1;          // LDS byte offset within a raw slot
  uint32_t gsrc = 0;      // byte offset of the chunk within tile 0
  uint32_t gstep = 2048;  // bytes per tile in the source
  bool is_eta = false;
  if (q < 384) {
    const int part = q >> 7, ch = q & 127, r = ch >> 3, p = ch & 7;
    const void* base = part == 0 ? a.k : (part == 1 ? a.q : a.v);
    rsrc = make_rsrc((const short*)base + uoff, (uint32_t)T * 128);
    gsrc = r * 128 + p * 16;
    ldst = part * 2048 + (part < 2 ? swz_chunk(r, p) : gsrc);
  } else if (q < 400) {
    rsrc = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    gsrc = (q - 384) * 4;
    gstep = 64;
    ldst = 3 * 2048 + (q - 384) * 4;
    is_eta = true;
  } else {
    rsrc = make_rsrc(a.eta, 0);
  }
  auto fetch = [&](int j) -> uint4 {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ldst >= 0 && j < ntiles) {
      const uint32_t off = gsrc + (uint32_t)j * gstep;
      if (is_eta) v.x = __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
      else v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
    return v;
  };
  auto stash = [&](int j, uint4 v) {
    if (ldst >= 0 && j < ntiles) {
      char* dst = smem + L_RAW + (j & 1) * RAWB + ldst;
      if (is_eta) *(uint32_t*)dst = v.x;
      else *(uint4*)dst = v;
    }
  };

  const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.z + uoff, (uint32_t)T * 256);

  stash(0, fetch(0));
  uint4 pf = fetch(1);
  wg_barrier();

  YOps g2prev[4];  // Gn2 operands of the previous pass (for its Z reduction)
  int prev_tile = -1, prev_pass = 0;

  for (int j = 0; j < ntiles; ++j) {
    const char* raw = smem + L_RAW + (j & 1) * RAWB;
    const char* Kt = raw;
    const char* Qt = raw + 2048;
    const char* Vt = raw + 4096;
    const float* Et = (const float*)(raw + 6144);
    bf16x8 kop[2], qop[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kop[h] = row_chunk(Kt, c, h, g);
      qop[h] = row_chunk(Qt, c, h, g);
    }
    // per-tile operands that depend on K, Q only
    f32x4 Am = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) Am = mfma_k32(kop[h], qop[h], Am);  // A[s = 4g+r][t = c]
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > c) Am[r] = 0.f;
    const Split4 as = split4(Am);
    const bf16x8 aop = cat44(as.hi, as.lo);
    bf16x8 kt2[4];  // [kt | kt], kt[e] = K[t = 4g+e][sigma(m, c)]
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 x = mfma_k32(kop[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});
      const uint32_t p0 = pack_exact(x[0], x[1]), p1 = pack_exact(x[2], x[3]);
      kt2[m] = __builtin_bit_cast(bf16x8, make_uint4(p0, p1, p0, p1));
    }
    const f32x4 eta4 = *(const f32x4*)(Et + 4 * g);

    for (int p = 0; p < npass; ++p) {
      // ================= reduce Z of the previous pass (waves 0..3, block mi = w)
      if (w < 4 && prev_tile >= 0) {
        const int mi = w;
        f32x4 Zt = {0, 0, 0, 0}, A2 = {0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          Zt += *(const f32x4*)(smem + L_ZP + (v * 4 + mi) * 1024 + lane * 16);
          A2 += *(const f32x4*)(smem + L_A2P + v * 1024 + lane * 16);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > c) A2[r] = 0.f;
        const Split4 a2s = split4(A2);
        Zt = mm_pre(cat44(a2s.hi, a2s.lo), g2prev[mi], Zt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 4 * g + r;
          const bool act = !SUB || (tl / bsub) == prev_pass;
          const float zr = Zt[r];
          if (act)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zr), rz,
                                                  (uint32_t)(((prev_tile * 16 + tl) * 64 + 16 * mi + c) * 4), 0, 2);
        }
      }

      // eta of this pass (sub-batch p of the tile)
      f32x4 e2;
#pragma unroll
      for (int r = 0; r < 4; ++r) e2[r] = (!SUB || (4 * g + r) / bsub == p) ? 2.f * eta4[r] : 0.f;

      // ================= forward at the gradient point
      Split8 w1s[2][2];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int h = 0; h < 2; ++h) w1s[n][h] = split8(W1[n][2 * h], W1[n][2 * h + 1]);
      f32x4 Z1[2], D[2], X2t[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        Z1[n] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Z1[n] = mfma_k32(kop[h], w1s[n][h].hi, Z1[n]);
          Z1[n] = mfma_k32(kop[h], w1s[n][h].lo, Z1[n]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const GeluOut o = gelu_and_grad(Z1[n][r]);
          X2t[n][r] = o.g;  // X2^T[t = 4g+r][u = 32w + 16n + c]
          D[n][r] = o.dg;
        }
      }
      const Split4 x2ts[2] = {split4(X2t[0]), split4(X2t[1])};
      // X2[u][t] in accumulator layout (u = 4g+r, t = c), as an operand over u
      Split8 x2op;
      {
        const f32x4 t0 = mfma_k32(cat44(x2ts[0].hi, x2ts[0].lo), itr, f32x4{0, 0, 0, 0});
        const f32x4 t1 = mfma_k32(cat44(x2ts[1].hi, x2ts[1].lo), itr, f32x4{0, 0, 0, 0});
        x2op = split8(t0, t1);
      }
      Split8 w2ts[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) w2ts[mi] = split8(W2T[0][mi], W2T[1][mi]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 z2 = mm3(x2op, w2ts[mi], f32x4{0, 0, 0, 0});  // partial Z2^T[t][i]
        *(f32x4*)(smem + L_Z2P + (w * 4 + mi) * 1024 + lane * 16) = z2;
      }
      wg_barrier();  // B1: partial Z2 written

      // ================= Gn2 = 2 eta (V - Z2), waves 0..3 (block mi = w)
      if (w < 4) {
        const int mi = w;
        f32x4 Z2 = {0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < NW; ++v) Z2 += *(const f32x4*)(smem + L_Z2P + (v * 4 + mi) * 1024 + lane * 16);
        Z2 = mfma_k32(*(const bf16x8*)(Vt + c * 128 + (16 * mi + 8 * (g & 1)) * 2), negI, Z2);  // Z2 - V
        f32x4 G;
#pragma unroll
        for (int r = 0; r < 4; ++r) G[r] = -e2[r] * Z2[r];
        const Split4 gs = split4(G);
        *(uint4*)(smem + L_G2A + mi * 1024 + lane * 16) = pack_split(gs);
        const f32x4 GT = mfma_k32(cat44(gs.hi, gs.lo), itr, f32x4{0, 0, 0, 0});  // Gn2[i][t]
        *(uint4*)(smem + L_G2B + mi * 1024 + lane * 16) = pack_split(split4(GT));
      }
      wg_barrier();  // B2: Gn2 ready

      // ================= backward to layer 1: Gn1^T = (Gn2^T W2) * GELU'(Z1)
      Split4 g2s[4], g2t[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        g2s[mi] = unpack_split(*(const uint4*)(smem + L_G2A + mi * 1024 + lane * 16));
        g2t[mi] = unpack_split(*(const uint4*)(smem + L_G2B + mi * 1024 + lane * 16));
      }
      f32x4 G1[2];
#pragma unroll
      for (int nu = 0; nu < 2; ++nu) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Split8 ga{cat44(g2t[2 * kb].hi, g2t[2 * kb + 1].hi),
                          cat44(g2t[2 * kb].lo, g2t[2 * kb + 1].lo)};
          acc = mm3(ga, split8(W2N[2 * kb][nu], W2N[2 * kb + 1][nu]), acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) G1[nu][r] = acc[r] * D[nu][r];
      }
      const Split4 g1s[2] = {split4(G1[0]), split4(G1[1])};

      // ================= outputs: Z1q, X2q, partial Z and X2^T X2q
      f32x4 X2qt[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4 z1q = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          z1q = mfma_k32(qop[h], w1s[n][h].hi, z1q);
          z1q = mfma_k32(qop[h], w1s[n][h].lo, z1q);
        }
        z1q = mm_pre(aop, yops(g1s[n]), z1q);
#pragma unroll
        for (int r = 0; r < 4; ++r) X2qt[n][r] = gelu_and_grad(z1q[r]).g;
      }
      Split8 x2qop;
      {
        const Split4 s0 = split4(X2qt[0]), s1 = split4(X2qt[1]);
        const f32x4 t0 = mfma_k32(cat44(s0.hi, s0.lo), itr, f32x4{0, 0, 0, 0});
        const f32x4 t1 = mfma_k32(cat44(s1.hi, s1.lo), itr, f32x4{0, 0, 0, 0});
        x2qop = split8(t0, t1);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 zp = mm3(x2qop, w2ts[mi], f32x4{0, 0, 0, 0});
        *(f32x4*)(smem + L_ZP + (w * 4 + mi) * 1024 + lane * 16) = zp;
      }
      *(f32x4*)(smem + L_A2P + w * 1024 + lane * 16) = mm3(x2op, x2qop, f32x4{0, 0, 0, 0});

      // ================= rank-16 updates of both layers
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8 gg = cat44(g1s[n].hi, g1s[n].lo);
#pragma unroll
        for (int m = 0; m < 4; ++m) W1[n][m] = mfma_k32(kt2[m], gg, W1[n][m]);
      }
      YOps g2y[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) g2y[mi] = yops(g2s[mi]);
#pragma unroll
      for (int nu = 0; nu < 2; ++nu) {
        const bf16x8 xa = cat44(x2ts[nu].hi, x2ts[nu].lo);
        const YOps xy = yops(x2ts[nu]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          W2T[nu][mi] = mm_pre(xa, g2y[mi], W2T[nu][mi]);                          // += X2 Gn2^T
          W2N[mi][nu] = mm_pre(cat44(g2s[mi].hi, g2s[mi].lo), xy, W2N[mi][nu]);  // += Gn2 X2^T
        }
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) g2prev[mi] = g2y[mi];
      prev_tile = j;
      prev_pass = p;

      if (p == npass - 1) stash(j + 1, pf);  // next tile's inputs into the other slot
      wg_barrier();  // B0: partials of this pass and the next tile's inputs ready
    }
    pf = fetch(j + 2);
  }

  // Z of the last pass
  if (w < 4 && prev_tile >= 0) {
    const int mi = w;
    f32x4 Zt = {0, 0, 0, 0}, A2 = {0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      Zt += *(const f32x4*)(smem + L_ZP + (v * 4 + mi) * 1024 + lane * 16);
      A2 += *(const f32x4*)(smem + L_A2P + v * 1024 + lane * 16);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > c) A2[r] = 0.f;
    const Split4 a2s = split4(A2);
    Zt = mm_pre(cat44(a2s.hi, a2s.lo), g2prev[mi], Zt);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 4 * g + r;
      const bool act = !SUB || (tl / bsub) == prev_pass;
      const float zr = Zt[r];
      if (act)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zr), rz,
                                              (uint32_t)(((prev_tile * 16 + tl) * 64 + 16 * mi + c) * 4), 0, 2);
    }
  }

  // final state
  float* w1o = a.w1_out + (size_t)unit * HID * 64;
  float* w2o = a.w2_out + (size_t)unit * 64 * HID;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *(f32x4*)(w1o + (32 * w + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) = W1[n][m];
#pragma unroll
  for (int nu = 0; nu < 2; ++nu)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      *(f32x4*)(w2o + (16 * mi + c) * HID + 32 * w + 16 * nu + 4 * g) = W2T[nu][mi];
}

}  // namespace

hipError_t launch_mlp(const MlpArgs& a, bool f32in, hipStream_t s) {
  if (f32in || a.b > 16) return hipErrorNotSupported;
  if (a.b == 16)
    hipLaunchKernelGGL(mlp_scan_kernel<false>, dim3(a.units), dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL(mlp_scan_kernel<true>, dim3(a.units), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
