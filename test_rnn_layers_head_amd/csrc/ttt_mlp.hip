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
// Work split: one workgroup per (batch, head) unit, NW waves.  Wave w owns
// the hidden units u in [U w, U w + U), U = 256 / NW, as NB = U / 16 blocks:
// its rows of W1 and its columns of W2, all in fp32 registers for the whole
// sequence.  NW = 8 (two waves per SIMD, 32 hidden units each) for b = 16:
// the second wave hides the first one's dependency and LDS waits; the b < 16
// variant keeps more per-pass state and runs NW = 4 (one wave per SIMD with
// the whole register file, so nothing spills).  W2 enters
// contractions over u (forward) and over i (backward), so each wave keeps
// its W2 block in both accumulator layouts (W2T: lane holds i = c and 4
// consecutive u, in registers; W2N: lane holds u = c and 4 consecutive i,
// in the wave's own LDS area, read and written block by block) and updates
// both on MFMA.  The two cross-wave sums per tile (Z2 and Z over hidden units)
// go through LDS: every wave writes its partial, wave w < 4 reduces the
// 16-column block w of d = 64.  Transposes of 16x16 fp32 blocks use an MFMA with the
// identity as the other operand (exact for hi + lo bf16 halves).
//
// Inputs are register-staged one tile ahead by the waves themselves (each
// lane moves 16-byte chunks of K, Q, V or one eta), so no wave issues
// LDS-DMA and no wave is idle.  Mini-batches b < 16 (b | 16) run each
// sub-batch of a tile as its own pass with eta masked to that sub-batch.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int HID = 256;              // hidden units
constexpr int RAWB = 2048 * 3 + 64;   // K (swizzled), Q (swizzled), V, eta
template <int NW>
struct MlpGeom {
  static constexpr int U = HID / NW;          // hidden units per wave
  static constexpr int NB = U / 16;           // 16-blocks per wave
  static constexpr int NCH = NB / 2;          // K=32 chunks over the wave's units
  // LDS map (bytes)
  static constexpr int L_RAW = 0;                      // 2 raw tile slots
  static constexpr int L_Z2P = L_RAW + 2 * RAWB;       // [wave][mi][lane] f32x4 partial Z2^T
  static constexpr int L_ZP = L_Z2P + NW * 4 * 1024;   // [wave][mi][lane] f32x4 partial Z^T
  static constexpr int L_A2P = L_ZP + NW * 4 * 1024;   // [wave][lane] f32x4 partial X2^T X2q
  static constexpr int L_G2A = L_A2P + NW * 1024;      // [mi][lane] hi|lo of Gn2^T (t x i)
  static constexpr int L_G2B = L_G2A + 4 * 1024;       // [mi][lane] hi|lo of Gn2 (i x t)
  static constexpr int L_W2N = L_G2B + 4 * 1024;       // [wave][mi][nu][lane] f32x4: W2 (i x u)
  static constexpr int L_TOTAL = L_W2N + NW * 4 * NB * 1024;
  static constexpr int LOADS = (400 + NW * 64 - 1) / (NW * 64);  // staged chunks per lane
};

__device__ __forceinline__ int swz_chunk(int r, int p) { return r * 128 + ((p ^ (r & 7)) << 4); }
__device__ __forceinline__ bf16x8 row_chunk(const char* tile, int r, int h, int g) {
  return *(const bf16x8*)(tile + swz_chunk(r, 4 * h + g));
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

// Sum of the NW partial blocks of a cross-wave reduction, and the final Z of
// one pass for output block mi: Z^T = sum partials + triu(sum A2)^T Gn2^T.
template <int NW, bool SUB>
__device__ __forceinline__ void reduce_store_z(const char* smem, int lane, int c, int g, int mi,
                                               const YOps& g2, __amdgpu_buffer_rsrc_t rz,
                                               int tile, int pass, int bsub) {
  using G = MlpGeom<NW>;
  f32x4 Zt = {0, 0, 0, 0}, A2 = {0, 0, 0, 0};
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    Zt += *(const f32x4*)(smem + G::L_ZP + (v * 4 + mi) * 1024 + lane * 16);
    A2 += *(const f32x4*)(smem + G::L_A2P + v * 1024 + lane * 16);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * g + r > c) A2[r] = 0.f;
  const Split4 a2s = split4(A2);
  Zt = mm_pre(cat44(a2s.hi, a2s.lo), g2, Zt);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tl = 4 * g + r;
    const float zr = Zt[r];  // element by value
    if (!SUB || (tl / bsub) == pass)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zr), rz,
                                            (uint32_t)(((tile * 16 + tl) * 64 + 16 * mi + c) * 4), 0, 2);
  }
}

template <int NW, bool SUB>
__global__ void __launch_bounds__(NW * 64) mlp_scan_kernel(MlpArgs a) {
  using G = MlpGeom<NW>;
  constexpr int U = G::U, NB = G::NB, NCH = G::NCH;
  static_assert(NW == 4 || NW == 8, "waves 0..3 each own one 16-column block of d in the reductions");
  __shared__ __attribute__((aligned(16))) char smem[G::L_TOTAL];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x;
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int ntiles = (T + 15) >> 4;
  const int bsub = SUB ? a.b : 16;
  const int npass = 16 / bsub;
  const int u0 = U * w;  // first hidden unit of this wave

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

  // hi/lo splits of fp32 blocks form the residual on the matrix unit
  const NegSel ns = make_negsel(c, g);

  // ---------------------------------------------------------------- state
  const size_t wsel = a.w0_per_batch ? unit : head;
  const float* w1g = a.w1_0 + wsel * HID * 64;
  const float* w2g = a.w2_0 + wsel * 64 * HID;
  f32x4 W1[NB][4];   // [n][m]:  W1[u = u0 + 16n + c][sigma(m, 4g + r)]
  f32x4 W2T[NB][4];  // [nu][mi]: W2[i = 16mi + c][u = u0 + 16nu + 4g + r]
  // W2N block [mi][nu] (W2[i = 16mi + 4g + r][u = u0 + 16nu + c]) lives in LDS
  char* const w2n = smem + G::L_W2N + w * (4 * NB * 1024) + lane * 16;
  auto w2n_at = [&](int mi, int nu) { return (f32x4*)(w2n + (mi * NB + nu) * 1024); };
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      W1[n][m] = *(const f32x4*)(w1g + (u0 + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1));
#pragma unroll
  for (int nu = 0; nu < NB; ++nu)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      W2T[nu][mi] = *(const f32x4*)(w2g + (16 * mi + c) * HID + u0 + 16 * nu + 4 * g);
      f32x4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = w2g[(16 * mi + 4 * g + r) * HID + u0 + 16 * nu + c];
      *w2n_at(mi, nu) = x;  // read back only by this wave
    }

  // ------------------------------------------------------- input staging
  // Chunk q of a tile (q = lane-flat index + NW*64*round): q < 128 a K chunk,
  // q < 256 a Q chunk, q < 384 a V chunk, q < 400 one eta; zero past T.
  const size_t uoff = (size_t)unit * T * 64;
  __amdgpu_buffer_rsrc_t rsrc[G::LOADS];
  int ldst[G::LOADS];
  uint32_t gsrc[G::LOADS], gstep[G::LOADS];
  // The tensor a wave reads depends only on its first chunk (64-chunk
  // blocks never straddle two tensors), so the descriptors are built from a
  // wave-uniform index and stay in scalar registers.
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int l = 0; l < G::LOADS; ++l) {
    const int q0 = wu * 64 + l * NW * 64;  // first chunk of this wave
    const int q = q0 + lane;
    ldst[l] = -1;
    gsrc[l] = 0;
    gstep[l] = 2048;
    if (q0 < 384) {
      const int part = q0 >> 7, ch = q & 127, r = ch >> 3, p = ch & 7;
      const void* base = part == 0 ? a.k : (part == 1 ? a.q : a.v);
      rsrc[l] = make_rsrc((const short*)base + uoff, (uint32_t)T * 128);
      gsrc[l] = r * 128 + p * 16;
      ldst[l] = part * 2048 + (part < 2 ? swz_chunk(r, p) : (int)gsrc[l]);
    } else {
      rsrc[l] = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
      if (q < 400) {
        gsrc[l] = (q - 384) * 4;
        gstep[l] = 64;
        ldst[l] = 3 * 2048 + (q - 384) * 4;
      }
    }
  }
  auto fetch = [&](int j, uint4* v) {
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) {
      v[l] = make_uint4(0, 0, 0, 0);
      if (ldst[l] >= 0 && j < ntiles) {
        const uint32_t off = gsrc[l] + (uint32_t)j * gstep[l];
        if (gstep[l] == 64) v[l].x = __builtin_amdgcn_raw_buffer_load_b32(rsrc[l], off, 0, 0);
        else v[l] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc[l], off, 0, 0));
      }
    }
  };
  auto stash = [&](int j, const uint4* v) {
#pragma unroll
    for (int l = 0; l < G::LOADS; ++l) {
      if (ldst[l] >= 0 && j < ntiles) {
        char* dst = smem + G::L_RAW + (j & 1) * RAWB + ldst[l];
        if (gstep[l] == 64) *(uint32_t*)dst = v[l].x;
        else *(uint4*)dst = v[l];
      }
    }
  };

  const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.z + uoff, (uint32_t)T * 256);

  uint4 pf[G::LOADS];
  fetch(0, pf);
  stash(0, pf);
  fetch(1, pf);
  wg_barrier();

  YOps g2prev;  // Gn2 operands (block mi = w) of the previous pass
  int prev_tile = -1, prev_pass = 0;

  for (int j = 0; j < ntiles; ++j) {
    const char* raw = smem + G::L_RAW + (j & 1) * RAWB;
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
    const f32x4 eta4 = *(const f32x4*)(Et + 4 * g);

    for (int p = 0; p < npass; ++p) {
      // ================= Z of the previous pass, output block mi = w
      if (prev_tile >= 0 && w < 4)
        reduce_store_z<NW, SUB>(smem, lane, c, g, w, g2prev, rz, prev_tile, prev_pass, bsub);

      f32x4 e2;  // 2 eta of this pass's sub-batch
#pragma unroll
      for (int r = 0; r < 4; ++r) e2[r] = (!SUB || (4 * g + r) / bsub == p) ? 2.f * eta4[r] : 0.f;

      // ================= forward at the gradient point; W1 Q for the outputs
      f32x4 Z1[NB], ZQ[NB], D[NB], X2t[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const Split8 s0 = split8_mfma(W1[n][0], W1[n][1], ns), s1 = split8_mfma(W1[n][2], W1[n][3], ns);
        f32x4 z = {0, 0, 0, 0}, zq = {0, 0, 0, 0};
        z = mfma_k32(kop[0], s0.hi, z);
        z = mfma_k32(kop[0], s0.lo, z);
        z = mfma_k32(kop[1], s1.hi, z);
        z = mfma_k32(kop[1], s1.lo, z);
        zq = mfma_k32(qop[0], s0.hi, zq);
        zq = mfma_k32(qop[0], s0.lo, zq);
        zq = mfma_k32(qop[1], s1.hi, zq);
        zq = mfma_k32(qop[1], s1.lo, zq);
        Z1[n] = z;
        ZQ[n] = zq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const GeluOut o = gelu_and_grad(z[r]);
          X2t[n][r] = o.g;  // X2^T[t = 4g+r][u = u0 + 16n + c]
          D[n][r] = o.dg;
        }
      }
      Split4 x2ts[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) x2ts[n] = split4(X2t[n]);
      // X2[u][t] in accumulator layout (u = 4g+r, t = c): operand over u, chunk ch
      // covers blocks 2ch, 2ch+1 (slot 8g + e <-> u = u0 + 32ch + 16(e/4) + 4g + e%4)
      Split8 x2op[NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const f32x4 t0 = mfma_k32(cat44(x2ts[2 * ch].hi, x2ts[2 * ch].lo), itr, f32x4{0, 0, 0, 0});
        const f32x4 t1 = mfma_k32(cat44(x2ts[2 * ch + 1].hi, x2ts[2 * ch + 1].lo), itr, f32x4{0, 0, 0, 0});
        x2op[ch] = split8_mfma(t0, t1, ns);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        f32x4 z2 = {0, 0, 0, 0};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) z2 = mm3(x2op[ch], split8_mfma(W2T[2 * ch][mi], W2T[2 * ch + 1][mi], ns), z2);
        *(f32x4*)(smem + G::L_Z2P + (w * 4 + mi) * 1024 + lane * 16) = z2;  // partial Z2^T[t][i]
      }
      wg_barrier();  // B1: partial Z2 written

      // ================= Gn2 = 2 eta (V - Z2) for output block mi = w
      if (w < 4) {
        const int mi = w;
        f32x4 Z2 = {0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < NW; ++v) Z2 += *(const f32x4*)(smem + G::L_Z2P + (v * 4 + mi) * 1024 + lane * 16);
        Z2 = mfma_k32(*(const bf16x8*)(Vt + c * 128 + (16 * mi + 8 * (g & 1)) * 2), negI, Z2);  // Z2 - V
        f32x4 Gv;
#pragma unroll
        for (int r = 0; r < 4; ++r) Gv[r] = -e2[r] * Z2[r];
        const Split4 gs = split4(Gv);
        *(uint4*)(smem + G::L_G2A + mi * 1024 + lane * 16) = pack_split(gs);
        const f32x4 GT = mfma_k32(cat44(gs.hi, gs.lo), itr, f32x4{0, 0, 0, 0});  // Gn2[i][t]
        *(uint4*)(smem + G::L_G2B + mi * 1024 + lane * 16) = pack_split(split4(GT));
      }
      wg_barrier();  // B2: Gn2 ready

      // ================= backward to layer 1: Gn1^T = (Gn2^T W2) * GELU'(Z1)
      Split4 g2s[4];
      Split8 ga[2];
      {
        Split4 g2t[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          g2s[mi] = unpack_split(*(const uint4*)(smem + G::L_G2A + mi * 1024 + lane * 16));
          g2t[mi] = unpack_split(*(const uint4*)(smem + G::L_G2B + mi * 1024 + lane * 16));
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ga[kb] = Split8{cat44(g2t[2 * kb].hi, g2t[2 * kb + 1].hi), cat44(g2t[2 * kb].lo, g2t[2 * kb + 1].lo)};
      }
      Split4 g1s[NB];
#pragma unroll
      for (int nu = 0; nu < NB; ++nu) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mm3(ga[kb], split8_mfma(*w2n_at(2 * kb, nu), *w2n_at(2 * kb + 1, nu), ns), acc);
        f32x4 g1;
#pragma unroll
        for (int r = 0; r < 4; ++r) g1[r] = acc[r] * D[nu][r];
        g1s[nu] = split4(g1);
      }

      // ================= outputs: Z1q, X2q, partial Z and X2^T X2q
      Split4 x2qs[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const f32x4 z1q = mm_pre(aop, yops(g1s[n]), ZQ[n]);
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = gelu_and_grad(z1q[r]).g;
        x2qs[n] = split4(x);
      }
      Split8 x2qop[NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const f32x4 t0 = mfma_k32(cat44(x2qs[2 * ch].hi, x2qs[2 * ch].lo), itr, f32x4{0, 0, 0, 0});
        const f32x4 t1 = mfma_k32(cat44(x2qs[2 * ch + 1].hi, x2qs[2 * ch + 1].lo), itr, f32x4{0, 0, 0, 0});
        x2qop[ch] = split8_mfma(t0, t1, ns);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        f32x4 zp = {0, 0, 0, 0};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) zp = mm3(x2qop[ch], split8_mfma(W2T[2 * ch][mi], W2T[2 * ch + 1][mi], ns), zp);
        *(f32x4*)(smem + G::L_ZP + (w * 4 + mi) * 1024 + lane * 16) = zp;
      }
      {
        f32x4 a2 = {0, 0, 0, 0};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) a2 = mm3(x2op[ch], x2qop[ch], a2);
        *(f32x4*)(smem + G::L_A2P + w * 1024 + lane * 16) = a2;
      }

      // ================= rank-16 updates of both layers
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 x = mfma_k32(kop[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});  // K[t][sigma(m,c)]
        const uint32_t p0 = pack_rne(x[0], x[1]), p1 = pack_rne(x[2], x[3]);
        const bf16x8 kt2 = __builtin_bit_cast(bf16x8, make_uint4(p0, p1, p0, p1));
#pragma unroll
        for (int n = 0; n < NB; ++n) W1[n][m] = mfma_k32(kt2, cat44(g1s[n].hi, g1s[n].lo), W1[n][m]);
      }
      YOps g2y[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) g2y[mi] = yops(g2s[mi]);
#pragma unroll
      for (int nu = 0; nu < NB; ++nu) {
        const bf16x8 xa = cat44(x2ts[nu].hi, x2ts[nu].lo);
        const YOps xy = yops(x2ts[nu]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          W2T[nu][mi] = mm_pre(xa, g2y[mi], W2T[nu][mi]);                          // += X2 Gn2^T
          *w2n_at(mi, nu) = mm_pre(cat44(g2s[mi].hi, g2s[mi].lo), xy, *w2n_at(mi, nu));  // += Gn2 X2^T
        }
      }
      if (w == 0) g2prev = g2y[0];
      if (w == 1) g2prev = g2y[1];
      if (w == 2) g2prev = g2y[2];
      if (w == 3) g2prev = g2y[3];
      prev_tile = j;
      prev_pass = p;

      if (p == npass - 1) stash(j + 1, pf);  // next tile's inputs into the other slot
      wg_barrier();  // B0: partials of this pass and the next tile's inputs ready
    }
    fetch(j + 2, pf);
  }

  if (prev_tile >= 0 && w < 4)
    reduce_store_z<NW, SUB>(smem, lane, c, g, w, g2prev, rz, prev_tile, prev_pass, bsub);

  // final state
  float* w1o = a.w1_out + (size_t)unit * HID * 64;
  float* w2o = a.w2_out + (size_t)unit * 64 * HID;
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *(f32x4*)(w1o + (u0 + 16 * n + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) = W1[n][m];
#pragma unroll
  for (int nu = 0; nu < NB; ++nu)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      *(f32x4*)(w2o + (16 * mi + c) * HID + u0 + 16 * nu + 4 * g) = W2T[nu][mi];
}

}  // namespace

hipError_t launch_mlp(const MlpArgs& a, bool f32in, hipStream_t s) {
  constexpr int NW = 4;
  if (f32in || a.b > 16) return hipErrorNotSupported;
  if (a.b == 16)
    hipLaunchKernelGGL((mlp_scan_kernel<2 * NW, false>), dim3(a.units), dim3(2 * NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_scan_kernel<NW, true>), dim3(a.units), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
