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
// For training, a variant also stores the state before every mini-batch
// (the checkpoints of §6.12), straight from the registers.
//
// LayerNorm + residual variant (§4.4 wrapper, f(x) = x + LN(W2 GELU(W1 x)),
// LN over the d = 64 outputs of one token with gamma, beta per head): with
// Y = Z2 at the gradient point, rs = 1 / sqrt(var_i Y + eps), Yh = (Y - mean) rs
// and g = 2 gamma (K + gamma Yh + beta - V) (the loss gradient at Yh),
//   Gn2 = -rs (g - mean_i g - Yh mean_i (g Yh)) diag(eta)
// replaces the plain -2 (Z2 - V) diag(eta), and every output is
// z = q + gamma LN-hat(Z) + beta.  The per-token sums over i cross the four
// reducing waves through LDS: (sum Y, sum Y^2), then (sum g, sum g Yh), each
// behind a workgroup barrier, and the output's (sum Z, sum Z^2) behind the
// next tile's first barrier, off the recurrence.  The variance is the
// one-pass E[Y^2] - mean^2, clamped at 0.  K - V and q enter the
// accumulator layout exactly, as one-hot MFMA selections of the bf16 tiles.
//
// Inputs are register-staged one tile ahead by the waves themselves (each
// lane moves 16-byte chunks of K, Q, V or one eta), so no wave issues
// LDS-DMA and no wave is idle.  Mini-batches b < 16 (b | 16) run each
// sub-batch of a tile as its own pass with eta masked to that sub-batch.
#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_mlp_ops.h"

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
  // LayerNorm sums: 3 areas (Y, the VJP, the outputs) x 2 values x [mi][t]
  static constexpr int L_ST = L_W2N + NW * 4 * NB * 1024;
  static constexpr int L_TOTAL = L_ST + 3 * 512;
  static constexpr int LOADS = (400 + NW * 64 - 1) / (NW * 64);  // staged chunks per lane
};

// Sum of the NW partial blocks of a cross-wave reduction: the Z of one pass
// for output block mi (before the LayerNorm of the wrapped variant),
// Z^T = sum partials + triu(sum A2)^T Gn2^T.
template <int NW>
__device__ __forceinline__ f32x4 reduce_z(const char* smem, int lane, int c, int g, int mi,
                                          const YOps& g2) {
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
  return mm_pre(cat44(a2s.hi, a2s.lo), g2, Zt);
}
// Store output block mi of one pass: lane (c, g) holds Z[t = 4g + r][16 mi + c]
template <bool SUB>
__device__ __forceinline__ void store_z(f32x4 Zt, int c, int g, int mi, __amdgpu_buffer_rsrc_t rz,
                                        int tile, int pass, int bsub) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tl = 4 * g + r;
    const float zr = Zt[r];  // element by value
    if (!SUB || (tl / bsub) == pass)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zr), rz,
                                            (uint32_t)(((tile * 16 + tl) * 64 + 16 * mi + c) * 4), 0, 2);
  }
}

// LayerNorm sums over i of one output block: lane (c, g) holds x[t = 4g + r]
// at i = 16 mi + c; the row of 16 lanes sums to the block's total for its 4
// tokens, which lane c = 0 leaves in LDS (area [2][mi][16 t] floats).
__device__ __forceinline__ void ln_put(char* area, int mi, int c, int g, f32x4 x, f32x4 y) {
  f32x4 sx, sy;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sx[r] = row_sum16(x[r]);
    sy[r] = row_sum16(y[r]);
  }
  if (c == 0) {
    *(f32x4*)(area + (mi * 16 + 4 * g) * 4) = sx;
    *(f32x4*)(area + 256 + (mi * 16 + 4 * g) * 4) = sy;
  }
}
// Totals over the four blocks (fixed order) for tokens 4g .. 4g + 3.
__device__ __forceinline__ void ln_get(const char* area, int g, f32x4& sx, f32x4& sy) {
  sx = f32x4{0, 0, 0, 0};
  sy = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    sx += *(const f32x4*)(area + (mi * 16 + 4 * g) * 4);
    sy += *(const f32x4*)(area + 256 + (mi * 16 + 4 * g) * 4);
  }
}

// CKPT: also store the state before every mini-batch (W1 [256][64] and W2
// [64][256] per unit and mini-batch, the layouts of the final state) for the
// backward; the stores are fire-and-forget and leave the recurrence alone.
// LN: the LayerNorm + residual wrapper (gamma, beta, eps from the arguments).
// HOLD: mini-batches of b = 16 tpm tokens (tpm > 1): the gradients of all
// tpm tiles of a mini-batch are taken at the state W0 of its start, the
// outputs and updates use the running state (in the dual form the output of
// token t is W_cur q_t plus the in-tile triangular term, W_cur holding the
// earlier tiles' updates).  At each mini-batch start the bf16 hi/lo operands
// of W1 go into this wave's LDS area (the W2 copy with i on the rows is not
// kept: nothing else needs it), and W2 into the final-state output (this
// wave's columns, in its layout; the final state overwrites it at the end),
// read back where its products need it, by the lane that wrote it; W2 with i
// on the rows comes from MFMA transposes of those blocks.
template <int NW, bool SUB, bool CKPT = false, bool LN = false, bool HOLD = false>
__global__ void __launch_bounds__(NW * 64) mlp_scan_kernel(MlpLnArgs la) {
  using G = MlpGeom<NW>;
  const MlpArgs& a = la.s;
  constexpr int U = G::U, NB = G::NB, NCH = G::NCH;
  static_assert(NW == 4 || NW == 8, "waves 0..3 each own one 16-column block of d in the reductions");
  static_assert(!HOLD || (NW == 8 && !SUB), "held gradient point: the 8-wave variant");
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
  const int tpm = HOLD ? a.b / 16 : 1;  // tiles per mini-batch
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
  // LayerNorm wrapper: gamma, beta of output i = 16 (w % 4) + c
  float lg = 0.f, lb = 0.f;
  if constexpr (LN) {
    lg = la.gamma[head * 64 + 16 * (w & 3) + c];
    lb = la.beta[head * 64 + 16 * (w & 3) + c];
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
      if constexpr (!HOLD) {
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = w2g[(16 * mi + 4 * g + r) * HID + u0 + 16 * nu + c];
        *w2n_at(mi, nu) = x;  // read back only by this wave
      }
    }
  // HOLD: the gradient point's W2 blocks, read back by the lane that wrote them
  float* const h2 = a.w2_out + (size_t)unit * 64 * HID;
  auto w2_held = [&](int nu, int mi) {  // W2[16 mi + c][u0 + 16 nu + 4g + r]
    return *(const f32x4*)(h2 + (16 * mi + c) * HID + u0 + 16 * nu + 4 * g);
  };

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

  // Outputs.  Block mi = w % 4 of the previous pass's Z goes out from waves
  // OUT0 .. OUT0 + 3 at the start of the next pass; in the wrapped variant
  // with 8 waves (LATE) from waves 4..7 between its first two barriers,
  // where they would otherwise wait for the gradient, taking the Gn2
  // operands from LDS rather than holding them through the forward.
  constexpr bool LATE = LN && NW == 8;
  constexpr int OUT0 = LATE ? 4 : 0;
  const bool outw = w >= OUT0 && w < OUT0 + 4;
  const int omi = w & 3;
  YOps g2prev;  // Gn2 operands (block omi) of the previous pass
  int prev_tile = -1, prev_pass = 0;
  // first stage: the plain variant stores the block; the wrapped one leaves
  // its LayerNorm sums in LDS and reads -q while the tile is in the ring
  auto out_first = [&](int tile, int pass, f32x4& zo, f32x4& qn) {
    if constexpr (LATE)
      zo = reduce_z<NW>(smem, lane, c, g, omi,
                        yops(unpack_split(*(const uint4*)(smem + G::L_G2A + omi * 1024 + lane * 16))));
    else
      zo = reduce_z<NW>(smem, lane, c, g, omi, g2prev);
    if constexpr (LN) {
      const char* Qp = smem + G::L_RAW + (tile & 1) * RAWB + 2048;
      qn = mfma_k32(*(const bf16x8*)(Qp + swz_chunk(c, 2 * omi + (g & 1))), negI, f32x4{0, 0, 0, 0});
      f32x4 z2;
#pragma unroll
      for (int r = 0; r < 4; ++r) z2[r] = zo[r] * zo[r];
      ln_put(smem + G::L_ST + 2 * 512, omi, c, g, zo, z2);
    } else {
      store_z<SUB>(zo, c, g, omi, rz, tile, pass, bsub);
    }
  };
  // second stage (wrapped, after a barrier): z = q + gamma LN-hat(Z) + beta
  auto out_second = [&](int tile, int pass, f32x4 zo, f32x4 qn) {
    f32x4 s1, s2, zr;
    ln_get(smem + G::L_ST + 2 * 512, g, s1, s2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mu = s1[r] * (1.f / 64);
      const float ro = rsqrtf(fmaxf(fmaf(s2[r], 1.f / 64, -mu * mu), 0.f) + la.eps);
      zr[r] = fmaf(lg, (zo[r] - mu) * ro, lb) - qn[r];
    }
    store_z<SUB>(zr, c, g, omi, rz, tile, pass, bsub);
  };
  const int nmb = HOLD ? (T + a.b - 1) / a.b : (T + bsub - 1) / bsub;  // mini-batches (checkpoints)
  // this wave's rows of W1 and columns of W2 (W1 [256][64], W2 [64][256], the
  // layouts of the final state)
  auto store_state = [&](float* w1o, float* w2o) {
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
  };
  // the same for the checkpoint of mini-batch mb: nontemporal buffer stores
  // through descriptors built in scalar registers, the lane's part of the
  // offsets loop-invariant, so that a burst of them needs no vector
  // registers beyond the state (an address spilled around the burst would be
  // reloaded behind all of its stores: the memory counter is in order).  The
  // stores are issued for every pass, those past the last mini-batch through
  // an empty descriptor (dropped by the hardware): with the same instruction
  // count on every path the compiler's wait for the next tile's inputs leaves
  // them in flight, instead of waiting for them all.  A pass issues them in
  // four quarters (every other block of W1, then of W2) at four points
  // before the update: a burst of all of them at once stalls the issuing
  // waves on the memory unit's queue.
  const uint32_t w1off = CKPT ? (uint32_t)(((u0 + c) * 64 + 8 * g) * 4) : 0u;
  const uint32_t w2off = CKPT ? (uint32_t)((c * HID + u0 + 4 * g) * 4) : 0u;
  auto store_ckpt = [&](int mb, int quarter) {
    typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
    const bool in = mb < nmb;
    const size_t co = ((size_t)unit * nmb + (in ? mb : 0)) * HID * 64;
    if (quarter < 2) {  // W1 blocks n = quarter, quarter + 2, ...
      const __amdgpu_buffer_rsrc_t r1 = make_rsrc(a.w1_ckpt + co, in ? HID * 64 * 4 : 0u);
#pragma unroll
      for (int n = quarter; n < NB; n += 2)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, W1[n][m]), r1,
                                                 w1off + (uint32_t)((16 * n * 64 + 32 * (m >> 1) + 4 * (m & 1)) * 4),
                                                 0, 2);
    } else {  // W2 blocks nu = quarter - 2, quarter, ...
      const __amdgpu_buffer_rsrc_t r2 = make_rsrc(a.w2_ckpt + co, in ? HID * 64 * 4 : 0u);
#pragma unroll
      for (int nu = quarter - 2; nu < NB; nu += 2)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, W2T[nu][mi]), r2,
                                                 w2off + (uint32_t)((16 * mi * HID + 16 * nu) * 4), 0, 2);
    }
  };

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
      // mini-batch starting at token 16 j + bsub p (HOLD: at tile j, if any;
      // nmb, an empty checkpoint, otherwise)
      const int mb = HOLD ? (j % tpm == 0 ? j / tpm : nmb) : j * npass + p;
      if constexpr (HOLD)
        if (j % tpm == 0) {  // the gradient point's W2
#pragma unroll
          for (int nu = 0; nu < NB; ++nu)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
              *(f32x4*)(h2 + (16 * mi + c) * HID + u0 + 16 * nu + 4 * g) = W2T[nu][mi];
        }
      if constexpr (CKPT) store_ckpt(mb, 0);
      // ================= Z of the previous pass (4 waves: now; the wrapped
      // variant normalises after B2, holding Z and q)
      f32x4 zo = {0, 0, 0, 0}, qn = {0, 0, 0, 0};
      const int out_tile = prev_tile, out_pass = prev_pass;
      if constexpr (!LATE)
        if (out_tile >= 0 && outw) out_first(out_tile, out_pass, zo, qn);

      f32x4 e2;  // 2 eta of this pass's sub-batch
#pragma unroll
      for (int r = 0; r < 4; ++r) e2[r] = (!SUB || (4 * g + r) / bsub == p) ? 2.f * eta4[r] : 0.f;

      // ================= forward at the gradient point; W1 Q for the outputs
      f32x4 Z1[NB], ZQ[NB], D[NB], X2t[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const Split8 s0 = split8_mfma(W1[n][0], W1[n][1], ns), s1 = split8_mfma(W1[n][2], W1[n][3], ns);
        f32x4 z = {0, 0, 0, 0}, zq = {0, 0, 0, 0};
        if constexpr (HOLD) {  // W1's operands at the gradient point, [n][s0 hi, lo, s1 hi, lo][lane]
          char* const hb = w2n + n * 4096;
          if (j % tpm == 0) {
            *(bf16x8*)hb = s0.hi;
            *(bf16x8*)(hb + 1024) = s0.lo;
            *(bf16x8*)(hb + 2048) = s1.hi;
            *(bf16x8*)(hb + 3072) = s1.lo;
          }
          const Split8 t0{*(const bf16x8*)hb, *(const bf16x8*)(hb + 1024)};
          const Split8 t1{*(const bf16x8*)(hb + 2048), *(const bf16x8*)(hb + 3072)};
          z = mfma_k32(kop[0], t0.hi, z);
          z = mfma_k32(kop[0], t0.lo, z);
          z = mfma_k32(kop[1], t1.hi, z);
          z = mfma_k32(kop[1], t1.lo, z);
        } else {
          z = mfma_k32(kop[0], s0.hi, z);
          z = mfma_k32(kop[0], s0.lo, z);
          z = mfma_k32(kop[1], s1.hi, z);
          z = mfma_k32(kop[1], s1.lo, z);
        }
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
      Split8 w2s[4][NCH];  // hi/lo of W2 at the gradient point: Z2 and the outputs
      if constexpr (!HOLD) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) w2s[mi][ch] = split8_mfma(W2T[2 * ch][mi], W2T[2 * ch + 1][mi], ns);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        f32x4 z2 = {0, 0, 0, 0};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          if constexpr (HOLD)
            z2 = mm3(x2op[ch], split8_mfma(w2_held(2 * ch, mi), w2_held(2 * ch + 1, mi), ns), z2);
          else
            z2 = mm3(x2op[ch], w2s[mi][ch], z2);
        }
        *(f32x4*)(smem + G::L_Z2P + (w * 4 + mi) * 1024 + lane * 16) = z2;  // partial Z2^T[t][i]
      }
      wg_barrier();  // B1: partial Z2 written
      if constexpr (CKPT) store_ckpt(mb, 1);

      // ================= LATE: the previous pass's Z from waves 4..7
      if constexpr (LATE)
        if (out_tile >= 0 && outw) out_first(out_tile, out_pass, zo, qn);

      // ================= Gn2 = 2 eta (V - Z2) for output block mi = w
      // (wrapped variant: the LayerNorm VJP, two rounds of sums over i)
      // (LATE: waves 0..3 keep Y and K - V in the registers that waves 4..7
      // use for the previous Z and -q, so the two roles share them)
      f32x4 Z2v = {0, 0, 0, 0}, KVv = {0, 0, 0, 0};
      f32x4& Z2 = LATE ? zo : Z2v;
      f32x4& KV = LATE ? qn : KVv;
      if (w < 4) {
        const int mi = w;
#pragma unroll
        for (int v = 0; v < NW; ++v) Z2 += *(const f32x4*)(smem + G::L_Z2P + (v * 4 + mi) * 1024 + lane * 16);
        const bf16x8 vch = *(const bf16x8*)(Vt + c * 128 + (16 * mi + 8 * (g & 1)) * 2);
        if constexpr (LN) {
          KV = mfma_k32(*(const bf16x8*)(Kt + swz_chunk(c, 2 * mi + (g & 1))), negI, KV);  // -K
#pragma unroll
          for (int r = 0; r < 4; ++r) KV[r] = -KV[r];
          KV = mfma_k32(vch, negI, KV);  // K - V
          f32x4 y2;
#pragma unroll
          for (int r = 0; r < 4; ++r) y2[r] = Z2[r] * Z2[r];
          ln_put(smem + G::L_ST, mi, c, g, Z2, y2);
        } else {
          Z2 = mfma_k32(vch, negI, Z2);  // Z2 - V
        }
      }
      f32x4 rs, yh, gv;
      if constexpr (LN) {
        wg_barrier();  // sums of Y (and of the previous pass's Z)
        if constexpr (LATE)
          if (out_tile >= 0 && outw) out_second(out_tile, out_pass, zo, qn);
        if (w < 4) {
          f32x4 s1, s2;
          ln_get(smem + G::L_ST, g, s1, s2);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float mu = s1[r] * (1.f / 64);
            rs[r] = rsqrtf(fmaxf(fmaf(s2[r], 1.f / 64, -mu * mu), 0.f) + la.eps);
            yh[r] = (Z2[r] - mu) * rs[r];
            gv[r] = 2.f * lg * (KV[r] + fmaf(lg, yh[r], lb));
          }
          f32x4 gy;
#pragma unroll
          for (int r = 0; r < 4; ++r) gy[r] = gv[r] * yh[r];
          ln_put(smem + G::L_ST + 512, w, c, g, gv, gy);
        }
        wg_barrier();  // sums of the VJP
      }
      if (w < 4) {
        const int mi = w;
        f32x4 Gv;
        if constexpr (LN) {
          f32x4 m1, m2;
          ln_get(smem + G::L_ST + 512, g, m1, m2);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Gv[r] = -0.5f * e2[r] * rs[r] * (gv[r] - m1[r] * (1.f / 64) - yh[r] * m2[r] * (1.f / 64));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) Gv[r] = -e2[r] * Z2[r];
        }
        const Split4 gs = split4(Gv);
        *(uint4*)(smem + G::L_G2A + mi * 1024 + lane * 16) = pack_split(gs);
        const f32x4 GT = mfma_k32(cat44(gs.hi, gs.lo), itr, f32x4{0, 0, 0, 0});  // Gn2[i][t]
        *(uint4*)(smem + G::L_G2B + mi * 1024 + lane * 16) = pack_split(split4(GT));
      }
      wg_barrier();  // B2: Gn2 ready
      if constexpr (CKPT) store_ckpt(mb, 2);
      if constexpr (LN && !LATE)
        if (out_tile >= 0 && outw) out_second(out_tile, out_pass, zo, qn);

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
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (HOLD)  // W2 with i on the rows: transposes of the held blocks
            acc = mm3(ga[kb],
                      split8_mfma(transpose16(w2_held(nu, 2 * kb), itr), transpose16(w2_held(nu, 2 * kb + 1), itr), ns),
                      acc);
          else
            acc = mm3(ga[kb], split8_mfma(*w2n_at(2 * kb, nu), *w2n_at(2 * kb + 1, nu), ns), acc);
        }
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
        for (int ch = 0; ch < NCH; ++ch) {
          if constexpr (LN || HOLD)  // split again: not held through the LayerNorm rounds; HOLD:
            // the running state, not the gradient point
            zp = mm3(x2qop[ch], split8_mfma(W2T[2 * ch][mi], W2T[2 * ch + 1][mi], ns), zp);
          else
            zp = mm3(x2qop[ch], w2s[mi][ch], zp);
        }
        *(f32x4*)(smem + G::L_ZP + (w * 4 + mi) * 1024 + lane * 16) = zp;
      }
      {
        f32x4 a2 = {0, 0, 0, 0};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) a2 = mm3(x2op[ch], x2qop[ch], a2);
        *(f32x4*)(smem + G::L_A2P + w * 1024 + lane * 16) = a2;
      }

      // ================= rank-16 updates of both layers
      if constexpr (CKPT) store_ckpt(mb, 3);
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
          W2T[nu][mi] = mm_pre(xa, g2y[mi], W2T[nu][mi]);  // += X2 Gn2^T
          if constexpr (!HOLD)
            *w2n_at(mi, nu) = mm_pre(cat44(g2s[mi].hi, g2s[mi].lo), xy, *w2n_at(mi, nu));  // += Gn2 X2^T
        }
      }
      if constexpr (!LATE) {  // the output waves are 0..3
        if (w == 0) g2prev = g2y[0];
        if (w == 1) g2prev = g2y[1];
        if (w == 2) g2prev = g2y[2];
        if (w == 3) g2prev = g2y[3];
      }
      prev_tile = j;
      prev_pass = p;

      if (p == npass - 1) stash(j + 1, pf);  // next tile's inputs into the other slot
      wg_barrier();  // B0: partials of this pass and the next tile's inputs ready
    }
    fetch(j + 2, pf);
  }

  // the last pass's outputs (prev_tile is the same in every wave)
  f32x4 zo = {0, 0, 0, 0}, qn = {0, 0, 0, 0};
  if (prev_tile >= 0 && outw) out_first(prev_tile, prev_pass, zo, qn);
  if constexpr (LN) {
    wg_barrier();  // the output sums
    if (prev_tile >= 0 && outw) out_second(prev_tile, prev_pass, zo, qn);
  }

  store_state(a.w1_out + (size_t)unit * HID * 64, a.w2_out + (size_t)unit * 64 * HID);  // final state
}

}  // namespace

hipError_t launch_mlp(const MlpArgs& a, bool f32in, hipStream_t s) {
  constexpr int NW = 4;
  // fp32 inputs: the primal kernel
  if (f32in || (a.b > 16 && a.b % 16 != 0)) return launch_mlp_primal(a, f32in, s);
  const MlpLnArgs la{a, nullptr, nullptr, 0.f};
  if (a.b > 16) {  // mini-batches of several tiles: the gradient point held in memory
    if (a.w1_ckpt)
      return launch(mlp_scan_kernel<2 * NW, false, true, false, true>, dim3(a.units), dim3(2 * NW * 64), s, la);
    return launch(mlp_scan_kernel<2 * NW, false, false, false, true>, dim3(a.units), dim3(2 * NW * 64), s, la);
  }
  if (a.w1_ckpt) {
    if (a.b == 16) return launch(mlp_scan_kernel<2 * NW, false, true>, dim3(a.units), dim3(2 * NW * 64), s, la);
    return launch(mlp_scan_kernel<NW, true, true>, dim3(a.units), dim3(NW * 64), s, la);
  }
  if (a.b == 16) return launch(mlp_scan_kernel<2 * NW, false>, dim3(a.units), dim3(2 * NW * 64), s, la);
  return launch(mlp_scan_kernel<NW, true>, dim3(a.units), dim3(NW * 64), s, la);
}

hipError_t launch_mlp_ln(const MlpLnArgs& a, bool f32in, hipStream_t s) {
  constexpr int NW = 4;
  if (f32in || (a.s.b > 16 && a.s.b % 16 != 0)) return launch_mlp_ln_primal(a, f32in, s);
  if (a.s.b > 16)  // mini-batches of several tiles: the gradient point held in memory
    return launch(mlp_scan_kernel<2 * NW, false, false, true, true>, dim3(a.s.units), dim3(2 * NW * 64), s, a);
  if (a.s.b == 16)
    return launch(mlp_scan_kernel<2 * NW, false, false, true>, dim3(a.s.units), dim3(2 * NW * 64), s, a);
  return launch(mlp_scan_kernel<NW, true, false, true>, dim3(a.s.units), dim3(NW * 64), s, a);
}

}  // namespace ttt
