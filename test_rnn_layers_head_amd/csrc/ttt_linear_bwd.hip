// Backward of the TTT-Linear scan (b | 16), gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): training differentiates through the inner loop;
// the forward keeps the state at the start of every mini-batch (the
// kappa = T / b checkpoints of §6.12) and the backward walks the mini-batches
// in reverse.  Per mini-batch (columns are tokens, D = diag(eta), W the
// checkpointed state, A = triu(K^T Q) with s <= t, §3.6):
//   forward   E = W K - V, G = 2 E D, Z = W Q - G A, W' = W - G K^T
//   backward  (Zb, Wb' the adjoints of Z and W'; Gn = Wb' K + Zb A^T is
//             minus the adjoint of G)
//     Gt = 2 Gn D                      (= dL/dV, and -dL/dE)
//     Wb = Wb' + Zb Q^T - Gt K^T       (the adjoint of W)
//     Ab = triu(-G^T Zb)
//     dQ = W^T Zb + K Ab
//     dK = -W^T Gt + Q Ab^T - Wb'^T G
//     deta_t = -sum_i Gn[i, t] 2 E[i, t]
//
// One workgroup per (batch, head) unit, nine waves.  For each 16-row slice s
// of the adjoint state Wb (its rows evolve independently, like the
// forward's) a chain wave (s) and an output wave (s + 4), which share a
// SIMD, so each hides the other's latencies:
//   chain wave, tile i:   Wb (MFMA accumulators) -> Wb' K + Zb A^T with rows
//       in lanes -> Gt -> dV and the update Wb += [Q | -K] [Zb | Gt]^T; the
//       same with tokens in lanes -> Gn; and Wb' with columns in lanes.  Gn
//       and that copy of Wb' go to the output wave through LDS.
//   output wave, tile i-1: E = W K - V from the slice's rows of the
//       checkpoint (read from HBM two tiles ahead), G, and the partial sums
//       over the slice's rows of dQ, dK, Ab and deta, into LDS.
//   chain wave, tile i-2: adds the four slices' partials for 16 columns,
//       applies K Ab and Q Ab^T, writes dQ, dK (slice 0 also deta).
// The ninth wave streams K, Q, V and eta in reverse order into an LDS ring
// by buffer->LDS DMA (a wave that also read LDS would have to wait for its
// own DMA before every read); dz is read by each wave straight into
// registers two tiles ahead.  One barrier per tile.  The chain and output
// waves run the same branch-free body for all ntiles + 2 iterations:
// iterations outside the sequence see zero inputs (their loads fall outside
// the buffer descriptors), which leave the state unchanged, and their stores
// fall outside the outputs; so every iteration issues the same memory
// operations and the compiler's wait counts stay exact.  Mini-batches of
// b < 16 tokens each take a tile of their own, rows b..15 of which read as
// zero tokens (eta = 0, so they leave the state and every other token's
// outputs unchanged) and drop their outputs the same way.  The adjoint state
// never leaves the chip.
//
// Mini-batches of b = 16 n tokens (n > 1, HOLD): every gradient of a
// mini-batch is taken at its start state W0 (§3.5), so each 16-token tile t
// has E = W0 K - V, G = 2 E D, Z = W_t Q - G A, W_{t+1} = W_t - G K^T with
// W_t the running state.  Backward per tile, Wb' the adjoint of W_{t+1}:
//   Gn, Gt, Ab, dV and deta as above;  dQ = W_t^T Zb + K Ab;
//   dK = -W0^T Gt + Q Ab^T - Wb'^T G;  Wb = Wb' + Zb Q^T, and -Gt K^T goes
//   to the gradient point's adjoint H, added to Wb at the mini-batch start.
// The chain waves keep H in four more accumulators.  The output waves need
// W_t for dQ: they rebuild it in reverse, W_t = W_{t+1} + G K^T with the
// tile's own G, restarting from the exact checkpoint at every mini-batch
// start (the state the next tile in reverse order ends with); the last
// mini-batch starts from W_T = W0 - sum G K^T over its tiles, formed before
// the loop.  The checkpoints are one per mini-batch.
//
// Products: 16x16x32 bf16 MFMA with fp32 accumulation.  K, Q, V are exact in
// bf16; fp32 operands (states, dz, A, G, Gt, Ab) enter as hi + lo bf16 pairs
// and the three significant products (hi*hi, hi*lo, lo*hi) are kept, about
// 2^-16 relative per product.  Transposed copies (Q, K and the two states
// with columns in lanes) come from one-hot selection MFMAs, which are exact.
//
// 16x16x32 bf16 layouts (wave64, lane (c, g), c = lane % 16, g = lane / 16):
// A lane holds A[c][8g .. 8g + 7], B lane holds B[8g .. 8g + 7][c],
// accumulator register r holds C[4g + r][c].  Contractions over the 16
// tokens (or 16 rows) of a lane's registers use the slots of lane group g as
// [4 values hi | the same 4 values lo], both operands alike.
// The state accumulators hold columns in the permuted order
// sigma(m, 4g + r) = 32 (m >> 1) + 8g + 4 (m & 1) + r, so that the hi/lo
// split of blocks 2h, 2h + 1 is operand chunk h in natural column order.
#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_linear_ops.h"

namespace ttt {
namespace {

struct BwdGeom {
  static constexpr int KB = 16 * 64 * 2;          // K, Q or V tile: bf16 [token][col], swizzled
  static constexpr int SLOT = 3 * KB + 64;        // + eta
  static constexpr int NI = 2 + 2 + 2 + 1;        // DMA ops per tile
  static constexpr int D = 3;                     // tiles in flight
  static constexpr int NST = D + 2;               // tile i is read until iteration i + 1
  // partial sums of one output wave: dQ, dK fragments (4 blocks), Ab, deta
  static constexpr int RQ = 4 * 64 * 16;
  static constexpr int RA = 64 * 16;
  static constexpr int RW = 2 * RQ + RA + 256;
  // chain -> output hand-over per slice: Gn (16 B) and Wb' hi/lo (64 B) per lane
  static constexpr int HO = 64 * 80;
  static constexpr int RING = NST * SLOT;
  static constexpr int RED = RING;                // 2 buffers x 4 slices x RW
  static constexpr int HOB = RED + 2 * 4 * RW;    // 2 buffers x 4 slices x HO
  static constexpr int LDS = HOB + 2 * 4 * HO;
  static constexpr int THREADS = 9 * 64;        // + the DMA wave
};

// column of block m, position p (0..15) of the state accumulators
__device__ __forceinline__ int scol(int m, int p) {
  return 32 * (m >> 1) + 8 * (p >> 2) + 4 * (m & 1) + (p & 3);
}

__device__ __forceinline__ uint2 pack4(f32x4 x) {
  return make_uint2(pack_rne(x[0], x[1]), pack_rne(x[2], x[3]));
}

__device__ __forceinline__ f32x4 bf4(uint2 u) {
  return f32x4{__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
               __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u)};
}

template <bool HOLD>
__global__ void __launch_bounds__(BwdGeom::THREADS) linear_bwd_kernel(LinearBwdArgs a) {
  using G = BwdGeom;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int s = wave & 3;  // rows 16 s .. 16 s + 15
  const int unit = blockIdx.x;
  const int T = a.T, bt = a.bt, ntiles = (T + bt - 1) / bt;
  const int niter = ntiles + 2;  // iteration k: chain tile k, outputs of tile k-1, finalize of k-2
  const size_t uoff = (size_t)unit * T * 64;
  if (ntiles == 0) {  // no tokens: dW0 = dW_T (or 0); w_ckpt may be NULL
    if (wave < 4) {
      const float* dwT = a.dw_T ? a.dw_T + (size_t)unit * a.dw_stride + (16 * wave + c) * 64 : nullptr;
      float* o = a.dw0 ? a.dw0 + (size_t)unit * a.dw0_stride + (16 * wave + c) * 64 : nullptr;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (o) *(f32x4*)(o + 16 * m + 4 * g) = dwT ? *(const f32x4*)(dwT + 16 * m + 4 * g) : f32x4{0, 0, 0, 0};
    }
    return;
  }
  const s16x4 z4 = {0, 0, 0, 0};
  const __amdgpu_buffer_rsrc_t rdz = make_rsrc(a.dz + uoff, (uint32_t)T * 256);
  // iteration-order tile k covers tokens bt (ntiles - 1 - k) ..; tiles past
  // either end read as zeros (their offsets fall outside the descriptors),
  // and so do rows r >= bt (token T: just past every descriptor)
  auto tok0 = [&](int k) { return (ntiles - 1 - k) * bt; };
  auto tk = [&](int t0, int r) { return r < bt ? t0 + r : T; };
  // one-hot selectors: B operand that picks column scol(m, c) out of a
  // natural-order chunk, for m even (sel[0]) and odd (sel[1])
  bf16x8 sel[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sel[p][e] = (bf16)((g == (c >> 2) && e == 4 * p + (c & 3)) ? 1.f : 0.f);

  if (wave < 4) {  // ====================================================== chain
    // (with tok_out == 0 the descriptors hold no records: the stores are dropped)
    const uint32_t ot = a.tok_out ? (uint32_t)T : 0u;
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc(a.dq + uoff, ot * 256);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(a.dk + uoff, ot * 256);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(a.dv + uoff, ot * 256);
    const __amdgpu_buffer_rsrc_t rde = make_rsrc(a.deta + (size_t)unit * T, ot * 4);
    auto st32 = [](float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    };
    // Wr[m] register r = Wb[row 16 s + c][scol(m, 4g + r)]
    f32x4 Wr[4], Hr[4];  // Hr: the gradient point's adjoint (HOLD)
#pragma unroll
    for (int m = 0; m < 4; ++m) Hr[m] = f32x4{0, 0, 0, 0};
    {
      const float* dwT = a.dw_T ? a.dw_T + (size_t)unit * a.dw_stride + (16 * s + c) * 64 : nullptr;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        Wr[m] = dwT ? *(const f32x4*)(dwT + scol(m, 4 * g)) : f32x4{0, 0, 0, 0};
    }
    // Zb with rows in lanes: register r = Zb[row 16s + c][t = 4g + r] of tile k
    auto zload = [&](int k, f32x4& z) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        z[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                   rdz, (uint32_t)(tk(tok0(k), 4 * g + r) * 64 + 16 * s + c) * 4, 0, 0));
    };
    // Sums the four slices' partials of one tile for column block s and
    // writes dQ, dK (slice 0 also deta).  q4p, k4p: Q, K of that tile at
    // columns scol(s, c), tokens 4g .. 4g + 3.
    auto finalize = [&](int buf, uint2 q4p, uint2 k4p, int t0) {
      const char* rb = smem + G::RED + buf * 4 * G::RW;
      f32x4 dq = {0, 0, 0, 0}, dk = {0, 0, 0, 0}, ab1 = {0, 0, 0, 0}, ab2 = {0, 0, 0, 0};
      float de = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const char* rw = rb + w * G::RW;
        const f32x4 x = *(const f32x4*)(rw + (s * 64 + lane) * 16);
        const f32x4 y = *(const f32x4*)(rw + G::RQ + (s * 64 + lane) * 16);
        const f32x4 z = *(const f32x4*)(rw + 2 * G::RQ + lane * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dq[r] += x[r];
          dk[r] += y[r];
          ab1[r] += z[r];
          // transposed read: element (s' = c, t = 4g + r)
          ab2[r] += *(const float*)(rw + 2 * G::RQ + ((4 * g + r + 16 * (c >> 2)) * 16 + (c & 3) * 4));
        }
        de += ((const float*)(rw + 2 * G::RQ + G::RA))[c];
      }
      // Ab = triu(-sum): ab1 register r = Ab[s' = 4g + r][t = c], ab2 = Ab[s' = c][t = 4g + r]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ab1[r] = (4 * g + r <= c) ? -ab1[r] : 0.f;
        ab2[r] = (c <= 4 * g + r) ? -ab2[r] : 0.f;
      }
      const Split4 a1 = split4(ab1), a2 = split4(ab2);
      dq = mfma_k32(cat44(a1.hi, a1.lo), cat8(k4p, k4p), dq);  // + K Ab
      dk = mfma_k32(cat44(a2.hi, a2.lo), cat8(q4p, q4p), dk);  // + Q Ab^T
      const int col = scol(s, c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t off = (uint32_t)(tk(t0, 4 * g + r) * 64 + col) * 4;
        const float vq = dq[r], vk = dk[r];  // scalar copies: bit_cast of an element reads element 0
        st32(vq, rdq, off);
        st32(vk, rdk, off);
      }
      st32(de, rde, (s == 0 && g == 0) ? (uint32_t)tk(t0, c) * 4 : 0x80000000u);
    };

    // Q, K of the two previous tiles at columns scol(s, c) (for finalize)
    uint2 q4a = make_uint2(0, 0), k4a = make_uint2(0, 0), q4b = q4a, k4b = k4a;
    f32x4 zA, zB, zC;  // dz rows of tiles k, k + 1, k + 2 in rotation
    zload(0, zA);
    zload(1, zB);
    auto body = [&](int k, const f32x4& zc, f32x4& zn) {
      zload(k + 2, zn);
      wg_barrier();  // B_k: tile k in LDS; partials of tile k - 2 complete
      finalize((k - 2) & 1, q4b, k4b, tok0(k - 2));
      q4b = q4a;
      k4b = k4a;
      {
        const char* st = smem + (k % G::NST) * G::SLOT;
        const char* Kt = st;
        const char* Qt = st + G::KB;
        const float* Et = (const float*)(st + 3 * G::KB);
        const int t0 = tok0(k);
        const bf16x8 kc[2] = {row_chunk(Kt, c, 0, g), row_chunk(Kt, c, 1, g)};
        const bf16x8 qc[2] = {row_chunk(Qt, c, 0, g), row_chunk(Qt, c, 1, g)};
        // A^T: register r = A[s' = c][t = 4g + r] = k_c . q_{4g+r}, kept for s' <= t
        f32x4 At = mfma_k32(qc[0], kc[0], f32x4{0, 0, 0, 0});
        At = mfma_k32(qc[1], kc[1], At);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c > 4 * g + r) At[r] = 0.f;
        const Split4 as = split4(At);
        const Split4 zrs = split4(zc);
        const f32x4 er = *(const f32x4*)(Et + 4 * g);

        const Split8 ws0 = split8(Wr[0], Wr[1]), ws1 = split8(Wr[2], Wr[3]);
        f32x4 Pr = mfma_k32(kc[0], ws0.hi, f32x4{0, 0, 0, 0});  // (Wb' K)[row c][t = 4g + r]
        Pr = mfma_k32(kc[0], ws0.lo, Pr);
        Pr = mfma_k32(kc[1], ws1.hi, Pr);
        Pr = mfma_k32(kc[1], ws1.lo, Pr);
        f32x4 Mr = mfma_k32(cat44(as.hi, as.lo), cat44(zrs.hi, zrs.hi), f32x4{0, 0, 0, 0});
        Mr = mfma_k32(cat44(as.hi, z4), cat44(zrs.lo, zrs.lo), Mr);  // (Zb A^T)[row c][t = 4g + r]
        f32x4 Gtr;
#pragma unroll
        for (int r = 0; r < 4; ++r) Gtr[r] = 2.f * er[r] * (Pr[r] + Mr[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = Gtr[r];
          st32(gv, rdv, (uint32_t)(tk(t0, 4 * g + r) * 64 + 16 * s + c) * 4);
        }
        // tokens in lanes: Gn register r = [row 16s + 4g + r][t = c]
        f32x4 Pt = mfma_k32(ws0.hi, kc[0], f32x4{0, 0, 0, 0});
        Pt = mfma_k32(ws0.lo, kc[0], Pt);
        Pt = mfma_k32(ws1.hi, kc[1], Pt);
        Pt = mfma_k32(ws1.lo, kc[1], Pt);
        f32x4 Gn = mfma_k32(cat44(zrs.hi, zrs.lo), cat44(as.hi, as.hi), Pt);
        Gn = mfma_k32(cat44(zrs.hi, z4), cat44(as.lo, as.lo), Gn);
        // hand-over: Gn, and Wb' with columns in lanes (register r =
        // Wb'[row 16s + 4g + r][scol(m, c)]) as hi | lo bf16
        char* ho = smem + G::HOB + ((k & 1) * 4 + s) * G::HO + lane * 16;
        *(f32x4*)ho = Gn;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint2 bh = pack4(mfma_k32((m >> 1) ? ws1.hi : ws0.hi, sel[m & 1], f32x4{0, 0, 0, 0}));
          const uint2 bl = pack4(mfma_k32((m >> 1) ? ws1.lo : ws0.lo, sel[m & 1], f32x4{0, 0, 0, 0}));
          *(uint4*)(ho + (1 + m) * 1024) = make_uint4(bh.x, bh.y, bl.x, bl.y);
        }
        {
          const Split4 gts = split4(Gtr);
          const bf16x8 zgh = cat44(zrs.hi, gts.hi), zgl = cat44(zrs.lo, gts.lo);
#pragma unroll
          for (int m = 0; m < 4; ++m) {  // Wb = Wb' + Zb Q^T - Gt K^T
            // Q, K with columns scol(m, c) in lanes, tokens 4g .. 4g + 3 in registers
            const uint2 q4 = pack4(mfma_k32(qc[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0}));
            const uint2 k4 = pack4(mfma_k32(kc[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0}));
            {  // kept for this wave's column block of the outputs (no branch)
              const uint32_t keep = 0u - (uint32_t)(m == s);
              q4a = make_uint2((q4.x & keep) | (q4a.x & ~keep), (q4.y & keep) | (q4a.y & ~keep));
              k4a = make_uint2((k4.x & keep) | (k4a.x & ~keep), (k4.y & keep) | (k4a.y & ~keep));
            }
            const uint2 k4n = make_uint2(k4.x ^ 0x80008000u, k4.y ^ 0x80008000u);
            if constexpr (HOLD) {  // Wb' + Zb Q^T here, -Gt K^T into H
              Wr[m] = mfma_k32(cat8(q4, q4), cat44(zrs.hi, zrs.lo), Wr[m]);
              Hr[m] = mfma_k32(cat8(k4n, k4n), cat44(gts.hi, gts.lo), Hr[m]);
            } else {
              const bf16x8 qk = cat8(q4, k4n);
              Wr[m] = mfma_k32(qk, zgh, Wr[m]);
              Wr[m] = mfma_k32(qk, zgl, Wr[m]);
            }
          }
        }
        if constexpr (HOLD) {
          if ((ntiles - 1 - k) % a.tpm == 0) {  // a mini-batch start: W0 is this state
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              Wr[m] += Hr[m];
              Hr[m] = f32x4{0, 0, 0, 0};
            }
          }
        }
      }
      wait_lgkm0();  // the hand-over is in LDS before the next barrier
    };
    for (int k = 0; k < niter; k += 3) {
      body(k, zA, zC);
      if (k + 1 < niter) body(k + 1, zB, zA);
      if (k + 2 < niter) body(k + 2, zC, zB);
    }
    if (a.dw0) {
      float* o = a.dw0 + (size_t)unit * a.dw0_stride + (16 * s + c) * 64;
#pragma unroll
      for (int m = 0; m < 4; ++m) *(f32x4*)(o + scol(m, 4 * g)) = Wr[m];
    }
    return;
  }

  if (wave == 8) {  // ===================================================== DMA
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const short*)a.k + uoff, (uint32_t)T * 128);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const short*)a.q + uoff, (uint32_t)T * 128);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const short*)a.v + uoff, (uint32_t)T * 128);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    // iteration-order tile k (16-byte chunk p of token row r lands at chunk
    // p ^ (r & 7)); tiles past either end read zeros into a free slot
    auto issue = [&](int k) {
      char* st = smem + (k % G::NST) * G::SLOT;
      const int t0 = tok0(k);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = 8 * n + (lane >> 3);
        const uint32_t vo = (uint32_t)tk(t0, r) * 128 + (((lane & 7) ^ (r & 7)) << 4);
        dma16(rk, st + n * 1024, vo);
        dma16(rq, st + G::KB + n * 1024, vo);
        dma16(rv, st + 2 * G::KB + n * 1024, vo);
      }
      if (lane < 16) dma4(re, st + 3 * G::KB, (uint32_t)tk(t0, lane) * 4);
    };
    for (int k = 0; k < G::D; ++k) issue(k);
    wait_vmcnt<G::NI * (G::D - 1)>();  // tile 0 landed
    for (int k = 0; k < niter; ++k) {
      wg_barrier();  // B_k
      issue(k + G::D);  // into the slot of tile k - 2, read last before B_k
      wait_vmcnt<G::NI * (G::D - 1)>();  // tile k + 1 landed
    }
    return;
  }

  // ========================================================== output waves
  // the slice's rows of the checkpoint of tile k (Wr's layout) and dz with
  // tokens in lanes (register r = Zb[row 16s + 4g + r][t = c])
  struct Pf {
    f32x4 w[4];
    f32x4 z;
  };
  const int nck = HOLD ? (ntiles + a.tpm - 1) / a.tpm : ntiles;  // checkpoints per unit
  auto pload = [&](int k, Pf& p) {
    const int kc = k < 0 ? 0 : (k < ntiles ? k : ntiles - 1);
    const int ci = HOLD ? (ntiles - 1 - kc) / a.tpm : ntiles - 1 - kc;
    const float* src = a.w_ckpt + ((size_t)unit * nck + ci) * 4096 + (16 * s + c) * 64;
#pragma unroll
    for (int m = 0; m < 4; ++m) p.w[m] = *(const f32x4*)(src + scol(m, 4 * g));
    p.z = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
              rdz, (uint32_t)(tk(tok0(k), c) * 64 + 16 * s + 4 * g) * 4, 0, 0));
  };
  // HOLD: W <- W + sgn G K^T over one tile in Wr's layout, with
  // G = 2 (W0 K - V) D at the gradient point W0 (split w0a, w0b); kc: the
  // K chunks of token c, vr / er: V[t = 4g + r][row 16s + c] and eta[4g + r];
  // neg = 0x80008000 negates K (sgn = -1)
  auto gk_update = [&](f32x4* W, const Split8& w0a, const Split8& w0b, const bf16x8* kc, f32x4 vr,
                       f32x4 er, uint32_t neg) {
    f32x4 Er = mfma_k32(kc[0], w0a.hi, f32x4{0, 0, 0, 0});  // (W0 K)[row c][t = 4g + r]
    Er = mfma_k32(kc[0], w0a.lo, Er);
    Er = mfma_k32(kc[1], w0b.hi, Er);
    Er = mfma_k32(kc[1], w0b.lo, Er);
    f32x4 Gr;
#pragma unroll
    for (int r = 0; r < 4; ++r) Gr[r] = 2.f * er[r] * (Er[r] - vr[r]);
    const Split4 gs = split4(Gr);
    const bf16x8 gb = cat44(gs.hi, gs.lo);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint2 k4 = pack4(mfma_k32(kc[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0}));
      const uint2 kx = make_uint2(k4.x ^ neg, k4.y ^ neg);
      W[m] = mfma_k32(cat8(kx, kx), gb, W[m]);
    }
  };
  // HOLD: W at the end of the next tile that outputs() takes
  f32x4 Wrun[4];
  if constexpr (HOLD) {
    const float* src = a.w_ckpt + ((size_t)unit * nck + nck - 1) * 4096 + (16 * s + c) * 64;
#pragma unroll
    for (int m = 0; m < 4; ++m) Wrun[m] = *(const f32x4*)(src + scol(m, 4 * g));
    const Split8 w0a = split8(Wrun[0], Wrun[1]), w0b = split8(Wrun[2], Wrun[3]);
    const unsigned short* kg = (const unsigned short*)a.k + uoff;
    const unsigned short* vg = (const unsigned short*)a.v + uoff;
    const float* eg = a.eta + (size_t)unit * T;
    for (int jf = (nck - 1) * a.tpm; jf < ntiles; ++jf) {  // the last mini-batch's tiles
      const int t0 = 16 * jf;
      bf16x8 kc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 x = t0 + c < T ? *(const uint4*)(kg + (size_t)(t0 + c) * 64 + 32 * h + 8 * g)
                                   : make_uint4(0, 0, 0, 0);
        kc[h] = __builtin_bit_cast(bf16x8, x);
      }
      f32x4 vr, er;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * g + r;
        vr[r] = t < T ? __builtin_bit_cast(float, (uint32_t)vg[(size_t)t * 64 + 16 * s + c] << 16) : 0.f;
        er[r] = t < T ? eg[t] : 0.f;
      }
      gk_update(Wrun, w0a, w0b, kc, vr, er, 0x80008000u);
    }
  }
  // partial sums over this slice's rows for tile p (iteration order)
  auto outputs = [&](int p, const Pf& pf) {
    const char* st = smem + (p % G::NST) * G::SLOT;
    const char* Kt = st;
    const char* Vt = st + 2 * G::KB;
    const float* Et = (const float*)(st + 3 * G::KB);
    const char* ho = smem + G::HOB + ((p & 1) * 4 + s) * G::HO + lane * 16;
    const f32x4 Gn = *(const f32x4*)ho;
    uint2 BBh[4], BBl[4];
    auto load_bb = [&] {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint4 b = *(const uint4*)(ho + (1 + m) * 1024);
        BBh[m] = make_uint2(b.x, b.y);
        BBl[m] = make_uint2(b.z, b.w);
      }
    };
    if constexpr (!HOLD) load_bb();
    const bf16x8 kc[2] = {row_chunk(Kt, c, 0, g), row_chunk(Kt, c, 1, g)};
    const float et = Et[c];
    const Split4 zts = split4(pf.z);
    const Split8 wa_0 = split8(pf.w[0], pf.w[1]), wa_1 = split8(pf.w[2], pf.w[3]);
    if constexpr (HOLD) {  // dQ reads the running state W_t, rebuilt here
      char* rw = smem + G::RED + ((p & 1) * 4 + s) * G::RW;
      f32x4 vr;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[r] = __builtin_bit_cast(float, (uint32_t)*(const unsigned short*)(Vt + swz(4 * g + r, 16 * s + c))
                                              << 16);
      f32x4 Wt[4] = {Wrun[0], Wrun[1], Wrun[2], Wrun[3]};
      gk_update(Wt, wa_0, wa_1, kc, vr, *(const f32x4*)(Et + 4 * g), 0u);
      // a mini-batch start: the tile before it ends at the exact checkpoint;
      // iterations outside the sequence (pf not loaded) leave Wrun alone
      const int jf = ntiles - 1 - p;
      const bool in = jf >= 0 && jf < ntiles, start = in && jf % a.tpm == 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) Wrun[m] = start ? pf.w[m] : (in ? Wt[m] : Wrun[m]);
      const Split8 wt_0 = split8(Wt[0], Wt[1]), wt_1 = split8(Wt[2], Wt[3]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {  // register r = [t = 4g + r][col scol(m, c)]: W_t^T Zb
        const uint2 qh = pack4(mfma_k32((m >> 1) ? wt_1.hi : wt_0.hi, sel[m & 1], f32x4{0, 0, 0, 0}));
        const uint2 ql = pack4(mfma_k32((m >> 1) ? wt_1.lo : wt_0.lo, sel[m & 1], f32x4{0, 0, 0, 0}));
        f32x4 dq = mfma_k32(cat44(zts.hi, zts.lo), cat8(qh, qh), f32x4{0, 0, 0, 0});
        dq = mfma_k32(cat44(zts.hi, z4), cat8(ql, ql), dq);
        *(f32x4*)(rw + (m * 64 + lane) * 16) = dq;
      }
    }
    f32x4 Ew = mfma_k32(wa_0.hi, kc[0], f32x4{0, 0, 0, 0});
    Ew = mfma_k32(wa_0.lo, kc[0], Ew);
    Ew = mfma_k32(wa_1.hi, kc[1], Ew);
    Ew = mfma_k32(wa_1.lo, kc[1], Ew);
    const f32x4 vv = bf4(*(const uint2*)(Vt + swz(c, 16 * s + 4 * g)));
    f32x4 Gtt, Gw;
    float dp = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = Ew[r] - vv[r];
      Gtt[r] = 2.f * et * Gn[r];
      Gw[r] = 2.f * et * e;
      dp -= Gn[r] * 2.f * e;
    }
    dp += __shfl_xor(dp, 16);
    dp += __shfl_xor(dp, 32);
    char* rw = smem + G::RED + ((p & 1) * 4 + s) * G::RW;
    if constexpr (HOLD) load_bb();  // (late: fewer registers live across the rebuild)
    // W with columns in lanes: WB[m] register r = W[row 16s + 4g + r][scol(m, c)]
    uint2 WBh[4], WBl[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      WBh[m] = pack4(mfma_k32((m >> 1) ? wa_1.hi : wa_0.hi, sel[m & 1], f32x4{0, 0, 0, 0}));
      WBl[m] = pack4(mfma_k32((m >> 1) ? wa_1.lo : wa_0.lo, sel[m & 1], f32x4{0, 0, 0, 0}));
    }
    const Split4 gts = split4(Gtt), gws = split4(Gw);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // register r = [t = 4g + r][col scol(m, c)]
      if constexpr (!HOLD) {
        f32x4 dq = mfma_k32(cat44(zts.hi, zts.lo), cat8(WBh[m], WBh[m]), f32x4{0, 0, 0, 0});
        dq = mfma_k32(cat44(zts.hi, z4), cat8(WBl[m], WBl[m]), dq);  // W^T Zb
        *(f32x4*)(rw + (m * 64 + lane) * 16) = dq;
      }
      f32x4 dk = mfma_k32(cat44(gts.hi, gts.lo), cat8(WBh[m], WBh[m]), f32x4{0, 0, 0, 0});
      dk = mfma_k32(cat44(gts.hi, z4), cat8(WBl[m], WBl[m]), dk);  // W^T Gt
      dk = mfma_k32(cat44(gws.hi, gws.lo), cat8(BBh[m], BBh[m]), dk);
      dk = mfma_k32(cat44(gws.hi, z4), cat8(BBl[m], BBl[m]), dk);  // + Wb'^T G
      *(f32x4*)(rw + G::RQ + (m * 64 + lane) * 16) = -dk;
    }
    // G^T Zb: register r = sum_rows G[row][s' = 4g + r] Zb[row][t = c]
    f32x4 ab = mfma_k32(cat44(gws.hi, gws.lo), cat44(zts.hi, zts.hi), f32x4{0, 0, 0, 0});
    ab = mfma_k32(cat44(gws.hi, z4), cat44(zts.lo, zts.lo), ab);
    *(f32x4*)(rw + 2 * G::RQ + lane * 16) = ab;
    ((float*)(rw + 2 * G::RQ + G::RA))[lane] = dp;  // lanes c < 16 hold the sums
  };

  // Prefetch of tile p happens at iteration p - 1 (p = 0: before the loop),
  // its use at iteration p + 1; three register sets rotate by unrolling.
  // HOLD keeps the running state in registers as well and prefetches one
  // iteration ahead instead, with two sets.
  if constexpr (HOLD) {
    Pf pA, pB;  // tile -1 (iteration 0) is never loaded: outputs() ignores it
    auto body = [&](int k, const Pf& pc, Pf& pn) {
      pload(k, pn);
      wg_barrier();  // B_k: tile k in LDS; hand-over of tile k - 1 complete
      outputs(k - 1, pc);
      wait_lgkm0();  // the partials are in LDS before the next barrier
    };
    for (int k = 0; k < niter; k += 2) {
      body(k, pB, pA);
      if (k + 1 < niter) body(k + 1, pA, pB);
    }
  } else {
    Pf pA, pB, pC;
    pload(0, pA);
    auto body = [&](int k, const Pf& pc, Pf& pn) {
      pload(k + 1, pn);
      wg_barrier();  // B_k: tile k in LDS; hand-over of tile k - 1 complete
      outputs(k - 1, pc);
      wait_lgkm0();  // the partials are in LDS before the next barrier
    };
    for (int k = 0; k < niter; k += 3) {
      body(k, pC, pB);
      if (k + 1 < niter) body(k + 1, pA, pC);
      if (k + 2 < niter) body(k + 2, pB, pA);
    }
  }
}

// Chunked backward, serial part.  Per tile the adjoint of the state walks
// as Wb = Wb' (I - 2 K D K^T) + (terms without Wb'), the forward's factor,
// which is symmetric; so over chunk p the end adjoint E_p maps to the start
// adjoint E_p M_p^T + C_p, with M_p the chunk's forward map (W_end = W_start
// M_p + ...) and C_p the chunk's backward from a zero end adjoint.  From
// E_{P-1} = dW_T (or 0), E_{p-1} = E_p M_p^T + C_p; the start adjoint of
// chunk 0 is dW0.  Chunk p's dq region holds E_p (written here, floats
// 0..4095), M_p (4096..8191) and C_p (8192..12287), each [64][64].
// Workgroup = (unit, 8 rows); thread (r, col pair).
constexpr int ACOMB_ROWS = 8;

__global__ void __launch_bounds__(256) chunk_adjoint_combine_kernel(const float* dw_T, float* dq,
                                                                    float* dw0, int Tc, int P) {
  __shared__ float Mp[64 * 65];           // M_p, row pitch 65 (conflict-free column reads)
  __shared__ float Er[ACOMB_ROWS][64];    // the rows' current adjoint
  const int u = blockIdx.x, row0 = blockIdx.y * ACOMB_ROWS, t = threadIdx.x;
  const int r = t >> 5, col = 2 * (t & 31);
  for (int e = t; e < ACOMB_ROWS * 64; e += 256)
    Er[e >> 6][e & 63] = dw_T ? dw_T[(size_t)u * 4096 + (row0 + (e >> 6)) * 64 + (e & 63)] : 0.f;
  auto chunk = [&](int p) { return dq + ((size_t)u * P + p) * Tc * 64; };
  // registers: this thread's four float4 of the next M and its two C' values,
  // loaded while the current step runs
  f32x4 mnext[4];
  float2 cnext;
  auto fetch = [&](int p) {
    const float* reg = chunk(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) mnext[q] = *(const f32x4*)(reg + 4096 + 4 * (t + 256 * q));
    cnext = *(const float2*)(reg + 8192 + (row0 + r) * 64 + col);
  };
  fetch(P - 1);
  for (int p = P - 1; p >= 0; --p) {
    float* reg = chunk(p);
    __syncthreads();  // Er complete, Mp free
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = t + 256 * q;
      float* d = Mp + (e >> 4) * 65 + 4 * (e & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = mnext[q][i];
    }
    const float2 cc = cnext;
    if (p > 0) fetch(p - 1);
    for (int e = t; e < ACOMB_ROWS * 64; e += 256) reg[(row0 + (e >> 6)) * 64 + (e & 63)] = Er[e >> 6][e & 63];
    __syncthreads();  // Mp complete
    float a0 = cc.x, a1 = cc.y;
#pragma unroll 16
    for (int k = 0; k < 64; ++k) {
      const float e = Er[r][k];
      a0 = fmaf(e, Mp[col * 65 + k], a0);
      a1 = fmaf(e, Mp[(col + 1) * 65 + k], a1);
    }
    __syncthreads();  // Er fully read
    Er[r][col] = a0;
    Er[r][col + 1] = a1;
  }
  __syncthreads();
  for (int e = t; e < ACOMB_ROWS * 64; e += 256)
    dw0[(size_t)u * 4096 + (row0 + (e >> 6)) * 64 + (e & 63)] = Er[e >> 6][e & 63];
}

}  // namespace

hipError_t launch_linear_bwd(const LinearBwdArgs& a, hipStream_t s) {
  if (a.tpm > 1) return launch(linear_bwd_kernel<true>, dim3(a.units), dim3(BwdGeom::THREADS), s, a);
  return launch(linear_bwd_kernel<false>, dim3(a.units), dim3(BwdGeom::THREADS), s, a);
}

hipError_t launch_linear_bwd_chunked(const LinearBwdArgs& a, int P, int rows, hipStream_t s) {
  const int Tc = a.T / P;
  if (P < 2 || a.T % P != 0 || Tc % 16 != 0 || Tc < 192 || !a.dw0) return hipErrorInvalidValue;
  // M_p: each chunk's forward scan from the identity with V = 0 (Q is not
  // read), into its dq floats 4096..8191; chunk p of unit u is sequence
  // u * P + p of length Tc
  LinearArgs f{};
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.eta = a.eta;
  f.w0 = nullptr;
  f.z = nullptr;
  f.w_out = a.dq + 4096;
  f.w0_per_batch = 1;
  f.units = a.units * P;
  f.H = a.H;
  f.T = Tc;
  f.b = 16;
  f.v_zero = 1;
  f.w0_mode = W0_IDENTITY;
  f.wout_stride = Tc * 64;
  hipError_t e = launch_linear(f, false, rows, s);
  if (e != hipSuccess) return e;
  // C_p: each chunk's backward from a zero end adjoint; only its start
  // adjoint is kept, in its dq floats 8192..12287
  LinearBwdArgs c = a;
  c.units = a.units * P;
  c.T = Tc;
  c.dw_T = nullptr;
  c.tok_out = 0;
  c.dw0 = a.dq + 8192;
  c.dw0_stride = Tc * 64;
  e = launch_linear_bwd(c, s);
  if (e != hipSuccess) return e;
  e = launch(chunk_adjoint_combine_kernel, dim3(a.units, 64 / ACOMB_ROWS), dim3(256), s, a.dw_T,
             a.dq, a.dw0, Tc, P);
  if (e != hipSuccess) return e;
  // every chunk from its end adjoint (its dq floats 0..4095, read before any
  // of that memory is written: the first tokens' outputs come last)
  c.dw_T = a.dq;
  c.dw_stride = Tc * 64;
  c.tok_out = 1;
  c.dw0 = nullptr;
  return launch_linear_bwd(c, s);
}

}  // namespace ttt
