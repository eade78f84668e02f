// TTT-Linear forward scan, bf16 Q/K/V (the production path), gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): mini-batch GD with the gradient taken at the state
// before the mini-batch (§3.5), evaluated per 16-token tile in the dual form
// of §3.6 with the per-token eta of §4.6 and f(x) = W x (§4.4):
//   P = W K, G = 2 (P - V) diag(eta), Z = W Q - G triu(K^T Q), W <- W - G K^T
// (columns are tokens; the inclusive causal mask lets token t see its own
// update, §3.1).  The kernels carry Gn = -G ("negative gradient").
//
// Workgroup = one (batch, head, slice of ROWS rows of W):
//   waves 0 .. NCW-1  compute waves, 16 rows of W each, fp32 state resident
//                     in MFMA accumulators for the whole sequence;
//   waves NCW, NCW+1  helpers: build every per-tile operand that depends only
//                     on K, Q, eta, two tiles ahead, into a double-buffered
//                     "prepared" LDS area laid out lane-linear (conflict-free
//                     16-byte reads); helper 0 makes triu(K^T Q), K_{j-1}^T K_j
//                     and 2 eta, helper 1 the update operand (and the
//                     sub-batch inverse);
//   wave NCW+2        loader: buffer->LDS DMA of 16-token K/Q/V/eta tiles,
//                     D tiles ahead, into a ring (zero-filled past T).
// The compute waves read every LDS operand of a tile one iteration before
// they use it (registers double as a second pipeline stage), so no LDS
// latency sits between a tile barrier and the serial chain that follows it.
// Nothing is scheduled across a tile barrier, which keeps those stages in
// place, and the compute waves run at the highest wave priority.
//
// Serial chain per tile.  Only P_j = W_j K_j feeds the recurrence.  Using
//   P_{j+1} = W_j K_{j+1} + Gn_j (K_j^T K_{j+1})     (W_{j+1} = W_j + Gn_j K_j^T)
// the large product W_j K_{j+1} is formed one tile early from W_j, so the
// per-tile critical path is two MFMAs plus the gradient's few VALU ops; the
// W update, the bf16 hi/lo split of W and the output products overlap with
// it.  The outputs need no lookahead: R_j = W_j Q_j is formed from the same
// split of W_j, off the chain.  V enters P's accumulator exactly, as (-I)
// applied to V's rows on MFMA, so the chain yields P - V directly.
//
// The outputs are formed transposed (W Q rather than (W Q)^T), so each lane
// holds 4 consecutive rows of one token and stores them in one 16-byte write.
//
// Precision: fp32 operands enter bf16 MFMA as hi + lo pairs (three products
// kept, error ~2^-16 relative); K, Q, V are exact bf16; accumulation fp32.
//
// Column order.  Compute wave register W[m][r] of lane (c, g) holds
// W[row c][sigma(m, 4g + r)] with sigma(m, 4g + r) = 32(m/2) + 8g + 4(m%2) + r,
// the accumulator layout of the rank-16 update with a permuted output index.
// With it, the reduction slots 8g..8g+7 of the K=32 MFMA that forms W K
// are the 8 consecutive columns 32h + 8g .. +7, i.e. one 16-byte chunk of a
// K row.  K/Q tiles are stored with chunk p of row r at position
// p ^ (r & 7) (applied by the DMA's source addresses), which makes those
// 16-row chunk reads bank-conflict free.
#include <type_traits>

#include "ttt_device.h"
#include "ttt_launch.h"
#include "ttt_linear_ops.h"

namespace ttt {
namespace {

enum { MODE_B16 = 0, MODE_SUB = 1, MODE_MULTI = 2 };

// DEPTH: tiles the loader keeps in flight beyond the two the compute waves
// are working on (0 = the default, as many as the vmcnt field can count, at
// most 10).  Any depth >= 1 gives bit-identical results: the ring only
// changes when tiles land, never what is computed.
template <int ROWS, int DEPTH = 0>
struct Geom {
  static constexpr int NCW = ROWS / 16;
  static constexpr int KB = 16 * 64 * 2;         // K or Q tile (bf16)
  static constexpr int VB = 16 * ROWS * 2;       // V tile, this slice's columns
  static constexpr int RAW = 2 * KB + VB + 64;   // + eta (16 fp32)
  static constexpr int NI = 4 + (VB + 1023) / 1024 + 1;  // DMA ops per tile
  static constexpr int D = DEPTH > 0 ? DEPTH : ((63 / NI) < 10 ? (63 / NI) : 10);
  static_assert(D >= 1 && NI * D < 64, "in-flight DMA count must fit vmcnt");
  static constexpr int NST = D + 3;
  // prepared-operand slot (per tile), byte offsets
  static constexpr int P_E2 = 0;                  // 2 eta_t, 16 fp32
  static constexpr int P_A = 64;                  // triu(K^T Q), hi | lo
  static constexpr int P_MKK = P_A + 1024;        // K_{j-1}^T K_j, hi | lo
  static constexpr int P_KT = P_MKK + 1024;       // update operand K[t][j], x4
  static constexpr int P_U = P_KT + 4096;         // sub-batch inverse (b < 16)
  static constexpr int PREP = P_U + 1024;
  static constexpr int LDS = NST * RAW + 2 * PREP;
  static constexpr int THREADS = (NCW + 3) * 64;  // + 2 helpers + loader
};

// TPM: tiles per mini-batch when it is fixed at compile time (b = 32, 64),
// so a tile's position inside its mini-batch costs nothing; 0 = read from
// the arguments (other multiples of 16).  Unused below b = 16.
// CKPT: also store the state at the start of every mini-batch, the
// checkpoints the backward pass reads (b = 16: every tile; 16 | b: every
// b / 16 tiles); for b < 16 each b-token mini-batch
// takes a tile of its own (a.bt = b), rows b..15 reading as zero tokens
// (eta = 0 leaves the state and the other tokens' outputs unchanged) and
// dropping their outputs: the b = 16 arithmetic on padded tiles.
template <int MODE, int ROWS, int TPM, bool CKPT = false, int DEPTH = 0>
__global__ void __launch_bounds__((Geom<ROWS>::THREADS))
linear_scan_bf16_kernel(LinearArgs a) {
  using G = Geom<ROWS, DEPTH>;
  constexpr int NSPLIT = 64 / ROWS;
  // with checkpoints: per compute wave a 16-row staging tile (rows padded by 4 words)
  constexpr int CK_TILE = CKPT ? 16 * 68 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS + G::NCW * CK_TILE];
  char* const raw = smem;
  char* const prep = smem + G::NST * G::RAW;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;

  int unit, slice;
  if (NSPLIT == 1) {
    unit = blockIdx.x;
    slice = 0;
  } else {  // slices of one unit on one XCD (workgroups go round-robin over 8)
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    slice = slot % NSPLIT;
    unit = (slot / NSPLIT) * 8 + xcd;
  }
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int bt = CKPT ? a.bt : 16;  // tokens per tile
  const int ntiles = CKPT ? (T + bt - 1) / bt : (T + 15) >> 4;
  const int row0 = slice * ROWS;
  // token of row r of tile j (T, just past every descriptor, for rows >= bt)
  auto tokrow = [&](int j, int r) {
    if constexpr (CKPT)
      return r < bt ? j * bt + r : T;
    else
      return j * 16 + r;
  };

  // ================================================================ loader
  // Barriers B_-2, B_-1, B_0 .. B_{ntiles-1}.  B_j (j >= 0) releases compute
  // iteration j (which reads raw tile j+2 for the next iteration) and helper
  // iteration j (which prepares tile j+2 from raw tile j+2); before it the
  // loader makes sure raw tiles <= j+2 have landed.  B_-2 guarantees raw
  // tiles 0 and 1.  Raw tile t is last read before B_t (its Q rows, one
  // iteration ahead of the outputs of tile t), so tile j+D+2 is issued after
  // B_{j-1} into the slot of tile j-1: NST = D + 3 slots.
  if (wave == G::NCW + 2) {
    const uint32_t ubytes = (uint32_t)T * 128;
    const size_t uoff = (size_t)unit * T * 64;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const short*)a.k + uoff, ubytes);
    // no outputs: Q is not needed; v_zero: V reads as zeros (no memory access)
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const short*)a.q + uoff, a.z ? ubytes : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const short*)a.v + uoff, a.v_zero ? 0u : ubytes);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    const int krow = lane >> 3, kpos = lane & 7;
    auto issue = [&](int j) {
      char* st = raw + (j % G::NST) * G::RAW;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = 8 * n + krow;
        const uint32_t off = (uint32_t)tokrow(j, r) * 128 + ((kpos ^ (r & 7)) << 4);
        dma16(rk, st + n * 1024, off);
        dma16(rq, st + G::KB + n * 1024, off);
      }
#pragma unroll
      for (int n = 0; n < (G::VB + 1023) / 1024; ++n) {
        const int byte = n * 1024 + lane * 16;
        if (G::VB % 1024 == 0 || byte < G::VB) {
          const int tok = byte / (ROWS * 2), cb = byte % (ROWS * 2);
          dma16(rv, st + 2 * G::KB + n * 1024, (uint32_t)tokrow(j, tok) * 128 + row0 * 2 + cb);
        }
      }
      if (lane < 16) dma4(re, st + 2 * G::KB + G::VB, (uint32_t)tokrow(j, lane) * 4);
    };
    const int pro = ntiles < G::D + 2 ? ntiles : G::D + 2;
    for (int j = 0; j < pro; ++j) issue(j);
    if (pro == G::D + 2) wait_vmcnt<G::NI * G::D>();  // tiles 0, 1 landed
    else wait_vmcnt<0>();
    wg_barrier_pinned();  // B_{-2}
    wg_barrier_pinned();  // B_{-1}
    for (int j = 0; j < ntiles; ++j) {
      if (j + G::D + 2 < ntiles) {
        issue(j + G::D + 2);
        wait_vmcnt<G::NI * G::D>();  // tiles <= j+2 landed
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier_pinned();  // B_j
    }
    return;
  }

  // ================================================================ helper
  // Iteration j (between B_j and B_{j+1}, j = -2 .. ntiles-2) prepares tile
  // j+2 (if it exists) into prepared slot j & 1; compute iteration j+1 reads
  // it into registers, and had read that slot's previous tile before B_j.
  if (wave >= G::NCW) {
    const bool h0 = wave == G::NCW;  // helper 0 or helper 1
    bf16x8 kprev[2], sel[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      for (int e = 0; e < 8; ++e) {
        kprev[h][e] = (bf16)0.f;
        // slot 8g+e of block m/2 selects column sigma(m, c) for m % 2 == h
        sel[h][e] = (bf16)((g == (c >> 2) && e == 4 * h + (c & 3)) ? 1.f : 0.f);
      }
    wg_barrier_pinned();  // B_{-2}
    for (int j = -2; j < ntiles - 1; ++j) {
      const int tn = j + 2;
      if (tn >= ntiles) {  // nothing left to prepare: keep the barrier count
        wg_barrier_pinned();      // B_{j+1}
        continue;
      }
      const char* st = raw + (tn % G::NST) * G::RAW;
      const char* Kt = st;
      const char* Qt = st + G::KB;
      const float* Et = (const float*)(st + 2 * G::KB + G::VB);
      char* pp = prep + (tn & 1) * G::PREP;

      bf16x8 kop[2], qop[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        kop[h] = row_chunk(Kt, c, h, g);
        qop[h] = row_chunk(Qt, c, h, g);
      }
      // all products first (independent MFMAs back to back), then the
      // conversions, then the stores
      if (h0) {
        f32x4 A = {0, 0, 0, 0}, Mkk = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          A = mfma_k32(kop[h], qop[h], A);        // A[s = 4g+r][t = c] = k_s . q_t
          Mkk = mfma_k32(kprev[h], kop[h], Mkk);  // k^{prev}_s . k_t
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > c) A[r] = 0.f;
        put_split(pp + G::P_A, lane, A);
        put_split(pp + G::P_MKK, lane, Mkk);
        if (lane < 16) ((float*)(pp + G::P_E2))[lane] = 2.f * Et[lane];
      } else {
        f32x4 KS[4];
        // Update operand kt[m][e] = K[t = 4g+e][sigma(m, c)], formed exactly
        // as K S_m with the one-hot selection S_m[j][c] = [j == sigma(m, c)]
        // (only the 32 columns of block m/2 can be selected).
#pragma unroll
        for (int m = 0; m < 4; ++m) KS[m] = mfma_k32(kop[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t p0 = pack_rne(KS[m][0], KS[m][1]), p1 = pack_rne(KS[m][2], KS[m][3]);
          *(uint4*)(pp + G::P_KT + m * 1024 + lane * 16) = make_uint4(p0, p1, p0, p1);  // [kt | kt]
        }
      }

      if (MODE == MODE_SUB && h0) {  // helper 0 only
        // Sub-batches of b tokens inside the tile: G (I + N) = E with
        // N[s][t] = 2 eta_t k_s.k_t for sub-batch(s) < sub-batch(t);
        // U = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), cut at N^{16/b}.
        const int bsub = a.b;
        f32x4 M = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) M = mfma_k32(kop[h], kop[h], M);
        const float eta_c = Et[c];
        const f32x4 eta4 = *(const f32x4*)(Et + 4 * g);
        f32x4 N, NT, I;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 4 * g + r;
          N[r] = (s / bsub < c / bsub) ? 2.f * eta_c * M[r] : 0.f;
          NT[r] = (c / bsub < s / bsub) ? 2.f * eta4[r] * M[r] : 0.f;  // M symmetric
          I[r] = (s == c) ? 1.f : 0.f;
        }
        const f32x4 Z0 = {0, 0, 0, 0};
        auto mm = [&](f32x4 xt, f32x4 y) { return mm16_split(xt, y, Z0); };
        const int nblk = 16 / bsub;
        f32x4 U;
        if (nblk == 2) {
          U = I - N;
        } else {
          const f32x4 N2 = mm(NT, N), N2T = mm(N, NT);
          f32x4 tail;
          if (nblk == 4) {
            tail = I + N2;
          } else {
            const f32x4 N4 = mm(N2T, N2);
            f32x4 t4;
            if (nblk == 8) {
              t4 = I + N4;
            } else {
              const f32x4 N4T = mm(N2, N2T);
              t4 = mm(I + N4T, I + mm(N4T, N4));
            }
            tail = mm(I + N2T, t4);
          }
          U = mm(I - NT, tail);
        }
        put_split(pp + G::P_U, lane, U);
      }
      kprev[0] = kop[0];
      kprev[1] = kop[1];
      wait_lgkm0();
      wg_barrier_pinned();  // B_{j+1}
    }
    return;
  }

  // =============================================================== compute
  // The compute waves carry the serial chain; the helpers and the loader
  // share their SIMDs and must not delay it.
  __builtin_amdgcn_s_setprio(3);
  // Iteration j enters with W = W_j (fp32 accumulators), XB = W_{j-1} K_j - V_j
  // (formed in iteration j-1), gp = operands of Gn_{j-1}, and in registers the
  // prepared operands of tile j, the raw K/V operands of tile j+1 and the Q
  // operands of tile j (read from LDS during iteration j-1).
  const int rbase = row0 + wave * 16;
  f32x4 W[4];
  if (a.w0_mode == W0_IDENTITY || a.w0_mode == W0_ZERO) {
    const float one = a.w0_mode == W0_IDENTITY ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        W[m][r] = rbase + c == 32 * (m >> 1) + 8 * g + 4 * (m & 1) + r ? one : 0.f;
  } else if (a.w0_mode == W0_IN_Z) {
    const float* zu = a.z + (size_t)unit * T * 64;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      W[m] = *(const f32x4*)(zu + chunk_state_in_z(T, ROWS, rbase + c, 32 * (m >> 1) + 8 * g + 4 * (m & 1)));
  } else {
    const float* w0 = a.w0 + (size_t)(a.w0_per_batch ? unit : head) * 4096;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      W[m] = *(const f32x4*)(w0 + (rbase + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1));
  }
  const int tpm = MODE != MODE_MULTI ? 1 : (TPM > 0 ? TPM : (a.b >> 4));  // tiles per mini-batch
  const int nmb = MODE == MODE_MULTI ? (T + a.b - 1) / a.b : ntiles;        // mini-batches (checkpoints)
  const NegSel ns = make_negsel(c, g);
  // -I on the 16 V columns of this wave: X = -V_block lands in accumulator
  // layout when V's rows are the A-operand (slots 16..31 are unused).
  bf16x8 negI;
#pragma unroll
  for (int e = 0; e < 8; ++e) negI[e] = (bf16)((g < 2 && 8 * g + e == c) ? -1.f : 0.f);
  const int voff = 2 * G::KB + c * (ROWS * 2) + (16 * wave + 8 * (g & 1)) * 2;  // V row chunk
  YOps gp;  // operands of the previous tile's negative gradient
  gp.hh = cat44(s16x4{0, 0, 0, 0}, s16x4{0, 0, 0, 0});
  gp.l0 = gp.hh;
  Split8 wg[2];  // gradient point operands (b > 16)

  // raw operands for this lane: K and V row chunks of one tile and the Q row
  // chunks of the tile before it
  struct RawOps {
    bf16x8 k[2], v, q[2];
  };
  auto load_raw = [&](RawOps& r, const char* st, const char* sq) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r.k[h] = row_chunk(st, c, h, g);
      r.q[h] = row_chunk(sq + G::KB, c, h, g);
    }
    r.v = *(const bf16x8*)(st + voff);
  };
  // prepared operands of one tile for this lane
  struct PrepOps {
    f32x4 e2;
    bf16x8 mkk, att, kt[4], u;
  };
  auto load_prep = [&](PrepOps& p, const char* pp) {
    p.e2 = *(const f32x4*)(pp + G::P_E2 + 16 * g);
    p.mkk = get8(pp + G::P_MKK, lane);
    p.att = get8(pp + G::P_A, lane);
#pragma unroll
    for (int m = 0; m < 4; ++m) p.kt[m] = get8(pp + G::P_KT + m * 1024, lane);
    if constexpr (MODE == MODE_SUB) p.u = get8(pp + G::P_U, lane);
  };

  wg_barrier_pinned();  // B_{-2}: raw tiles 0 and 1 are in LDS
  f32x4 XB = {0, 0, 0, 0};
  RawOps ra;  // raw K/V of tile j+1, Q of tile j
  {
    const Split8 ws[2] = {split8_mfma(W[0], W[1], ns), split8_mfma(W[2], W[3], ns)};
    wg[0] = ws[0];
    wg[1] = ws[1];
    RawOps r0;
    load_raw(r0, raw, raw);
    XB = mfma_k32(r0.v, negI, XB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      XB = mfma_k32(r0.k[h], ws[h].hi, XB);
      XB = mfma_k32(r0.k[h], ws[h].lo, XB);
    }
    load_raw(ra, raw + 1 * G::RAW, raw);
  }
  wait_lgkm0();
  wg_barrier_pinned();  // B_{-1}: prepared tile 0 is in LDS
  PrepOps pa, pb;  // prepared operands of tiles j and j+1 (two register sets)
  RawOps rb;       // raw K/V of tile j+2, Q of tile j+1
  load_prep(pa, prep);

  // Z through a range-checked buffer: rows past T (padding of the last
  // tile) are dropped by the hardware, so the loop body has no branches and
  // the scheduler can interleave the serial chain with everything else.
  const __amdgpu_buffer_rsrc_t rz =
      make_rsrc(a.z ? a.z + (size_t)unit * T * 64 : a.w_out, a.z ? (uint32_t)T * 256 : 0u);
  uint32_t zoff = (uint32_t)((c * 64 + rbase + 4 * g) * 4);  // token c, rows 4g..4g+3

  // One tile: uses (pc, rc), fills (pn, rn) for the next one.  The loop
  // below alternates two register sets, so nothing is copied between
  // iterations and the reads have a whole tile of work to land.
  // POS: the tile's position in its mini-batch when known at compile time
  // (an std::integral_constant), -1 otherwise.
  auto tile = [&](const int j, auto POS, const PrepOps& pc, const RawOps& rc, PrepOps& pn,
                  RawOps& rn) {
    wait_lgkm0();
    wg_barrier_pinned();  // B_j
    // next iteration's operands: prepared tile j+1, raw K/V of tile j+2 and
    // Q of tile j+1 (stale past the end of the sequence, where they are never
    // used)
    load_prep(pn, prep + ((j + 1) & 1) * G::PREP);
    load_raw(rn, raw + ((j + 2) % G::NST) * G::RAW, raw + ((j + 1) % G::NST) * G::RAW);
    __builtin_amdgcn_sched_barrier(0);  // the reads go out first
    constexpr int pos = decltype(POS)::value;
    const bool new_mb = MODE != MODE_MULTI || (pos >= 0 ? pos == 0 : (j % tpm) == 0);
    const bool next_new_mb =
        MODE != MODE_MULTI || (pos >= 0 ? (pos + 1) % (TPM > 0 ? TPM : 1) == 0 : ((j + 1) % tpm) == 0);
    if constexpr (CKPT) {  // W_j, the state before mini-batch j / tpm, when one starts
      if (new_mb) {
        // through this wave's LDS tile, so that each store writes 4 whole rows
        // (1 KB of consecutive memory), nontemporally
        char* const ct = smem + G::LDS + wave * CK_TILE;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          *(f32x4*)(ct + (c * 68 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) * 4) = W[m];
        const int mb = MODE == MODE_MULTI ? j / tpm : j;
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(a.w_ckpt + ((size_t)unit * nmb + mb) * 4096 + __builtin_amdgcn_readfirstlane(rbase) * 64,
                      16u * 64u * 4u);  // (rbase pinned to a scalar register: a uniform descriptor)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = (lane >> 4) + 4 * kk, col = 4 * (lane & 15);
          const f32x4 v = *(const f32x4*)(ct + (row * 68 + col) * 4);
          typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4c, v), rc,
                                                 (uint32_t)((row * 64 + col) * 4), 0, 2);
        }
      }
    }

    // ---- serial chain: X_j = P_j - V_j, then Gn_j = 2 eta (v - p).
    // (gp is zero at j = 0; within a b > 16 mini-batch P keeps its gradient
    // point and takes no correction.)
    f32x4 X = mm_pre(pc.mkk, gp, XB);
    if (MODE == MODE_MULTI) X = new_mb ? X : XB;
    f32x4 E;
#pragma unroll
    for (int r = 0; r < 4; ++r) E[r] = -pc.e2[r] * X[r];
    if constexpr (MODE == MODE_SUB) E = mm_pre(pc.u, yops(split4(E)), f32x4{0, 0, 0, 0});
    const Split4 gs = split4(E);
    const YOps gy = yops(gs);

    // ---- split of W_j and the next tile's products with it
    const Split8 ws[2] = {split8_mfma(W[0], W[1], ns), split8_mfma(W[2], W[3], ns)};
    if (MODE == MODE_MULTI) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        wg[h].hi = new_mb ? ws[h].hi : wg[h].hi;
        wg[h].lo = new_mb ? ws[h].lo : wg[h].lo;
      }
    }
    f32x4 XBn = mfma_k32(rc.v, negI, f32x4{0, 0, 0, 0});
    f32x4 R = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 whi = ws[h].hi, wlo = ws[h].lo;
      if (MODE == MODE_MULTI) {
        whi = next_new_mb ? whi : wg[h].hi;
        wlo = next_new_mb ? wlo : wg[h].lo;
      }
      XBn = mfma_k32(rc.k[h], whi, XBn);
      XBn = mfma_k32(rc.k[h], wlo, XBn);
      R = mfma_k32(ws[h].hi, rc.q[h], R);
      R = mfma_k32(ws[h].lo, rc.q[h], R);
    }

    // ---- outputs: Z_j = W_j Q_j + Gn_j triu(K_j^T Q_j); lane (c, g) holds
    // rows 4g..4g+3 of token c
    const f32x4 Z = mm_pre_t(gy, pc.att, R);
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(u32x4, Z), rz, CKPT ? (uint32_t)((tokrow(j, c) * 64 + rbase + 4 * g) * 4) : zoff, 0, 2);
    zoff += 16 * 64 * 4;

    // ---- rank-16 update W_{j+1} = W_j + Gn_j K_j^T
    const bf16x8 g2 = cat44(gs.hi, gs.lo);
#pragma unroll
    for (int m = 0; m < 4; ++m) W[m] = mfma_k32(pc.kt[m], g2, W[m]);
    XB = XBn;
    gp = gy;
  };
  int j = 0;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using PN = std::integral_constant<int, -1>;
  if constexpr (MODE == MODE_MULTI && TPM == 4) {
    for (; j + 3 < ntiles; j += 4) {
      tile(j, P0{}, pa, ra, pb, rb);
      tile(j + 1, P1{}, pb, rb, pa, ra);
      tile(j + 2, P2{}, pa, ra, pb, rb);
      tile(j + 3, P3{}, pb, rb, pa, ra);
    }
    if (j < ntiles) tile(j, P0{}, pa, ra, pb, rb);
    if (j + 1 < ntiles) tile(j + 1, P1{}, pb, rb, pa, ra);
    if (j + 2 < ntiles) tile(j + 2, P2{}, pa, ra, pb, rb);
  } else if constexpr (MODE == MODE_MULTI && TPM == 2) {
    for (; j + 1 < ntiles; j += 2) {
      tile(j, P0{}, pa, ra, pb, rb);
      tile(j + 1, P1{}, pb, rb, pa, ra);
    }
    if (j < ntiles) tile(j, P0{}, pa, ra, pb, rb);
  } else {
    for (; j + 1 < ntiles; j += 2) {
      tile(j, PN{}, pa, ra, pb, rb);
      tile(j + 1, PN{}, pb, rb, pa, ra);
    }
    if (j < ntiles) tile(j, PN{}, pa, ra, pb, rb);
  }

  if (a.wout_every <= 1 || unit % a.wout_every == a.wout_every - 1) {
    float* wo = a.w_out + (size_t)(unit / (a.wout_every > 1 ? a.wout_every : 1)) * a.wout_stride;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *(f32x4*)(wo + (rbase + c) * 64 + 32 * (m >> 1) + 8 * g + 4 * (m & 1)) = W[m];
  }
}

template <int MODE, int ROWS, int TPM, bool CKPT = false, int DEPTH = 0>
hipError_t launch_one(const LinearArgs& a, hipStream_t s) {
  constexpr int NSPLIT = 64 / ROWS;
  const int blocks = NSPLIT == 1 ? a.units : ((a.units + 7) / 8) * 8 * NSPLIT;
  return launch(linear_scan_bf16_kernel<MODE, ROWS, TPM, CKPT, DEPTH>, dim3(blocks),
                dim3(Geom<ROWS>::THREADS), s, a);
}

template <int MODE, int TPM, bool CKPT = false, int DEPTH = 0>
hipError_t launch_rows(const LinearArgs& a, int rows, hipStream_t s) {
  switch (rows) {
    case 64: return launch_one<MODE, 64, TPM, CKPT, DEPTH>(a, s);
    case 32: return launch_one<MODE, 32, TPM, CKPT, DEPTH>(a, s);
    default: return launch_one<MODE, 16, TPM, CKPT, DEPTH>(a, s);
  }
}

}  // namespace

// Chunked scan, combination step: for every unit, the start state of each
// chunk, from w0 and the previous chunks' affine maps W_end = W_start M + C
// (M: the chunk run from the identity with V = 0; C: run from zero), which
// the first passes left in z (M at the chunk's tokens 0..63, C at 64..127).
// The start states go to the chunk's last 64 tokens of z (chunk_state_in_z).
// Rows of the state are independent (row i of W_start M + C needs row i of
// W_start only), so a workgroup takes 8 rows of one unit; thread t owns row
// t / 32, columns 2 (t % 32) and 2 (t % 32) + 1.  The next chunk's M and C
// are loaded while the current step computes.
constexpr int COMBINE_ROWS = 8;
__global__ void __launch_bounds__(256) chunk_combine_kernel(const float* w0, int w0_per_batch, int H,
                                                            float* z, int Tc, int P, int rows) {
  __shared__ f32x4 Ms[2][64 * 16];        // M of the current and the next chunk
  __shared__ float Wr[COMBINE_ROWS][64];  // the rows' current start state
  const int u = blockIdx.x, row0 = blockIdx.y * COMBINE_ROWS, t = threadIdx.x;
  const int r = t >> 5, col = 2 * (t & 31);
  const float* w0u = w0 + (size_t)(w0_per_batch ? u : u % H) * 4096;
  for (int e = t; e < COMBINE_ROWS * 64; e += 256) Wr[e >> 6][e & 63] = w0u[(row0 + (e >> 6)) * 64 + (e & 63)];
  auto chunk = [&](int p) { return z + ((size_t)u * P + p) * Tc * 64; };
  // registers: this thread's quarter-rows of the next M (four float4) and its two C values
  f32x4 mnext[4];
  float2 cnext = make_float2(0.f, 0.f);
  auto fetch = [&](int p) {
    const float* zc = chunk(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) mnext[q] = *(const f32x4*)(zc + 4 * (t + 256 * q));
    cnext = *(const float2*)(zc + 4096 + (row0 + r) * 64 + col);
  };
  fetch(0);
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int q = 0; q < 4; ++q) Ms[p & 1][t + 256 * q] = mnext[q];
    const float2 cc = cnext;
    if (p + 1 < P - 1) fetch(p + 1);
    __syncthreads();  // Ms[p & 1] and Wr complete
    float* zc = chunk(p);
    for (int e = t; e < COMBINE_ROWS * 64; e += 256)
      zc[chunk_state_in_z(Tc, rows, row0 + (e >> 6), e & 63)] = Wr[e >> 6][e & 63];
    if (p == P - 1) break;
    const float* Mf = (const float*)Ms[p & 1];
    float a0 = cc.x, a1 = cc.y;
#pragma unroll 16
    for (int k = 0; k < 64; ++k) {
      const float w = Wr[r][k];
      const float2 m = *(const float2*)(Mf + k * 64 + col);
      a0 = fmaf(w, m.x, a0);
      a1 = fmaf(w, m.y, a1);
    }
    __syncthreads();  // Wr fully read
    Wr[r][col] = a0;
    Wr[r][col + 1] = a1;
  }
}

hipError_t launch_linear_chunked(const LinearArgs& a, int P, int rows, hipStream_t s) {
  const int Tc = a.T / P;
  if (P < 2 || a.T % P != 0 || Tc % 16 != 0 || Tc < 192 || a.b != 16) return hipErrorInvalidValue;
  LinearArgs c = a;
  c.units = a.units * P;  // chunk p of unit u is sequence u * P + p of length Tc
  c.T = Tc;
  c.z = nullptr;
  c.w_ckpt = nullptr;
  // M: from the identity with V = 0, into z's tokens 0..63 of each chunk
  c.v_zero = 1;
  c.w0_mode = W0_IDENTITY;
  c.w_out = a.z;
  c.wout_stride = Tc * 64;
  c.wout_every = 1;
  hipError_t e = launch_rows<MODE_B16, 1>(c, rows, s);
  if (e != hipSuccess) return e;
  // C: from zero with V, into tokens 64..127
  c.v_zero = 0;
  c.w0_mode = W0_ZERO;
  c.w_out = a.z + 64 * 64;
  e = launch_rows<MODE_B16, 1>(c, rows, s);
  if (e != hipSuccess) return e;
  e = launch(chunk_combine_kernel, dim3(a.units, 64 / COMBINE_ROWS), dim3(256), s, a.w0,
             a.w0_per_batch, a.H, a.z, Tc, P, rows);
  if (e != hipSuccess) return e;
  // every chunk from its start state, with outputs (and the checkpoints,
  // which are laid out per 16-token tile, so chunk u * P + p's are unit u's
  // tiles of that chunk); the last chunk's final state is the unit's
  c.z = a.z;
  c.w0_mode = W0_IN_Z;
  c.w_out = a.w_out;
  c.wout_stride = 4096;
  c.wout_every = P;
  if (a.w_ckpt) {
    c.w_ckpt = a.w_ckpt;
    return launch_rows<MODE_B16, 1, true>(c, rows, s);
  }
  return launch_rows<MODE_B16, 1>(c, rows, s);
}

hipError_t launch_linear_bf16(const LinearArgs& a, int rows, hipStream_t s) {
  if (a.w_ckpt) {
    if (a.b == 16 || (a.b < 16 && a.bt == a.b)) return launch_rows<MODE_B16, 1, true>(a, rows, s);
    if (a.b == 32) return launch_rows<MODE_MULTI, 2, true>(a, rows, s);
    if (a.b == 64) return launch_rows<MODE_MULTI, 4, true>(a, rows, s);
    if (a.b > 16 && a.b % 16 == 0) return launch_rows<MODE_MULTI, 0, true>(a, rows, s);
    return hipErrorInvalidValue;
  }
  if (a.ring_depth == 1) return a.b == 16 ? launch_rows<MODE_B16, 1, false, 1>(a, rows, s)
                                          : hipErrorInvalidValue;
  if (a.b == 16) return launch_rows<MODE_B16, 1>(a, rows, s);
  if (a.b < 16) return launch_rows<MODE_SUB, 1>(a, rows, s);
  if (a.b == 32) return launch_rows<MODE_MULTI, 2>(a, rows, s);
  if (a.b == 64) return launch_rows<MODE_MULTI, 4>(a, rows, s);
  return launch_rows<MODE_MULTI, 0>(a, rows, s);
}

}  // namespace ttt
