// TTT-Linear forward scan for gfx950 (MI355X), mini-batch TTT in dual form:
// the fp32-input kernel (bf16 inputs take ttt_linear_bf16.hip).
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): §3.5 mini-batch GD with the gradient point at the
// state before the mini-batch, §3.6 dual form
//   W_b = W0 - 2 (W0 K - V) diag(eta) K^T,   Z = W0 Q - 2 (W0 K - V) diag(eta) triu(K^T Q),
// with the per-token eta of §4.6 and f(x) = W x (§4.4).  The causal mask keeps
// s <= t, so token t's output sees its own update (§3.1).
//
// Design (one GPU, one workgroup per (batch, head, slice of ROWS rows of W)):
//  * Rows of W evolve independently (the loss is a sum over output
//    components), so the 64 rows of a head are split over NCW = ROWS/16
//    compute waves; each wave owns 16 rows and keeps them in fp32 in MFMA
//    accumulator registers for the whole sequence.
//  * A separate loader wave streams 16-token tiles of K, Q, V (this slice's
//    columns) and eta from HBM into an LDS ring with buffer->LDS DMA, D tiles
//    ahead.  Buffer range checks zero-fill tokens past T (eta = 0 there, so a
//    padded token contributes nothing).
//  * Per 16-token tile each compute wave runs, on MFMA:
//      P^T = K^T W^T, R^T = Q^T W^T           (64x16x16, fp32 16x16x4 MFMA)
//      A   = triu(K^T Q)                       (16x16x64, fp32 MFMA)
//      Gn  = 2 (V - P) diag(eta)               (VALU; "negative gradient")
//      Z^T = R^T + A^T Gn^T                    (16x16x16, fp32 MFMA)
//      W^T += K Gn^T                           (rank-16 update into the fp32
//                                               accumulator that holds W)
//    The update's accumulator layout is reused directly as the next tile's
//    operand by permuting the reduction index (see ttt_device.h).
//  * Mini-batches b < 16 (b | 16) are solved inside the tile: the gradients of
//    the b-sized sub-batches satisfy G (I + N) = E with E the gradients at the
//    tile's starting state and N[s][t] = 2 eta_t k_s.k_t for s in an earlier
//    sub-batch than t, so G = E (I + N)^-1 with the nilpotent series
//    (I - N)(I + N^2)(I + N^4)(I + N^8) computed on MFMA.  b > 16 (16 | b)
//    keeps the gradient point's operand split across the tiles of a
//    mini-batch.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {

enum { MODE_B16 = 0, MODE_SUB = 1, MODE_MULTI = 2 };

template <int ROWS>
struct LinearGeom {
  static constexpr int NCW = ROWS / 16;          // compute waves
  static constexpr int ES = 4;                   // bytes per q/k/v element (fp32)
  static constexpr int KB = 16 * 64 * ES;        // K (or Q) tile bytes
  static constexpr int VB = 16 * ROWS * ES;      // V tile bytes (this slice)
  static constexpr int EB = 64;                  // eta tile bytes
  static constexpr int STAGE = 2 * KB + VB + EB; // one ring slot
  static constexpr int NI = 2 * (KB / 1024) + (VB + 1023) / 1024 + 1;  // DMA ops per tile
  static constexpr int D = (63 / NI) < 9 ? (63 / NI) : 9;             // tiles in flight
  static constexpr int NST = D + 2;              // ring slots (see loader comment)
  static constexpr int THREADS = (NCW + 1) * 64;
};

template <int MODE, int ROWS>
__global__ void __launch_bounds__((LinearGeom<ROWS>::THREADS))
linear_scan_kernel(LinearArgs a) {
  using G = LinearGeom<ROWS>;
  constexpr int NSPLIT = 64 / ROWS;
  __shared__ __attribute__((aligned(16))) char smem[G::NST * G::STAGE];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;

  // Workgroup -> (unit, slice).  Slices of one unit share an XCD (its L2),
  // since consecutive workgroup ids are dealt round-robin over the 8 XCDs.
  int unit, slice;
  if (NSPLIT == 1) {
    unit = blockIdx.x;
    slice = 0;
  } else {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    slice = slot % NSPLIT;
    unit = (slot / NSPLIT) * 8 + xcd;
  }
  if (unit >= a.units) return;
  const int head = unit % a.H;
  const int T = a.T;
  const int ntiles = (T + 15) >> 4;
  const int row0 = slice * ROWS;  // first row of W handled by this workgroup

  if (wave == G::NCW) {
    // ------------------------------------------------------------ loader
    // Ring discipline: tile j lives in slot j % NST.  Tile j+D is issued at
    // iteration j, after barrier j-1, when the compute waves are done with
    // tile j-2 (they finished it before arriving at barrier j-1) and may be
    // reading tile j-1; NST = D + 2 keeps those slots apart.
    const size_t ubytes = (size_t)T * 64 * G::ES;
    const char* kb = (const char*)a.k + (size_t)unit * ubytes;
    const char* qb = (const char*)a.q + (size_t)unit * ubytes;
    const char* vb = (const char*)a.v + (size_t)unit * ubytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)ubytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)ubytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)ubytes);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    auto issue = [&](int j) {
      char* st = smem + (j % G::NST) * G::STAGE;
      const uint32_t tb = (uint32_t)j * 16 * 64 * G::ES;
#pragma unroll
      for (int n = 0; n < G::KB / 1024; ++n) dma16(rk, st + n * 1024, tb + n * 1024 + lane * 16);
#pragma unroll
      for (int n = 0; n < G::KB / 1024; ++n)
        dma16(rq, st + G::KB + n * 1024, tb + n * 1024 + lane * 16);
#pragma unroll
      for (int n = 0; n < (G::VB + 1023) / 1024; ++n) {
        const int byte = n * 1024 + lane * 16;
        if (G::VB % 1024 == 0 || byte < G::VB) {
          const int tok = byte / (ROWS * G::ES), cb = byte % (ROWS * G::ES);
          dma16(rv, st + 2 * G::KB + n * 1024,
                (uint32_t)(j * 16 + tok) * 64 * G::ES + row0 * G::ES + cb);
        }
      }
      if (lane < 16) dma4(re, st + 2 * G::KB + G::VB, (uint32_t)(j * 16 + lane) * 4);
    };
    const int pro = ntiles < G::D ? ntiles : G::D;
    for (int j = 0; j < pro; ++j) issue(j);
    for (int j = 0; j < ntiles; ++j) {
      if (j + G::D < ntiles) {
        issue(j + G::D);
        wait_vmcnt<G::NI * G::D>();
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier();
    }
    return;
  }

  // -------------------------------------------------------------- compute
  const int rbase = row0 + wave * 16;  // first W row of this wave
  const float* w0 = a.w0 + (size_t)(a.w0_per_batch ? unit : head) * 4096;
  f32x4 W[4];  // W[m][r] = W[rbase + c][16 m + 4 g + r]
#pragma unroll
  for (int m = 0; m < 4; ++m)
    W[m] = *(const f32x4*)(w0 + (rbase + c) * 64 + 16 * m + 4 * g);

  // SUB mode: index of the sub-batch that token 4g+r / token c belongs to.
  const int bsub = a.b;
  f32x4 gpf[4];  // MULTI mode: the gradient point, fixed over a mini-batch
  const int tiles_per_mb = MODE == MODE_MULTI ? (a.b >> 4) : 1;

  float* zu = a.z + (size_t)unit * T * 64;

  for (int j = 0; j < ntiles; ++j) {
    wg_barrier();
    const char* st = smem + (j % G::NST) * G::STAGE;
    const char* Kt = st;
    const char* Qt = st + G::KB;
    const char* Vt = st + 2 * G::KB;
    const float* Et = (const float*)(st + 2 * G::KB + G::VB);

    const f32x4 eta4 = *(const f32x4*)(Et + 4 * g);  // eta of tokens 4g .. 4g+3
    float vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int off = (4 * g + r) * ROWS + wave * 16 + c;
      vv[r] = ((const float*)Vt)[off];
    }

    f32x4 P = {0, 0, 0, 0}, R = {0, 0, 0, 0}, A = {0, 0, 0, 0}, M = {0, 0, 0, 0};
    f32x4 kop[4], qop[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kop[m] = *(const f32x4*)(Kt + (c * 64 + 16 * m + 4 * g) * 4);
      qop[m] = *(const f32x4*)(Qt + (c * 64 + 16 * m + 4 * g) * 4);
    }
    if constexpr (MODE == MODE_MULTI) {
      if (j % tiles_per_mb == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) gpf[m] = W[m];
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 wp = MODE == MODE_MULTI ? gpf[m] : W[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        P = mfma_f32(kop[m][e], wp[e], P);
        R = mfma_f32(qop[m][e], W[m][e], R);
        A = mfma_f32(kop[m][e], qop[m][e], A);
        if constexpr (MODE == MODE_SUB) M = mfma_f32(kop[m][e], kop[m][e], M);
      }
    }

    // A[s = 4g+r][t = c], causal (inclusive) mask
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > c) A[r] = 0.f;

    // Negative gradient at the tile's gradient point: E[t=4g+r][i=c]
    f32x4 Gn;
#pragma unroll
    for (int r = 0; r < 4; ++r) Gn[r] = 2.f * eta4[r] * (vv[r] - P[r]);

    if constexpr (MODE == MODE_SUB) {
      // N[s][t] = 2 eta_t (k_s . k_t) if sub-batch(s) < sub-batch(t)
      const float eta_c = Et[c];
      f32x4 N, NT, I;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * g + r;
        N[r] = (s / bsub < c / bsub) ? 2.f * eta_c * M[r] : 0.f;
        NT[r] = (c / bsub < s / bsub) ? 2.f * eta4[r] * M[r] : 0.f;  // M symmetric
        I[r] = (s == c) ? 1.f : 0.f;
      }
      const f32x4 Z0 = {0, 0, 0, 0};
      auto mm = [&](f32x4 xt, f32x4 y) { return mm16_f32(xt, y, Z0); };
      // U = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), cut at N^nblk = 0
      const int nblk = 16 / bsub;
      f32x4 U;
      if (nblk == 2) {
        U = I - N;
      } else {
        const f32x4 N2 = mm(NT, N), N2T = mm(N, NT);
        f32x4 tail;  // (I + N^2)(I + N^4)(I + N^8), truncated
        if (nblk == 4) {
          tail = I + N2;
        } else {
          const f32x4 N4 = mm(N2T, N2);
          f32x4 t4;  // (I + N^4)(I + N^8), truncated
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
      // G = E U  <=>  G^T = U^T E^T : A-operand = accumulator layout of U
      Gn = mm16_f32(U, Gn, Z0);
    }

    // ---- rank-16 update of the resident state and the outputs
    f32x4 Zt = R;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        W[m] = mfma_f32(((const float*)Kt)[(4 * g + e) * 64 + 16 * m + c], Gn[e], W[m]);
    Zt = mm16_f32(A, Gn, Zt);

    // Z[t][i]: lane (c,g) holds tokens 16j + 4g + r of row rbase + c
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = j * 16 + 4 * g + r;
      if (t < T) zu[(size_t)t * 64 + rbase + c] = Zt[r];
    }
  }

  float* wo = a.w_out + (size_t)unit * 4096;
#pragma unroll
  for (int m = 0; m < 4; ++m) *(f32x4*)(wo + (rbase + c) * 64 + 16 * m + 4 * g) = W[m];
}

template <int MODE, int ROWS>
static hipError_t launch_one(const LinearArgs& a, hipStream_t s) {
  using G = LinearGeom<ROWS>;
  constexpr int NSPLIT = 64 / ROWS;
  int blocks = NSPLIT == 1 ? a.units : ((a.units + 7) / 8) * 8 * NSPLIT;
  return launch(linear_scan_kernel<MODE, ROWS>, dim3(blocks), dim3(G::THREADS), s, a);
}

template <int MODE>
static hipError_t launch_rows(const LinearArgs& a, int rows, hipStream_t s) {
  switch (rows) {
    case 64: return launch_one<MODE, 64>(a, s);
    case 32: return launch_one<MODE, 32>(a, s);
    default: return launch_one<MODE, 16>(a, s);
  }
}

hipError_t launch_linear(const LinearArgs& a, bool f32in, int rows, hipStream_t s) {
  if (!f32in) return launch_linear_bf16(a, rows, s);
  const int mode = a.b == 16 ? MODE_B16 : (a.b < 16 ? MODE_SUB : MODE_MULTI);
  if (mode == MODE_B16) return launch_rows<MODE_B16>(a, rows, s);
  if (mode == MODE_SUB) return launch_rows<MODE_SUB>(a, rows, s);
  return launch_rows<MODE_MULTI>(a, rows, s);
}

}  // namespace ttt
