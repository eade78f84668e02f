// Backward of the TTT-Linear scan (b = 16), gfx950.
//
// Method ("论文速览 | TTT", equinox-blog close reading of "Learning to
// (Learn at Test Time)"): training differentiates through the inner loop;
// the forward keeps the state at the start of every mini-batch (the
// kappa = T / b checkpoints of §6.12) and the backward walks the mini-batches
// in reverse.  Per mini-batch (columns are tokens, D = diag(eta), W the
// checkpointed state, A = triu(K^T Q) with s <= t, §3.6):
//   forward   E = W K - V, G = 2 E D, Z = W Q - G A, W' = W - G K^T
//   backward  (Zb, Wb' the adjoints of Z and W'; the gradient of the loss
//             with respect to G is Gb = -(Wb' K + Zb A^T))
//     Gt = 2 (Wb' K + Zb A^T) D        (= dL/dV, and -dL/dE)
//     Wb = Wb' + Zb Q^T - Gt K^T       (the adjoint of W)
//     Ab = triu(-G^T Zb)
//     dQ = W^T Zb + K Ab
//     dK = -W^T Gt + Q Ab^T - Wb'^T G
//     deta_t = -sum_i (Wb' K + Zb A^T)[i, t] 2 E[i, t]
// The adjoint recurrence has the forward's form (rows of Wb evolve
// independently), the other outputs do not feed it.  Two kernels:
//   1. the reverse scan over 16-row slices of Wb: writes dV = Gt, the
//      adjoint at the end of every mini-batch (Wb', a checkpoint of its own)
//      and finally dW0 = Wb_0;
//   2. one workgroup per (unit, mini-batch), fully parallel: dQ, dK, deta
//      from W, Wb' and the tile's inputs.
// All products are fp32 MFMA (16x16x4: exact fp32 products, fp32 sums).
//
// MFMA 16x16x4 f32 operand layouts (wave64, lane (c, g), c = lane % 16,
// g = lane / 16): A-operand lane holds A[c][g], B-operand lane holds B[g][c],
// accumulator register r holds C[4g + r][c].  A contraction over 16 tokens
// whose values a lane holds in registers r (token 4g + r) runs as four MFMAs
// k = 0..3 taking token 4g + k from each lane group g: the token order in
// the reduction is permuted, and both operands use the same permutation.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

__device__ __forceinline__ float bf(const uint16_t* p) {
  return __builtin_bit_cast(float, ((uint32_t)*p) << 16);
}

// ========================================================= 1. reverse scan
// Workgroup = (unit, slice of 16 rows): wave 0 computes, wave 1 streams the
// tiles in reverse order into an LDS ring (buffer->LDS DMA, D tiles ahead).
struct BwdGeom {
  static constexpr int KB = 16 * 64 * 2;  // K or Q tile, bf16 [token][col]
  static constexpr int ZB = 16 * 16 * 4;  // this slice's dz rows, fp32 [token][row]
  static constexpr int RAW = 2 * KB + ZB + 64;
  static constexpr int NI = 2 + 2 + 1 + 1;  // DMA ops per tile
  static constexpr int D = 8;
  static constexpr int NST = D + 2;
};

__global__ void __launch_bounds__(128) linear_bwd_state_kernel(LinearBwdArgs a) {
  using G = BwdGeom;
  __shared__ __attribute__((aligned(16))) char smem[G::NST * G::RAW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x >> 2, slice = blockIdx.x & 3;
  if (unit >= a.units) return;
  const int T = a.T, ntiles = (T + 15) >> 4;
  const int rbase = slice * 16;

  if (wave == 1) {  // ------------------------------------------- loader
    const size_t uoff = (size_t)unit * T * 64;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const short*)a.k + uoff, (uint32_t)T * 128);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const short*)a.q + uoff, (uint32_t)T * 128);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.dz + uoff, (uint32_t)T * 256);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta + (size_t)unit * T, (uint32_t)T * 4);
    // iteration i handles tile ntiles - 1 - i
    auto issue = [&](int i) {
      const int j = ntiles - 1 - i;
      char* st = smem + (i % G::NST) * G::RAW;
      const uint32_t tb = (uint32_t)j * 2048;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        dma16(rk, st + n * 1024, tb + n * 1024 + lane * 16);
        dma16(rq, st + G::KB + n * 1024, tb + n * 1024 + lane * 16);
      }
      // dz[t][rbase .. rbase + 15]: token lane / 4, 16-byte part lane % 4
      dma16(rz, st + 2 * G::KB, (uint32_t)((j * 16 + (lane >> 2)) * 64 + rbase) * 4 + (lane & 3) * 16);
      if (lane < 16) dma4(re, st + 2 * G::KB + G::ZB, (uint32_t)(j * 16 + lane) * 4);
    };
    const int pro = ntiles < G::D ? ntiles : G::D;
    for (int i = 0; i < pro; ++i) issue(i);
    for (int i = 0; i < ntiles; ++i) {
      if (i + G::D < ntiles) {
        issue(i + G::D);
        wait_vmcnt<G::NI * G::D>();  // tiles <= i landed
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier();  // B_i
    }
    return;
  }

  // -------------------------------------------------------------- compute
  // Wb[cb] register r = Wb[row rbase + c][col 16 cb + 4g + r]
  f32x4 Wb[4];
  const size_t so = (size_t)unit * 4096 + (size_t)(rbase + c) * 64 + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    Wb[cb] = a.dw_T ? *(const f32x4*)(a.dw_T + so + 16 * cb) : f32x4{0, 0, 0, 0};
  const __amdgpu_buffer_rsrc_t rdv =
      make_rsrc(a.dv + (size_t)unit * T * 64, (uint32_t)T * 256);
  for (int i = 0; i < ntiles; ++i) {
    const int j = ntiles - 1 - i;
    wg_barrier();  // B_i: tile j is in LDS
    const char* st = smem + (i % G::NST) * G::RAW;
    const uint16_t* Kt = (const uint16_t*)st;               // [token][col]
    const uint16_t* Qt = (const uint16_t*)(st + G::KB);     // [token][col]
    const float* Zs = (const float*)(st + 2 * G::KB);       // [token][row - rbase]
    const float* Et = (const float*)(st + 2 * G::KB + G::ZB);

    // Wb' = the adjoint after tile j: the checkpoint kernel 2 reads
    float* ck = a.wb_ckpt + ((size_t)unit * ntiles + j) * 4096;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      *(f32x4*)(ck + (size_t)(rbase + c) * 64 + 16 * cb + 4 * g) = Wb[cb];

    // A^T: register r = A[s = c][t = 4g + r] = k_s . q_t, kept for s <= t
    f32x4 At = {0, 0, 0, 0};
    for (int kk = 0; kk < 16; ++kk)
      At = mfma_f32(bf(Qt + c * 64 + 4 * kk + g), bf(Kt + c * 64 + 4 * kk + g), At);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (c > 4 * g + r) At[r] = 0.f;
    // M = Zb A^T: register r = M[row c][s = 4g + r]
    f32x4 M = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) M = mfma_f32(At[k], Zs[(4 * g + k) * 16 + c], M);
    // P = Wb' K: register r = P[row c][s = 4g + r]
    f32x4 P = {0, 0, 0, 0};
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) P = mfma_f32(bf(Kt + c * 64 + 16 * cb + 4 * g + r), Wb[cb][r], P);
    // Gt = 2 (P + M) D = dL/dV
    const f32x4 e4 = *(const f32x4*)(Et + 4 * g);
    f32x4 Gt;
#pragma unroll
    for (int r = 0; r < 4; ++r) Gt[r] = 2.f * e4[r] * (P[r] + M[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gv = Gt[r];  // bit_cast of a vector element itself reads element 0
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gv), rdv,
                                            (uint32_t)((j * 16 + 4 * g + r) * 64 + rbase + c) * 4, 0, 0);
    }
    // Wb += Zb Q^T - Gt K^T: accumulator cb, register r = [col 16 cb + 4g + r][row c]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = 4 * g + k;
        Wb[cb] = mfma_f32(bf(Qt + t * 64 + 16 * cb + c), Zs[t * 16 + c], Wb[cb]);
        Wb[cb] = mfma_f32(-bf(Kt + t * 64 + 16 * cb + c), Gt[k], Wb[cb]);
      }
  }
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) *(f32x4*)(a.dw0 + so + 16 * cb) = Wb[cb];
}

// ==================================================== 2. per-tile outputs
// Workgroup = (unit, tile j), four waves.  Wave w computes rows 16w .. +15
// of E, Gb and columns 16w .. +15 of dQ, dK.
__global__ void __launch_bounds__(256) linear_bwd_out_kernel(LinearBwdArgs a) {
  __shared__ float sW[64 * 64], sWb[64 * 64];  // W, Wb' [row][col]
  __shared__ float sK[16 * 64], sQ[16 * 64], sV[16 * 64], sZ[16 * 64];  // [token][col]
  __shared__ float sG[64 * 16], sGt[64 * 16];  // G, Gt [row][token]
  __shared__ float sEta[16], sDeta[4][16];
  const int T = a.T, ntiles = (T + 15) >> 4;
  const int unit = blockIdx.x / ntiles, j = blockIdx.x % ntiles;
  if (unit >= a.units) return;
  const int t0 = j * 16, nt = T - t0 < 16 ? T - t0 : 16;  // valid tokens of the tile
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;

  {  // stage the tile (tokens past T read as zero)
    const float4* w = (const float4*)(a.w_ckpt + ((size_t)unit * ntiles + j) * 4096);
    const float4* wb = (const float4*)(a.wb_ckpt + ((size_t)unit * ntiles + j) * 4096);
    for (int e = tid; e < 1024; e += 256) {
      ((float4*)sW)[e] = w[e];
      ((float4*)sWb)[e] = wb[e];
    }
    const size_t vo = ((size_t)unit * T + t0) * 64;
    for (int e = tid; e < 1024; e += 256) {
      const int t = e >> 6;
      const bool ok = t < nt;
      sK[e] = ok ? bf((const uint16_t*)a.k + vo + e) : 0.f;
      sQ[e] = ok ? bf((const uint16_t*)a.q + vo + e) : 0.f;
      sV[e] = ok ? bf((const uint16_t*)a.v + vo + e) : 0.f;
      sZ[e] = ok ? a.dz[vo + e] : 0.f;
    }
    if (tid < 16) sEta[tid] = tid < nt ? a.eta[(size_t)unit * T + t0 + tid] : 0.f;
  }
  __syncthreads();

  // ---- rows 16w + 4g + r, token c (accumulator layout [row][token])
  const int rw = 16 * wave;
  f32x4 E = {0, 0, 0, 0}, Pn = {0, 0, 0, 0};  // W K, Wb' K
  for (int kk = 0; kk < 16; ++kk) {
    const float kv = sK[c * 64 + 4 * kk + g];
    E = mfma_f32(sW[(rw + c) * 64 + 4 * kk + g], kv, E);
    Pn = mfma_f32(sWb[(rw + c) * 64 + 4 * kk + g], kv, Pn);
  }
  // A^T: register r = A[s = c][t = 4g + r] (s <= t)
  f32x4 At = {0, 0, 0, 0};
  for (int kk = 0; kk < 16; ++kk)
    At = mfma_f32(sQ[c * 64 + 4 * kk + g], sK[c * 64 + 4 * kk + g], At);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (c > 4 * g + r) At[r] = 0.f;
  // Zb A^T [row][s] = sum_t Zb[row][t] A[s][t] needs A with s in the lanes
  // of the B operand: wave 0 stores A[s][t] to LDS.
  __shared__ float sA[16 * 16];
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sA[c * 16 + 4 * g + r] = At[r];
  }
  __syncthreads();
  f32x4 M = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    M = mfma_f32(sZ[(4 * k + g) * 64 + rw + c], sA[c * 16 + 4 * k + g], M);
  // E = W K - V; Gn = Wb' K + Zb A^T (= -Gb); G = 2 E D; Gt = 2 Gn D
  float dpart = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = rw + 4 * g + r;
    const float e = E[r] - sV[c * 64 + row];
    const float gn = Pn[r] + M[r];
    sG[row * 16 + c] = 2.f * sEta[c] * e;
    sGt[row * 16 + c] = 2.f * sEta[c] * gn;
    dpart -= gn * 2.f * e;
  }
  // deta_t = -sum_rows Gn 2 E: fold the 4 rows of the lane, then the 4 lane
  // groups and the 4 waves
  dpart += __shfl_xor(dpart, 16);
  dpart += __shfl_xor(dpart, 32);
  if (g == 0) sDeta[wave][c] = dpart;
  __syncthreads();
  if (tid < nt)
    a.deta[(size_t)unit * T + t0 + tid] =
        (sDeta[0][tid] + sDeta[1][tid]) + (sDeta[2][tid] + sDeta[3][tid]);

  // ---- Ab = triu(-G^T Zb) [s][t]: register r = Ab[s = 4g + r][t = c]; and
  // its transpose AbT register r = Ab[s = c][t = 4g + r]
  f32x4 Ab = {0, 0, 0, 0}, AbT = {0, 0, 0, 0};
  for (int kk = 0; kk < 16; ++kk) {
    const int row = 4 * kk + g;
    Ab = mfma_f32(sG[row * 16 + c], sZ[c * 64 + row], Ab);
    AbT = mfma_f32(sZ[c * 64 + row], sG[row * 16 + c], AbT);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    Ab[r] = (4 * g + r <= c) ? -Ab[r] : 0.f;
    AbT[r] = (c <= 4 * g + r) ? -AbT[r] : 0.f;
  }

  // ---- columns 16w + 4g + r, token c (accumulator layout [col][token])
  const int cw = 16 * wave;
  f32x4 dQ = {0, 0, 0, 0}, dK = {0, 0, 0, 0};
  for (int kk = 0; kk < 16; ++kk) {
    const int row = 4 * kk + g;
    const float w = sW[row * 64 + cw + c];
    dQ = mfma_f32(w, sZ[c * 64 + row], dQ);                 // W^T Zb
    dK = mfma_f32(-w, sGt[row * 16 + c], dK);                // -W^T Gt
    dK = mfma_f32(-sWb[row * 64 + cw + c], sG[row * 16 + c], dK);  // -Wb'^T G
  }
  // + K Ab (contraction over s = 4g + k, Ab in registers of lane group g)
  // + Q Ab^T: dK[col][s] += sum_t Q[col][t] Ab[s][t], t = 4g + k
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    dQ = mfma_f32(sK[(4 * g + k) * 64 + cw + c], Ab[k], dQ);
    dK = mfma_f32(sQ[(4 * g + k) * 64 + cw + c], AbT[k], dK);
  }
  // register r = d?[col cw + 4g + r][token c]: one 16-byte store per lane
  if (c < nt) {
    const size_t o = ((size_t)unit * T + t0 + c) * 64 + cw + 4 * g;
    *(f32x4*)(a.dq + o) = dQ;
    *(f32x4*)(a.dk + o) = dK;
  }
}

}  // namespace

hipError_t launch_linear_bwd(const LinearBwdArgs& a, hipStream_t s) {
  const int ntiles = (a.T + 15) / 16;
  hipLaunchKernelGGL(linear_bwd_state_kernel, dim3(a.units * 4), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ntiles == 0) return hipSuccess;  // dw0 = dw_T (or 0): nothing per tile
  hipLaunchKernelGGL(linear_bwd_out_kernel, dim3(a.units * ntiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
