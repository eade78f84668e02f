// Learnable inner learning rate ("论文速览 | TTT", §4.6), gfx950:
//   eta[b][h][t] = eta_base * sigmoid(theta_lr[h] . x[b][t])
// for every token of the layer input x [B][T][dx] (bf16) and every head's gate
// vector theta_lr [H][dx] (fp32), written in the scans' eta layout [B][H][T].
//
// It is a skinny product (tokens x dx) . (dx x H) with a sigmoid epilogue,
// bound by the one pass over x.  Workgroup = 16 * TB tokens, four waves that
// split dx (wave w takes the 32-wide steps w, w + 4, ...), all heads in passes
// of 32; the four partial sums meet in LDS, where the epilogue also turns the
// [head][token] tiles into [b][h][t] rows.
//
// Products on the matrix unit: 16x16x32 bf16 MFMA with A = theta (heads x dx),
// B = x^T (dx x tokens).  x is exact in bf16; theta is split into three bf16
// terms hi + mid + lo (fp32 to within 2^-24 relative), so every product is
// exact and the sums are fp32.
//
// 16x16x32 bf16 operand layouts (wave64, lane (c, g), c = lane % 16,
// g = lane / 16): A lane holds A[c][8g .. 8g + 7], B lane holds
// B[8g .. 8g + 7][c], accumulator register r holds C[4g + r][c].
#include <algorithm>

#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
namespace {

constexpr int GATE_HP = 32;  // heads per pass: two 16-row blocks

struct Theta3 {
  bf16x8 hi, mid, lo;
};

// Eight fp32 values -> three bf16 terms (each the nearest-even rounding of
// what the previous terms leave; the residual subtractions are exact).
__device__ __forceinline__ Theta3 split3(float4 a, float4 b) {
  float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t p[3][4];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[k][e] = pack_rne(r[2 * e], r[2 * e + 1]);
      r[2 * e] -= __builtin_bit_cast(float, p[k][e] << 16);
      r[2 * e + 1] -= __builtin_bit_cast(float, p[k][e] & 0xffff0000u);
    }
  Theta3 t;
  t.hi = __builtin_bit_cast(bf16x8, make_uint4(p[0][0], p[0][1], p[0][2], p[0][3]));
  t.mid = __builtin_bit_cast(bf16x8, make_uint4(p[1][0], p[1][1], p[1][2], p[1][3]));
  t.lo = __builtin_bit_cast(bf16x8, make_uint4(p[2][0], p[2][1], p[2][2], p[2][3]));
  return t;
}

template <int TB>
__global__ void __launch_bounds__(256) lr_gate_kernel(GateArgs a) {
  constexpr int TOK = 16 * TB;
  constexpr int PITCH = TOK + 4;  // words per LDS row: the four lane groups hit distinct banks
  __shared__ float red[4][GATE_HP][PITCH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t ntok = (int64_t)a.B * a.T;
  const int64_t f0 = (int64_t)blockIdx.x * TOK;
  const int ksteps = a.dx >> 5;

  // this lane's x rows (tokens past the end re-read the last token; their
  // sums are never stored)
  const bf16x8* xr[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    int64_t f = f0 + 16 * tb + c;
    if (f >= ntok) f = ntok - 1;
    xr[tb] = (const bf16x8*)((const uint16_t*)a.x + f * a.dx + 8 * g);
  }

  for (int hp = 0; hp < a.H; hp += GATE_HP) {
    const int nhb = a.H - hp > 16 ? 2 : 1;  // head blocks in this pass (wave-uniform)
    const float* th[2];
    bool hv[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = hp + 16 * hb + c;
      hv[hb] = h < a.H;
      th[hb] = a.theta + (size_t)(hv[hb] ? h : 0) * a.dx + 8 * g;
    }
    f32x4 acc[2][TB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[hb][tb] = f32x4{0, 0, 0, 0};

    // one 32-wide step of x and theta in flight ahead of the one in use
    bf16x8 xv[TB];
    float4 tv[2][2];
    auto load = [&](int ks, bf16x8* xd, float4 (*td)[2]) {
      const int k0 = ks * 32;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) xd[tb] = xr[tb][k0 >> 3];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        td[hb][0] = make_float4(0.f, 0.f, 0.f, 0.f);
        td[hb][1] = td[hb][0];
        if (hb < nhb && hv[hb]) {
          td[hb][0] = *(const float4*)(th[hb] + k0);
          td[hb][1] = *(const float4*)(th[hb] + k0 + 4);
        }
      }
    };
    if (wave < ksteps) load(wave, xv, tv);
    for (int ks = wave; ks < ksteps; ks += 4) {
      bf16x8 xn[TB];
      float4 tn[2][2];
      if (ks + 4 < ksteps) load(ks + 4, xn, tn);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (hb < nhb) {
          const Theta3 s = split3(tv[hb][0], tv[hb][1]);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[hb][tb] = mfma_k32(s.hi, xv[tb], acc[hb][tb]);
            acc[hb][tb] = mfma_k32(s.mid, xv[tb], acc[hb][tb]);
            acc[hb][tb] = mfma_k32(s.lo, xv[tb], acc[hb][tb]);
          }
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) xv[tb] = xn[tb];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        tv[hb][0] = tn[hb][0];
        tv[hb][1] = tn[hb][1];
      }
    }
    // register r of acc[hb][tb] = partial sum of head hp + 16 hb + 4g + r, token 16 tb + c
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][16 * hb + 4 * g + r][16 * tb + c] = acc[hb][tb][r];
    __syncthreads();
    // epilogue: thread -> (token i, heads j0, j0 + 256 / TOK, ...)
    const int i = threadIdx.x % TOK;
    const int64_t f = f0 + i;
    if (f < ntok) {
      const int64_t bi = f / a.T, t = f - bi * a.T;
      for (int hl = threadIdx.x / TOK; hl < GATE_HP; hl += 256 / TOK) {
        const int h = hp + hl;
        if (h >= a.H) break;
        const float s = (red[0][hl][i] + red[1][hl][i]) + (red[2][hl][i] + red[3][hl][i]);
        a.eta[((size_t)bi * a.H + h) * a.T + t] = a.eta_base / (1.f + expf(-s));
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_lr_gate(const GateArgs& a, int tokens_per_workgroup, hipStream_t s) {
  const int64_t ntok = (int64_t)a.B * a.T;
  if (ntok == 0 || a.H == 0) return hipSuccess;
  if (tokens_per_workgroup == 0) tokens_per_workgroup = ntok >= 256 * 64 ? 64 : 32;
  switch (tokens_per_workgroup) {
    case 32: return launch(lr_gate_kernel<2>, dim3((unsigned)((ntok + 31) / 32)), dim3(256), s, a);
    case 64: return launch(lr_gate_kernel<4>, dim3((unsigned)((ntok + 63) / 64)), dim3(256), s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt

// ============================================================== backward
// dL/da = dL/deta * eta (1 - eta / eta_base) (= eta_base sigmoid' (a)), from
// the forward's eta, so the logits need not be recomputed;
//   dtheta_lr[h] = sum_{b,t} da[b][h][t] x[b][t],   dx[b][t] = sum_h da[b][h][t] theta_lr[h].
namespace ttt {
namespace {

// Inputs of da for one 16-token block in the dtheta layout: lane (c, g) holds
// tokens f0 + 4g .. f0 + 4g + 3 of head hp + 16 hb + c (eta and deta).
template <int HB>
struct DaQuad {
  f32x4 e[HB], de[HB];
};

// Loads from clamped (always valid) positions; masking happens on use.  eta
// and deta come through buffer descriptors with 32-bit byte offsets
// (B * T * H < 2^30).  VEC: T % 4 == 0, so a group of four tokens lies in
// one sequence and its four values are one aligned 16-byte load.
template <int HB, bool VEC>
__device__ __forceinline__ void load_da_quad(const GateBwdArgs& a, __amdgpu_buffer_rsrc_t re,
                                             __amdgpu_buffer_rsrc_t rd, int f0, int hp, int c, int g,
                                             DaQuad<HB>& o) {
  const int ntok = a.B * a.T;
  if constexpr (VEC) {
    const int fq = min(f0 + 4 * g, ntok - 4);
    const int bi = fq / a.T, t = fq - bi * a.T;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = min(hp + 16 * hb + c, a.H - 1);
      const uint32_t off = (uint32_t)((bi * a.H + h) * a.T + t) * 4u;
      o.e[hb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(re, off, 0, 0));
      o.de[hb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = min(f0 + 4 * g + r, ntok - 1);
      const int bi = f / a.T, t = f - bi * a.T;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = min(hp + 16 * hb + c, a.H - 1);
        const uint32_t off = (uint32_t)((bi * a.H + h) * a.T + t) * 4u;
        o.e[hb][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, off, 0, 0));
        o.de[hb][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, off, 0, 0));
      }
    }
  }
}

// One pipeline stage of the dtheta kernel: the x rows and da inputs of one block.
template <int NM, int HB>
struct DthStage {
  bf16x8 xr[(NM + 1) / 2];
  DaQuad<HB> da;
};

// Partial sums of dtheta over one chunk of tokens, for 16 * NM columns and
// the 16 * HB heads from hp on (one launch per pass): part[chunk][h][col].
// Four waves take interleaved 16-token blocks (J each, J a multiple of 3) and
// meet in LDS.
// Products on the matrix unit: x exact in bf16, brought to tokens-in-
// registers by a one-hot selection MFMA (exact), da as hi + lo.  The block
// loads run two blocks ahead in three rotating register sets (so no copy of
// a register that a load still writes); x rows come through a buffer
// descriptor over the block's rows inside the chunk, so rows past the chunk
// read as zeros without a branch.
template <int NM, int HB, bool VEC>
__global__ void __launch_bounds__(256) lr_gate_bwd_dtheta_kernel(GateBwdArgs a, float* part, int J,
                                                                 int hp) {
  __shared__ f32x4 red[4][HB][NM][64];
  // wave index as a scalar: the buffer descriptors built from it stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int ntok = a.B * a.T;
  const int col0 = blockIdx.x * 16 * NM;
  const int f_begin = blockIdx.y * 64 * J;
  const int f_end = min(ntok, f_begin + 64 * J);
  const float inv_base = a.eta_base != 0.f ? 1.f / a.eta_base : 0.f;
  // one-hot selectors: picks column 16p + c out of a 32-column chunk
  bf16x8 sel[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[p][e] = (bf16)((g == 2 * p + (c >> 3) && e == (c & 7)) ? 1.f : 0.f);
  // x rows are loaded whole (CPR 16-byte chunks per row, 64 / CPR rows per
  // load, so each load moves 1 KB of rows of 32 NM bytes) and rearranged into
  // the matrix unit's layout (lane (c, g): token c, chunk 4h + g) through a
  // per-wave LDS tile that shares the reduction buffer (used only after the
  // loop, each wave in its own part)
  constexpr int CPR = 2 * NM, RPI = 64 / CPR, PITCH = 16 * CPR + 16;
  const int lrow = lane / CPR, lchunk = lane % CPR;
  const uint32_t xoff = (uint32_t)((lrow * a.dx + col0) * 2 + 16 * lchunk);
  char* const xt_lds = (char*)&red[wave][0][0][0];
  static_assert(16 * PITCH <= (int)sizeof(red[0]), "staging tile fits the wave's reduction slot");
  const uint32_t ebytes = (uint32_t)(ntok * a.H) * 4u;
  const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta, ebytes), rd = make_rsrc(a.deta, ebytes);

  {
    f32x4 acc[HB][NM];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[hb][m] = f32x4{0, 0, 0, 0};

    // block j of this wave starts at token f_begin + 16 (wave + 4 j)
    auto load = [&](int j, DthStage<NM, HB>& st) {
      const int f0 = f_begin + 16 * (wave + 4 * j);
      // (uniform values pinned to scalar registers: a descriptor built from
      // a vector register would be split into a loop over distinct values)
      const int rows = __builtin_amdgcn_readfirstlane(min(max(f_end - f0, 0), 16));
      const int frow = __builtin_amdgcn_readfirstlane(min(f0, ntok));
      const __amdgpu_buffer_rsrc_t rx =
          make_rsrc((const uint16_t*)a.x + (int64_t)frow * a.dx, (uint32_t)(rows * a.dx * 2));
#pragma unroll
      for (int h = 0; h < (NM + 1) / 2; ++h)
        st.xr[h] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            rx, xoff + (uint32_t)(RPI * h * a.dx * 2), 0, 0));  // rows lrow + RPI h
      load_da_quad<HB, VEC>(a, re, rd, min(f0, ntok - 1), hp, c, g, st.da);
    };
    auto compute = [&](int j, const DthStage<NM, HB>& st) {
      const int f0 = f_begin + 16 * (wave + 4 * j);
      // tokens in registers: xt[m] register r = x[f0 + 4g + r][col0 + 16 m + c]
      // whole rows -> LDS tile -> lane (c, g) gets token c, columns 32 h + 8 g .. + 7
#pragma unroll
      for (int h = 0; h < (NM + 1) / 2; ++h)
        *(bf16x8*)(xt_lds + (lrow + RPI * h) * PITCH + 16 * lchunk) = st.xr[h];
      bf16x8 xa[(NM + 1) / 2];
#pragma unroll
      for (int h = 0; h < (NM + 1) / 2; ++h) xa[h] = *(const bf16x8*)(xt_lds + c * PITCH + 16 * (4 * h + g));
      uint2 xt[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 v = mfma_k32(xa[m >> 1], sel[m & 1], f32x4{0, 0, 0, 0});
        xt[m] = make_uint2(pack_rne(v[0], v[1]), pack_rne(v[2], v[3]));
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const bool hok = hp + 16 * hb + c < a.H;
        f32x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = st.da.e[hb][r];
          const float v = st.da.de[hb][r] * e * (1.f - e * inv_base);
          d[r] = (hok && f0 + 4 * g + r < f_end) ? v : 0.f;
        }
        const Split4 ds = split4(d);
        const bf16x8 dop = cat44(ds.hi, ds.lo);
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[hb][m] = mfma_k32(dop, cat8(xt[m], xt[m]), acc[hb][m]);
      }
    };
    // scheduling fences keep each set's loads where they stand, so a set is
    // never reloaded while its previous contents are still being read
    DthStage<NM, HB> sa, sb, sc;
    load(0, sa);
    load(1, sb);
    for (int j = 0; j < J; j += 3) {
      __builtin_amdgcn_sched_barrier(0);
      load(j + 2, sc);
      __builtin_amdgcn_sched_barrier(0);
      compute(j, sa);
      __builtin_amdgcn_sched_barrier(0);
      load(j + 3, sa);
      __builtin_amdgcn_sched_barrier(0);
      compute(j + 1, sb);
      __builtin_amdgcn_sched_barrier(0);
      load(j + 4, sb);
      __builtin_amdgcn_sched_barrier(0);
      compute(j + 2, sc);
    }

    // register r of acc[hb][m] = sum over this wave's tokens for head
    // hp + 16 hb + 4g + r, column col0 + 16 m + c
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int m = 0; m < NM; ++m) red[wave][hb][m][lane] = acc[hb][m];
    __syncthreads();
    for (int q = wave; q < HB * NM; q += 4) {
      const int hb = q / NM, m = q % NM;
      const f32x4 s4 = (red[0][hb][m][lane] + red[1][hb][m][lane]) + (red[2][hb][m][lane] + red[3][hb][m][lane]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = hp + 16 * hb + 4 * g + r;
        if (h < a.H) part[((size_t)blockIdx.y * a.H + h) * a.dx + col0 + 16 * m + c] = s4[r];
      }
    }
  }
}

// dtheta[h][col] = sum over the chunks, in chunk order
__global__ void __launch_bounds__(256) lr_gate_bwd_reduce_kernel(GateBwdArgs a, const float* part,
                                                                 int nchunk) {
  const int64_t n = (int64_t)a.H * a.dx;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float s = 0.f;
#pragma unroll 8
    for (int k = 0; k < nchunk; ++k) s += part[k * n + i];
    a.dtheta[i] = s;
  }
}

// da of 16 tokens for the dx kernel: lane (c, g) holds token f0 + c of heads
// hp + 4j + g, j < KS (eta and deta).
template <int KS>
struct DaCol {
  float e[KS], de[KS];
};

// dx[f][:] = sum_h da[f][h] theta[h][:] on the fp32 matrix unit (16x16x4
// f32 MFMA, exact fp32 products): per wave a tile of 16 NE columns, heads in
// passes of 4 KS.  Product e covers tile columns 16 e .. 16 e + 15 (its
// 16-row index m is the column 16 e + m): A = theta^T (lane (c, g): head
// 4j + g, column 16 e + c, loaded once per pass), B = da^T (lane (c, g):
// token c, head 4j + g); the result lane (c, g) holds token c, columns
// 16 e + 4g .. 16 e + 4g + 3.  The 16 x 16 NE result tile goes through the
// wave's own LDS tile (rows padded by four words: conflict-free both ways)
// and out row by row: 4 NE lanes per row, 16 NE * 4 contiguous bytes.
// Workgroup = four waves on one column tile, taking interleaved 16-token
// groups (G each, G a multiple of 3); the da loads run two groups ahead in
// three rotating register sets; dx goes out through a buffer descriptor over
// the group's rows, so rows past the chunk are dropped without a branch.
// One launch per pass of 4 KS heads from hp on; the passes after the first
// (ADD, H > 4 KS) add to what the earlier ones stored.  NT: nontemporal
// stores, for outputs too large to stay in the caches.
template <int NE, int KS, bool ADD, bool NT>
__global__ void __launch_bounds__(256) lr_gate_bwd_dx_kernel(GateBwdArgs a, int G, int hp) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int PITCH = 16 * NE + 4;  // words per LDS row
  constexpr int LPR = 4 * NE;         // lanes per output row
  __shared__ f32x4 tile[4][16 * PITCH / 4];
  // wave index as a scalar: the buffer descriptors built from it stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int ntok = a.B * a.T;
  const int col0 = blockIdx.x * 16 * NE;
  const int f_begin = blockIdx.y * 64 * G;
  const int f_end = min(ntok, f_begin + 64 * G);
  const float inv_base = a.eta_base != 0.f ? 1.f / a.eta_base : 0.f;
  // output lane mapping: row lane / LPR (+ 64 / LPR per store), columns 4 (lane % LPR) ..
  const int orow = lane / LPR, ocol = 4 * (lane % LPR);
  const uint32_t ooff = (uint32_t)((orow * a.dx + col0 + ocol) * 4);
  f32x4* const wt = tile[wave];
  const uint32_t ebytes = (uint32_t)(ntok * a.H) * 4u;  // B * T * H < 2^30
  const __amdgpu_buffer_rsrc_t re = make_rsrc(a.eta, ebytes), rd = make_rsrc(a.deta, ebytes);

  {
    float th[KS][NE];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int h = hp + 4 * j + g;
      const float* p = a.theta + (size_t)min(h, a.H - 1) * a.dx + col0 + c;
#pragma unroll
      for (int e = 0; e < NE; ++e) th[j][e] = h < a.H ? p[16 * e] : 0.f;
    }

    // group i of this wave starts at token f_begin + 16 (wave + 4 i)
    auto load = [&](int i, DaCol<KS>& st) {
      const int f = min(f_begin + 16 * (wave + 4 * i) + c, ntok - 1);
      const int bi = f / a.T, t = f - bi * a.T;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int h = min(hp + 4 * j + g, a.H - 1);
        const uint32_t off = (uint32_t)((bi * a.H + h) * a.T + t) * 4u;
        st.e[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, off, 0, 0));
        st.de[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, off, 0, 0));
      }
    };
    auto compute = [&](int i, const DaCol<KS>& st) {
      const int f0 = f_begin + 16 * (wave + 4 * i);
      const bool tok = f0 + c < f_end;
      float bj[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const float e = st.e[j];
        const float v = st.de[j] * e * (1.f - e * inv_base);
        bj[j] = (tok && hp + 4 * j + g < a.H) ? v : 0.f;
      }
      f32x4 acc[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        acc[e] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KS; ++j) acc[e] = mfma_f32(th[j][e], bj[j], acc[e]);
      }
      const int rows = __builtin_amdgcn_readfirstlane(min(max(f_end - f0, 0), 16));
      const int frow = __builtin_amdgcn_readfirstlane(min(f0, ntok));
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.dxo + (int64_t)frow * a.dx, (uint32_t)(rows * a.dx * 4));
#pragma unroll
      for (int e = 0; e < NE; ++e) wt[(c * PITCH + 16 * e + 4 * g) / 4] = acc[e];
#pragma unroll
      for (int k = 0; k < NE; ++k) {  // rows orow + (64 / LPR) k
        const int r = orow + (64 / LPR) * k;
        const uint32_t off = ooff + (uint32_t)((64 / LPR) * k * a.dx * 4);
        f32x4 o = wt[(r * PITCH + ocol) / 4];
        if constexpr (ADD) o += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ro, off, 0, NT ? 2 : 0);
      }
    };
    // scheduling fences keep each set's loads where they stand, so a set is
    // never reloaded while its previous contents are still being read
    DaCol<KS> sa, sb, sc;
    load(0, sa);
    load(1, sb);
    for (int i = 0; i < G; i += 3) {
      __builtin_amdgcn_sched_barrier(0);
      load(i + 2, sc);
      __builtin_amdgcn_sched_barrier(0);
      compute(i, sa);
      __builtin_amdgcn_sched_barrier(0);
      load(i + 3, sa);
      __builtin_amdgcn_sched_barrier(0);
      compute(i + 1, sb);
      __builtin_amdgcn_sched_barrier(0);
      load(i + 4, sb);
      __builtin_amdgcn_sched_barrier(0);
      compute(i + 2, sc);
    }
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

}  // namespace

// Workgroups of `kernel` (256 threads) resident on the current device at
// once, from the runtime's occupancy query (host-side, asked on every call:
// the library keeps nothing between calls).
// A failed query falls back to one workgroup per CU of 256 CUs (a sizing
// choice only); the launches report their own status (ttt::launch), so an
// error of the query is neither cleared nor blamed on them.
int resident_workgroups(const void* kernel) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  return std::max(per_cu, 1) * (cus > 0 ? cus : 256);
}

hipError_t launch_lr_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  const int ntok = a.B * a.T;  // B * T * dx < 2^31 (checked by the ABI)
  const int64_t nth = (int64_t)a.H * a.dx;
  if (ntok == 0 || a.H == 0) {  // dtheta = 0 (no tokens), dx = 0 (no heads)
    hipError_t e = hipSuccess;
    if (nth > 0) e = launch(fill_zero_kernel, dim3(256), dim3(256), s, a.dtheta, nth);
    if (e == hipSuccess && ntok > 0)
      e = launch(fill_zero_kernel, dim3(1024), dim3(256), s, a.dxo, (int64_t)ntok * a.dx);
    return e;
  }
  const bool small_h = a.H <= 16;
  // Token chunks are sized so that the whole grid is resident at once (no
  // second partial round of workgroups): per column tile, at most
  // resident / tiles chunks, each a multiple of 3 blocks per wave.
  auto per_wave = [&](const void* k, int tiles, int64_t units) {
    const int64_t slots = std::max<int64_t>(1, resident_workgroups(k) / tiles);
    const int64_t u = (units + 4 * slots - 1) / (4 * slots);  // 16-token units per wave
    return (int)(3 * ((u + 2) / 3));
  };

  // dtheta: chunks of 64 J tokens (J blocks of 16 per wave) whose partial
  // sums go to the start of dx's memory (nchunk * H <= B * T rows of dx) and
  // are summed in chunk order before dx itself is written; a single chunk
  // writes dtheta directly
  const int nm = a.dx % 128 == 0 ? 8 : a.dx % 64 == 0 ? 4 : 2;
  const int ncol1 = a.dx / (16 * nm);
  const bool vec = a.T % 4 == 0;
  const void* kd;
  if (nm == 8)
    kd = small_h ? (vec ? (const void*)lr_gate_bwd_dtheta_kernel<8, 1, true> : (const void*)lr_gate_bwd_dtheta_kernel<8, 1, false>)
                 : (vec ? (const void*)lr_gate_bwd_dtheta_kernel<8, 2, true> : (const void*)lr_gate_bwd_dtheta_kernel<8, 2, false>);
  else if (nm == 4)
    kd = small_h ? (vec ? (const void*)lr_gate_bwd_dtheta_kernel<4, 1, true> : (const void*)lr_gate_bwd_dtheta_kernel<4, 1, false>)
                 : (vec ? (const void*)lr_gate_bwd_dtheta_kernel<4, 2, true> : (const void*)lr_gate_bwd_dtheta_kernel<4, 2, false>);
  else
    kd = small_h ? (vec ? (const void*)lr_gate_bwd_dtheta_kernel<2, 1, true> : (const void*)lr_gate_bwd_dtheta_kernel<2, 1, false>)
                 : (vec ? (const void*)lr_gate_bwd_dtheta_kernel<2, 2, true> : (const void*)lr_gate_bwd_dtheta_kernel<2, 2, false>);
  int J = per_wave(kd, ncol1, (ntok + 15) / 16);
  auto chunks = [&](int j) { return (ntok + 64 * j - 1) / (64 * j); };
  while (chunks(J) > 1 && (int64_t)chunks(J) * a.H > ntok) J += 3;
  const int nchunk = chunks(J);
  float* part = nchunk == 1 ? a.dtheta : a.dxo;
  const dim3 g1((unsigned)ncol1, (unsigned)nchunk);
  for (int hp = 0; hp < a.H; hp += small_h ? 16 : 32) {
    void* args[] = {(void*)&a, (void*)&part, (void*)&J, (void*)&hp};
    const hipError_t e = hipLaunchKernel(kd, g1, dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (nchunk > 1) {
    const int64_t nb = (nth + 255) / 256;
    const hipError_t e = launch(lr_gate_bwd_reduce_kernel, dim3((unsigned)(nb < 1024 ? nb : 1024)),
                                dim3(256), s, a, (const float*)a.dxo, nchunk);
    if (e != hipSuccess) return e;
  }

  // dx: chunks of 64 G tokens per workgroup (G groups of 16 per wave), tiles
  // of 128 columns (32 when dx is not a multiple of 128); outputs beyond
  // 128 MB are stored nontemporally
  const int ne = a.dx % 128 == 0 ? 8 : 2;
  const int ncol2 = a.dx / (16 * ne);
  const bool nt = (int64_t)ntok * a.dx * 4 >= ((int64_t)128 << 20);
#define TTT_DXK(NE, KS, ADD) \
  (nt ? (const void*)lr_gate_bwd_dx_kernel<NE, KS, ADD, true> : (const void*)lr_gate_bwd_dx_kernel<NE, KS, ADD, false>)
  const void* kx0 = ne == 8 ? (small_h ? TTT_DXK(8, 4, false) : TTT_DXK(8, 8, false))
                            : (small_h ? TTT_DXK(2, 4, false) : TTT_DXK(2, 8, false));
  const void* kx1 = ne == 8 ? TTT_DXK(8, 8, true) : TTT_DXK(2, 8, true);
#undef TTT_DXK
  int G = per_wave(kx0, ncol2, (ntok + 15) / 16);
  const dim3 g2((unsigned)ncol2, (unsigned)((ntok + 64 * G - 1) / (64 * G)));
  for (int hp = 0; hp < a.H; hp += small_h ? 16 : 32) {
    void* args[] = {(void*)&a, (void*)&G, (void*)&hp};
    const hipError_t e = hipLaunchKernel(hp == 0 ? kx0 : kx1, g2, dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
