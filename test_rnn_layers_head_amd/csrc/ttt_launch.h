// Internal launch interface between the C ABI (ttt_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace ttt {

// Enqueue `kernel` on `s` and return the status of this launch alone: an
// error left pending on the calling thread by earlier HIP calls is neither
// reported nor cleared.
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> v(std::forward<A>(args)...);
  return std::apply(
      [&](auto&... x) {
        void* argv[] = {(void*)&x...};
        return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, s);
      },
      v);
}

struct LinearArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* w0;
  float* z;
  float* w_out;
  int w0_per_batch;
  int units;  // B * H
  int H;
  int T;
  int b;
  // optional: the state at the start of every mini-batch,
  // [units][ceil(T / b)][64][64] (bf16 inputs)
  float* w_ckpt = nullptr;
  // Passes of the chunked scan (bf16, b = 16; defaults: the plain scan).
  // z == nullptr: no outputs (Q is not read either).
  int v_zero = 0;   // V read as zeros
  int w0_mode = 0;  // start state: W0_ARG (w0, w0_per_batch), W0_IDENTITY, W0_ZERO, or W0_IN_Z
                    // (unit u's own last 64 tokens of z, layout of chunk_state_in_z)
  int wout_stride = 4096;  // floats between the final states of consecutive units
  int wout_every = 1;      // only units u with u % wout_every == wout_every - 1 write their
                           // final state, to w_out + (u / wout_every) * wout_stride
  int ring_depth = 0;      // bf16, b = 16: 0 = the default LDS ring depth, 1 = one tile in flight
  // With w_ckpt: tokens per tile, 16 or b < 16 (b | 16), each b-token
  // mini-batch then alone in a tile whose other rows read as zero tokens
  // (eta = 0: no contribution) and drop their outputs.
  int bt = 16;
};

enum { W0_ARG = 0, W0_IDENTITY = 1, W0_ZERO = 2, W0_IN_Z = 3 };

// Where the chunked scan keeps the start state of a sequence chunk: element
// (row, col) of the 64 x 64 state of unit u, for a pass with `rows` rows of
// the state per workgroup, lies in u's own z rows [T - 64, T), at the z
// position that the workgroup owning that row writes itself (and only after
// it has read the state): token T - 64 + i * (64 / rows) + col / rows,
// component row0 + col % rows, with row0 = row - row % rows, i = row % rows.
__host__ __device__ inline int64_t chunk_state_in_z(int T, int rows, int row, int col) {
  const int row0 = row - row % rows, i = row % rows;
  return (int64_t)(T - 64 + i * (64 / rows) + col / rows) * 64 + row0 + col % rows;
}

// TTT-Linear with the LayerNorm + residual inner model: gamma, beta [H][64].
struct LinearLnArgs {
  LinearArgs s;
  const float* gamma;
  const float* beta;
  float eps;
};

// TTT-Linear with the LayerNorm + residual inner model, primal form (any b,
// fp32 or bf16 q/k/v): the forward (s.w_ckpt non-NULL: also the state before
// every mini-batch, [units][ceil(T/b)][64][64]) and the backward.
hipError_t launch_linear_ln_primal(const LinearLnArgs& a, bool f32in, hipStream_t s);
struct LinearLnBwdArgs {
  const void* q;          // [units][T][64]
  const void* k;
  const void* v;
  const float* eta;       // [units][T]
  const float* w_ckpt;    // [units][ceil(T/b)][64][64]
  const float* gamma;     // [H][64]
  const float* beta;
  float eps;
  const float* dz;        // [units][T][64]
  const float* dw_T;      // [units][64][64] or NULL
  float* dq;              // [units][T][64]
  float* dk;
  float* dv;
  float* deta;            // [units][T]
  float* dw0;             // [units][64][64]
  float* dgamma;          // [units][64]
  float* dbeta;
  int units;
  int H;
  int T;
  int b;
};
hipError_t launch_linear_ln_primal_bwd(const LinearLnBwdArgs& a, bool f32in, hipStream_t s);
// bf16 q/k/v with b = 16: the dual-form backward (one wave per unit);
// otherwise the primal form.
hipError_t launch_linear_ln_bwd(const LinearLnBwdArgs& a, bool f32in, hipStream_t s);

struct MlpArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* w1_0;
  const float* w2_0;
  float* z;
  float* w1_out;
  float* w2_out;
  int w0_per_batch;
  int units;
  int H;
  int T;
  int b;
  // optional: the state at the start of every mini-batch,
  // [units][ceil(T / b)][256][64] and [units][ceil(T / b)][64][256]
  float* w1_ckpt = nullptr;
  float* w2_ckpt = nullptr;
};

// TTT-MLP with the LayerNorm + residual wrapper, f(x) = x + LN(W2 GELU(W1 x))
// (gamma, beta [H][64]).  launch_mlp_ln runs the dual-form scan for bf16
// q/k/v with b | 16 and the primal form (any b, fp32 or bf16) otherwise.
struct MlpLnArgs {
  MlpArgs s;
  const float* gamma;
  const float* beta;
  float eps;
};
hipError_t launch_mlp_ln(const MlpLnArgs& a, bool f32in, hipStream_t s);
hipError_t launch_mlp_ln_primal(const MlpLnArgs& a, bool f32in, hipStream_t s);

// Backward of the TTT-MLP scan (hidden = 256, any b, fp32 or bf16 q/k/v).
struct MlpBwdArgs {
  const void* q;          // [units][T][64]
  const void* k;
  const void* v;
  const float* eta;       // [units][T]
  const float* w1_ckpt;   // [units][ceil(T/b)][256][64]: W1 at every mini-batch start
  const float* w2_ckpt;   // [units][ceil(T/b)][64][256]
  const float* dz;        // [units][T][64]
  const float* dw1_T;     // [units][256][64] or NULL
  const float* dw2_T;     // [units][64][256] or NULL
  float* dq;              // [units][T][64]
  float* dk;
  float* dv;
  float* deta;            // [units][T]
  float* dw1_0;           // [units][256][64]
  float* dw2_0;           // [units][64][256]
  int units;
  int T;
  int b;
};
// bf16 q/k/v with b | 16: the dual-form backward (one workgroup of 8 waves
// per unit; for b < 16 one mini-batch per 16-token tile, its other rows
// zero tokens); otherwise the primal form token by token.
hipError_t launch_mlp_bwd(const MlpBwdArgs& a, bool f32in, hipStream_t s);
hipError_t launch_mlp_bwd_primal(const MlpBwdArgs& a, bool f32in, hipStream_t s);

// Backward of the TTT-Linear scan (b = 16, bf16 q/k/v).
struct LinearBwdArgs {
  const void* q;         // [units][T][64] bf16
  const void* k;
  const void* v;
  const float* eta;      // [units][T]
  const float* w_ckpt;   // [units][ceil(T/bt)][64][64]: W at every tile start (tpm = 1)
  const float* dz;       // [units][T][64]
  const float* dw_T;     // [units][64][64] or NULL
  float* dq;             // [units][T][64]
  float* dk;
  float* dv;
  float* deta;           // [units][T]
  float* dw0;            // [units][64][64], or NULL: not written
  int units;
  int H;
  int T;
  // Passes of the chunked backward (defaults: the plain backward).
  int dw_stride = 4096;   // floats between the dw_T of consecutive units
  int dw0_stride = 4096;  // floats between the dw0 of consecutive units
  int tok_out = 1;        // 0: dq, dk, dv, deta are not written
  // Tokens per tile: 16, or b < 16 (b | 16) with each b-token mini-batch
  // alone in a tile whose other rows read as zero tokens (eta = 0: no
  // contribution to the state) and whose outputs there are dropped.
  int bt = 16;
  // Mini-batches of 16 tpm tokens (tpm > 1): the gradient point is held
  // across tpm tiles; w_ckpt then holds one state per mini-batch,
  // [units][ceil(T / (16 tpm))][64][64].
  int tpm = 1;
};
hipError_t launch_linear_bwd(const LinearBwdArgs& a, hipStream_t s);

// TTT-Linear training support in the primal form (any b, fp32 or bf16 q/k/v):
// the checkpointing forward (a.w_ckpt [units][ceil(T/b)][64][64]) and the
// backward from those checkpoints.
struct LinearPrimalBwdArgs {
  const void* q;          // [units][T][64]
  const void* k;
  const void* v;
  const float* eta;       // [units][T]
  const float* w_ckpt;    // [units][ceil(T/b)][64][64]
  const float* dz;        // [units][T][64]
  const float* dw_T;      // [units][64][64] or NULL
  float* dq;              // [units][T][64]
  float* dk;
  float* dv;
  float* deta;            // [units][T]
  float* dw0;             // [units][64][64]
  int units;
  int T;
  int b;
};
hipError_t launch_linear_primal_ckpt(const LinearArgs& a, hipStream_t s);  // fp32 q/k/v
hipError_t launch_linear_primal_bwd(const LinearPrimalBwdArgs& a, hipStream_t s);  // fp32 q/k/v
// The backward in P sequence chunks of T / P tokens (a multiple of 16, at
// least 192): the chunks' forward maps, their backward from a zero end
// adjoint, a serial combine over the chunks, then every chunk from its end
// adjoint.  The first passes keep their 64 x 64 results in dq's memory of
// their chunk (tokens 0..191) before the last pass writes dq.  rows: rows of
// the state per workgroup of the forward-map pass.
hipError_t launch_linear_bwd_chunked(const LinearBwdArgs& a, int P, int rows, hipStream_t s);

// Learning-rate gate: eta[b][h][t] = eta_base * sigmoid(theta[h] . x[b][t]).
struct GateArgs {
  const void* x;       // [B][T][dx] bf16
  const float* theta;  // [H][dx]
  float* eta;          // [B][H][T]
  float eta_base;
  int B;
  int T;
  int H;
  int dx;  // multiple of 32
};
// tokens_per_workgroup: 32, 64 or 0 (chosen from the token count)
hipError_t launch_lr_gate(const GateArgs& a, int tokens_per_workgroup, hipStream_t s);

// Backward of the gate: dtheta [H][dx] and dxo [B][T][dx] from deta and the
// forward's eta [B][H][T].
struct GateBwdArgs {
  const void* x;       // [B][T][dx] bf16
  const float* theta;  // [H][dx]
  const float* eta;    // [B][H][T]
  const float* deta;   // [B][H][T]
  float* dtheta;       // [H][dx]
  float* dxo;          // [B][T][dx]
  float eta_base;
  int B;
  int T;
  int H;
  int dx;  // multiple of 32
};
hipError_t launch_lr_gate_bwd(const GateBwdArgs& a, hipStream_t s);

// One decode step for every (batch, head) unit.
struct StepArgs {
  const void* q;  // [B][H][d]
  const void* k;
  const void* v;
  const float* eta;  // [B][H]
  float* w;          // [B][H][...] state, in/out
  float* w_gp;       // gradient point, in/out (NULL: b == 1)
  float* w2;         // TTT-MLP second layer, in/out
  float* w2_gp;
  const int32_t* pos;  // [B]
  float* z;            // [B][H][d]
  int units;
  int H;
  int b;
};

// rows: rows of W per workgroup (64, 32 or 16).
hipError_t launch_linear(const LinearArgs& a, bool f32in, int rows, hipStream_t s);
// The chunked (sequence-parallel) TTT-Linear scan for bf16 inputs and b = 16:
// each unit's sequence in P chunks of T / P tokens (T / P a multiple of 16,
// at least 192), rows of the state per workgroup as in launch_linear.  z's
// memory holds the intermediate states, so its prior contents do not matter.
hipError_t launch_linear_chunked(const LinearArgs& a, int P, int rows, hipStream_t s);
hipError_t launch_linear_bf16(const LinearArgs& a, int rows, hipStream_t s);
hipError_t launch_linear_ln(const LinearLnArgs& a, hipStream_t s);
hipError_t launch_mlp(const MlpArgs& a, bool f32in, hipStream_t s);
// The TTT-MLP scan token by token in fp32 (any b >= 1, fp32 or bf16 q/k/v).
hipError_t launch_mlp_primal(const MlpArgs& a, bool f32in, hipStream_t s);
hipError_t launch_linear_step(const StepArgs& a, bool f32in, hipStream_t s);
hipError_t launch_linear_ln_step(const StepArgs& a, const float* gamma, const float* beta,
                                 float eps, bool f32in, hipStream_t s);
// TTT-MLP, hidden = 256: w, w_gp = W1 [B][H][256][64]; w2, w2_gp = W2 [B][H][64][256].
hipError_t launch_mlp_step(const StepArgs& a, bool f32in, hipStream_t s);
hipError_t launch_copy_state(const float* src, int per_unit, int units, int H, int n,
                             float* dst, hipStream_t s);

}  // namespace ttt
