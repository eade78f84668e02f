/*
 * ttt.h — C ABI of the MI355X (gfx950) TTT forward-scan library, libttt.so.
 *
 * The library computes the forward pass of a TTT layer's inner loop:
 * mini-batch test-time training of a fast-weight state W, evaluated in the
 * dual form.  Sources ("论文速览 | TTT", the equinox-blog close reading of
 * "Learning to (Learn at Test Time): RNNs with Expressive Hidden States"):
 *   §3.1  each token updates the state, the output is read from the UPDATED
 *         state: W_t = W_{t-1} - eta_t G_t, z_t = f(q_t; W_t);
 *   §3.3  loss l(W; t) = || f(k_t; W) - v_t ||^2 (sum over components, so the
 *         gradient carries a factor 2); k, v, q are the already-projected
 *         training, label and test views;
 *   §3.5  mini-batch GD: tokens [j*b, j*b + b) all take their gradient at the
 *         state before that mini-batch; a final partial mini-batch is shorter;
 *   §3.6  dual form for f(x) = W x;  §3.7 dual form for an MLP inner model;
 *   §4.4  TTT-Linear f(x) = W x and TTT-MLP f(x) = W2 GELU(W1 x) (GELU =
 *         x Phi(x), hidden width 4d);
 *   §4.6  a per-token inner learning rate eta_t scales token t's gradient.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers:  every tensor pointer is a DEVICE pointer on the current HIP
 *            device, owned by the caller; the library allocates nothing,
 *            frees nothing and keeps no state between calls.  Tensors are
 *            dense, row-major, and 16-byte aligned.
 * Streams:   `stream` is a hipStream_t (NULL = the null stream).  Work is
 *            enqueued asynchronously; the call returns after the launch.
 * Errors:    arguments are checked on the host before anything is enqueued;
 *            a non-TTT_OK status means nothing was launched.  A failed launch
 *            returns TTT_ERR_HIP.  Faults inside a kernel surface at the
 *            caller's next synchronisation.  ttt_last_error() gives a
 *            human-readable message for the calling thread's last failure.
 * Layouts:   q, k, v   [B][H][T][d]   in qkv_dtype (fp32 or bf16)
 *            eta       [B][H][T]      fp32
 *            z         [B][H][T][d]   fp32 (output)
 *            W[i][j]   i = output component, j = input component: f(x) = W x.
 *            Initial states are shared by the batch ([H][...], w0_per_batch =
 *            0, the learnt initial state of §4.5) or given per unit
 *            ([B][H][...], w0_per_batch = 1, e.g. to resume a sequence from a
 *            previous call's final state).  Final states are always per unit.
 * Aliasing:  z must not overlap any input.  A final-state output may alias
 *            its initial-state input only when w0_per_batch = 1 and the two
 *            pointers are equal (in-place resume); any other overlap is
 *            TTT_ERR_ALIAS.
 * Support:   d = 64; any 0 <= T < 2^24, B, H >= 0 with B*H*T*d < 2^31.
 *            TTT-Linear: fp32 or bf16 q/k/v; mini-batch b with b | 16 or
 *            16 | b (1, 2, 4, 8, 16, 32, 48, 64, ...).
 *            TTT-MLP: hidden = 256, fp32 or bf16 q/k/v, b | 16 or 16 | b.
 *            TTT-Linear with LayerNorm: fp32 or bf16 q/k/v, b | 16 or 16 | b.
 *            Anything else is TTT_ERR_UNSUPPORTED.
 *            Empty work (B*H == 0) returns TTT_OK without launching; T == 0
 *            copies the initial states to the final-state outputs.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 1

typedef enum {
  TTT_OK = 0,
  TTT_ERR_NULL = 1,        /* a required pointer is NULL                    */
  TTT_ERR_SHAPE = 2,       /* negative size or size product overflow        */
  TTT_ERR_DTYPE = 3,       /* qkv_dtype is not a ttt_dtype_t value          */
  TTT_ERR_UNSUPPORTED = 4, /* d, hidden or b outside the supported set      */
  TTT_ERR_ALIAS = 5,       /* an output overlaps an input (see Aliasing)    */
  TTT_ERR_HIP = 6,         /* the HIP runtime reported an error             */
  TTT_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned       */
  TTT_ERR_VALUE = 8,       /* a scalar argument is out of range             */
  /* not a status: makes every int32 a valid value of the type, so that a
     caller's out-of-range value reaches ttt_status_str well defined */
  TTT_STATUS_MAX_ENUM = 0x7fffffff
} ttt_status_t;

/* TTT_DTYPE_MAX_ENUM is not a dtype; it widens the type to every int32, so an
   unknown value from a caller is rejected as TTT_ERR_DTYPE, well defined. */
typedef enum { TTT_F32 = 0, TTT_BF16 = 1, TTT_DTYPE_MAX_ENUM = 0x7fffffff } ttt_dtype_t;

/*
 * TTT-Linear forward scan, f(x) = W x (§3.6 dual form, §4.4).
 *
 *   q, k, v : [B][H][T][d] qkv_dtype       eta : [B][H][T] fp32
 *   w0      : [H][d][d] fp32 (w0_per_batch = 0) or [B][H][d][d] (= 1)
 *   z       : out [B][H][T][d] fp32, z_t = W_t q_t with W_t after token t
 *   w_out   : out [B][H][d][d] fp32, the state after the last token
 *
 * Per (batch, head) the state evolves as
 *   W_t = W_{t-1} - 2 eta_t (W_{j*b} k_t - v_t) k_t^T,   j = t / b,
 * with W_{j*b} the state before mini-batch j, which is what the dual form
 * W_b = W0 - 2 (W0 K - V) diag(eta) K^T, Z = W0 Q - 2 (W0 K - V) diag(eta)
 * triu(K^T Q) computes per mini-batch.
 *
 * Sequence chunks.  Each mini-batch maps the state affinely,
 * W_b = W0 (I - 2 K diag(eta) K^T) + 2 V diag(eta) K^T, so a run of
 * mini-batches is one affine map W -> W M + C.  With few (batch, head) units
 * and long sequences (bf16 q/k/v, b = 16, B*H <= 32 and T >= 8192; then
 * P = 8 or 16 with B*H*P <= 256 and T / P >= 1024, a multiple of 16) the
 * scan cuts each sequence into P chunks: it forms every chunk's M (from the
 * identity with v = 0) and C (from zero), chains the maps to get each
 * chunk's start state, then runs all chunks at once with outputs.  z's
 * memory holds the intermediate maps and states before the outputs
 * overwrite them.  Results agree with the single-pass scan to rounding (not
 * bit for bit); ttt_linear_fwd_chunked (ttt_tuning.h) sets P explicitly.
 */
ttt_status_t ttt_linear_fwd(const void* q, const void* k, const void* v,
                            const float* eta, const float* w0,
                            int32_t w0_per_batch, int32_t B, int32_t H,
                            int32_t T, int32_t d, int32_t b,
                            ttt_dtype_t qkv_dtype, float* z, float* w_out,
                            void* stream);

/*
 * TTT-Linear with the LayerNorm + residual inner model (§4.4):
 *   f(x) = x + LN(W x),  LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps)
 *          + beta,
 * mean and population variance over the d components of one token.  The
 * inner loss ||f(k_t) - v_t||^2 (§3.3) is differentiated through the
 * LayerNorm; mini-batches as for ttt_linear_fwd (§3.5, §3.6), outputs
 * z_t = q_t + LN(W_t q_t) from the updated state (§3.1).
 *
 *   q, k, v        : [B][H][T][d] bf16          eta : [B][H][T] fp32
 *   w0             : [H][d][d] or [B][H][d][d] fp32 (as ttt_linear_fwd)
 *   ln_gamma, ln_beta : [H][d] fp32, the LayerNorm scale and shift of each
 *                    head (the page names the wrapper, not its parameters:
 *                    per head, shared by the batch)
 *   eps            : LayerNorm epsilon, finite and > 0, else TTT_ERR_VALUE
 *   z              : out [B][H][T][d] fp32;  w_out : out [B][H][d][d] fp32
 *
 * Support: d = 64, fp32 or bf16 q/k/v, b | 16 or 16 | b.  bf16 with 16 | b
 * runs the dual form per 16-token tile (one workgroup per (batch, head)).
 * Below 16 tokens a mini-batch's gradients depend non-linearly, through the
 * LayerNorm, on the updates of earlier mini-batches in the same tile, which
 * a one-tile dual form cannot evaluate; so bf16 with b < 16 gives each
 * mini-batch a 16-token tile of its own, its other rows zero tokens (eta = 0:
 * they change neither the state nor the other tokens' outputs, and their own
 * outputs are dropped), at 16 / b times the cost per token.  fp32 inputs run
 * the primal form token by token in fp32 arithmetic (256 threads per
 * (batch, head)).
 */
ttt_status_t ttt_linear_ln_fwd(const void* q, const void* k, const void* v,
                               const float* eta, const float* w0,
                               int32_t w0_per_batch, const float* ln_gamma,
                               const float* ln_beta, float eps, int32_t B,
                               int32_t H, int32_t T, int32_t d, int32_t b,
                               ttt_dtype_t qkv_dtype, float* z, float* w_out,
                               void* stream);

/*
 * TTT-MLP with the same LayerNorm + residual wrapper (§4.4 applies it to
 * both inner models):
 *   f(x) = x + LN(W2 GELU(W1 x)),  LN as for ttt_linear_ln_fwd.
 * The inner loss ||f(k_t) - v_t||^2 is differentiated through the LayerNorm
 * and then through both layers, every gradient of a mini-batch at the state
 * before it (§3.5, §3.7); outputs z_t = q_t + LN(W2_t GELU(W1_t q_t)) from
 * the updated state (§3.1).  Arguments as for ttt_mlp_fwd, plus ln_gamma,
 * ln_beta ([H][d] fp32, per head) and eps (finite and > 0, else
 * TTT_ERR_VALUE).
 *
 * Support: d = 64, hidden = 256, fp32 or bf16 q/k/v, b | 16 or 16 | b.
 * bf16 q/k/v with b | 16 or 16 | b runs the dual-form scan of ttt_mlp_fwd
 * (same work split and precision, and for b > 16 the same use of w2_out as
 * the held state during the call), the LayerNorm's per-token sums over the
 * 64 components crossing the reducing waves through LDS; fp32 inputs run the
 * primal form token by token in fp32 arithmetic (1024 threads per (batch,
 * head)).
 */
ttt_status_t ttt_mlp_ln_fwd(const void* q, const void* k, const void* v,
                            const float* eta, const float* w1_0,
                            const float* w2_0, int32_t w0_per_batch,
                            const float* ln_gamma, const float* ln_beta,
                            float eps, int32_t B, int32_t H, int32_t T,
                            int32_t d, int32_t hidden, int32_t b,
                            ttt_dtype_t qkv_dtype, float* z, float* w1_out,
                            float* w2_out, void* stream);

/*
 * Training support (§6.12: the outer loop differentiates through the inner
 * one; the forward keeps the state at the start of every mini-batch, the
 * kappa = T / b checkpoints, and the backward walks the mini-batches in
 * reverse).  Support: d = 64, bf16 or fp32 q/k/v, b dividing 16 or a
 * multiple of 16; else TTT_ERR_UNSUPPORTED.  bf16 with b | 16 runs the
 * dual-form kernels of b = 16; for b < 16 each mini-batch takes a 16-token
 * tile of its own whose other rows are zero tokens (eta = 0: they change
 * neither the state nor the other tokens' outputs, and their own outputs are
 * dropped), so the cost per token is 16 / b times that of b = 16.  With
 * b > 16 the checkpointing forwards are the dual-form scans; the TTT-Linear
 * backward is the b = 16 kernel with the gradient point held across b / 16
 * tiles (its adjoint kept apart and added at each mini-batch start, and the
 * running state of each tile rebuilt in reverse from the checkpoints, the
 * last mini-batch's end state first), the LayerNorm and TTT-MLP backward
 * kernels the primal form; fp32 q/k/v run the primal-form kernels (one token
 * at a time, fp32 arithmetic, no sequence chunks).  Sequence chunks: b = 16
 * only.
 *
 * ttt_linear_fwd_ckpt: ttt_linear_fwd plus
 *   w_ckpt : out [B][H][ceil(T/b)][d][d] fp32, the state before each
 *            mini-batch (w_ckpt[..][0] = W0).
 * It takes sequence chunks as ttt_linear_fwd does; the last pass writes the
 * checkpoints.
 *
 * ttt_linear_bwd: the gradient of a loss L(Z, W_T) with respect to the
 * scan's inputs, given
 *   dz   : [B][H][T][d] fp32, dL/dZ
 *   dw_T : [B][H][d][d] fp32, dL/dW_T, or NULL for zero
 *   q, k, v, eta : the forward's inputs; w_ckpt : from ttt_linear_fwd_ckpt
 * and writing (fp32)
 *   dq, dk, dv : [B][H][T][d];  deta : [B][H][T]
 *   dw0 : [B][H][d][d], per unit (sum over the batch for a shared W0)
 * Outputs must not overlap each other or an input.  T = 0 writes
 * dw0 = dw_T (or zeros).  One workgroup per (batch, head); the adjoint state
 * stays on chip, nothing beyond the outputs is written.
 *
 * Sequence chunks (when ttt_linear_fwd would chunk the same sizes).  The
 * adjoint of the state also walks affinely, Wb = Wb' (I - 2 K diag(eta) K^T)
 * + (terms without Wb'), with the forward's symmetric factor: over a chunk
 * whose forward map is W -> W M + C the end adjoint E maps to E M^T + C',
 * C' being the chunk's backward from a zero end adjoint.  The backward then
 * forms every chunk's M and C', chains them from dw_T to get each chunk's
 * end adjoint (and dw0), and runs all chunks at once with outputs.  dq's
 * memory holds the intermediate 64 x 64 matrices (its first 192 tokens of
 * each chunk) before the outputs overwrite them.  Results agree with the
 * single pass to rounding; ttt_linear_bwd_chunked (ttt_tuning.h) sets the
 * chunk count explicitly.
 */
ttt_status_t ttt_linear_fwd_ckpt(const void* q, const void* k, const void* v,
                                 const float* eta, const float* w0,
                                 int32_t w0_per_batch, int32_t B, int32_t H,
                                 int32_t T, int32_t d, int32_t b,
                                 ttt_dtype_t qkv_dtype, float* z, float* w_out,
                                 float* w_ckpt, void* stream);
ttt_status_t ttt_linear_bwd(const void* q, const void* k, const void* v,
                            const float* eta, const float* w_ckpt, int32_t B,
                            int32_t H, int32_t T, int32_t d, int32_t b,
                            ttt_dtype_t qkv_dtype, const float* dz,
                            const float* dw_T, float* dq, float* dk, float* dv,
                            float* deta, float* dw0, void* stream);

/*
 * Decode steps (§6.11: generation runs the primal form, one token at a
 * time).  One call advances every (batch, head) unit by one token.  A unit
 * carries two states, both updated in place:
 *   w     the state after the previous token (W_{t-1});
 *   w_gp  the gradient point: the state at the start of the current
 *         mini-batch (§3.5).
 * With p = pos mod b (mathematical modulo) the token first sets w_gp = w when
 * p == 0, then takes its gradient at w_gp, updates w, and outputs
 * z = f(q; w) from the updated state (§3.1).  A scan over a multiple of b
 * tokens ends exactly at the next gradient point, so a sequence may be
 * prefilled with the scan and continued with steps; to continue a prefill of
 * another length, prefill the largest multiple of b and step the rest.
 *
 *   q, k, v : [B][H][d] qkv_dtype (this token)     eta : [B][H] fp32
 *   w, w_gp : [B][H][d][d] fp32, in/out; w_gp may be NULL when b == 1
 *   pos     : [B] int32 (device), the token's index in its sequence
 *   z       : out [B][H][d] fp32
 * Support: d = 64, any b >= 1, fp32 or bf16 q/k/v.  Outputs (z, w, w_gp)
 * must not overlap each other or an input.  Empty work (B*H == 0) returns
 * TTT_OK without launching.
 */
ttt_status_t ttt_linear_step(const void* q, const void* k, const void* v,
                             const float* eta, float* w, float* w_gp,
                             const int32_t* pos, int32_t B, int32_t H,
                             int32_t d, int32_t b, ttt_dtype_t qkv_dtype,
                             float* z, void* stream);

/* The same for the LayerNorm + residual inner model of ttt_linear_ln_fwd:
 * ln_gamma, ln_beta [H][d] fp32, eps finite and > 0 (else TTT_ERR_VALUE);
 * any b >= 1. */
ttt_status_t ttt_linear_ln_step(const void* q, const void* k, const void* v,
                                const float* eta, float* w, float* w_gp,
                                const int32_t* pos, const float* ln_gamma,
                                const float* ln_beta, float eps, int32_t B,
                                int32_t H, int32_t d, int32_t b,
                                ttt_dtype_t qkv_dtype, float* z, void* stream);

/* The same for TTT-MLP, f(x) = W2 GELU(W1 x) (as ttt_mlp_fwd):
 *   w1, w1_gp : [B][H][hidden][d] fp32, in/out
 *   w2, w2_gp : [B][H][d][hidden] fp32, in/out
 * Both gradient points may be NULL when b == 1 (pass both or neither).
 * Support: d = 64, hidden = 256, any b >= 1, fp32 or bf16 q/k/v. */
ttt_status_t ttt_mlp_step(const void* q, const void* k, const void* v,
                          const float* eta, float* w1, float* w2, float* w1_gp,
                          float* w2_gp, const int32_t* pos, int32_t B, int32_t H,
                          int32_t d, int32_t hidden, int32_t b,
                          ttt_dtype_t qkv_dtype, float* z, void* stream);

/*
 * TTT-MLP forward scan, f(x) = W2 GELU(W1 x) (§3.7 dual form, §4.4).
 *
 *   w1_0 : [H][hidden][d] fp32 (or [B][H][hidden][d] when w0_per_batch = 1)
 *   w2_0 : [H][d][hidden] fp32 (or [B][H][d][hidden])
 *   z    : out [B][H][T][d] fp32, z_t = W2_t GELU(W1_t q_t)
 *   w1_out, w2_out : out [B][H][hidden][d], [B][H][d][hidden] fp32
 *
 * Both layers take their gradient of sum_t eta_t ||f(k_t) - v_t||^2 at the
 * state before the mini-batch (§3.5).  GELU is x * Phi(x).
 *
 * Two kernels serve the call.  bf16 q/k/v with b | 16 or 16 | b: the dual
 * form per 16-token tile, state resident in registers, products on bf16
 * MFMA with fp32 operands split into bf16 hi + lo, erf from Abramowitz &
 * Stegun 7.1.26 (absolute error <= 1.5e-7); for b > 16 the state at the
 * mini-batch start (the gradient point) is kept in LDS and in w2_out, which
 * is therefore written during the call and holds the final W2 only at its
 * end (in-place resume, w2_out == w2_0 with w0_per_batch = 1, stays valid).
 * fp32 q/k/v: the primal form token by token in fp32 arithmetic (the
 * library's erff), one workgroup of 1024 threads per (batch, head) with the
 * state and the gradient point in registers; exact but about 10x slower per
 * token, meant for parity.
 */
ttt_status_t ttt_mlp_fwd(const void* q, const void* k, const void* v,
                         const float* eta, const float* w1_0,
                         const float* w2_0, int32_t w0_per_batch, int32_t B,
                         int32_t H, int32_t T, int32_t d, int32_t hidden,
                         int32_t b, ttt_dtype_t qkv_dtype, float* z,
                         float* w1_out, float* w2_out, void* stream);

/*
 * Training support for TTT-Linear with the LayerNorm + residual inner model
 * (§6.12 with §4.4).  Support: d = 64, fp32 or bf16 q/k/v, b | 16 or 16 | b.
 *
 * ttt_linear_ln_fwd_ckpt: ttt_linear_ln_fwd plus
 *   w_ckpt : out [B][H][ceil(T/b)][d][d] fp32, the state before each
 *            mini-batch of b tokens.
 * ttt_linear_ln_bwd: the gradient of a loss L(Z, W_T) given
 *   dz : [B][H][T][d] fp32;  dw_T : [B][H][d][d] fp32 or NULL (zero);
 *   the forward's q, k, v, eta, ln_gamma, ln_beta, eps; w_ckpt from
 *   ttt_linear_ln_fwd_ckpt with the same b;
 * writing (fp32) dq, dk, dv [B][H][T][d], deta [B][H][T], dw0 [B][H][d][d]
 * and the LayerNorm parameters' adjoints dgamma, dbeta [B][H][d], per unit
 * (sum over the batch for the shared per-head parameters).
 * ttt_linear_ln_fwd_ckpt runs the kernel ttt_linear_ln_fwd picks (the
 * dual-form scan for bf16 q/k/v, else the primal form), which
 * also stores each mini-batch's starting state; z and w_out equal
 * ttt_linear_ln_fwd's bit for bit.  The backward applies the adjoint of
 * every forward operation (the LayerNorm statistics, the LayerNorm VJP of
 * the inner gradient, the update, the output) in reverse order, mini-batch
 * by mini-batch from the checkpoints: for bf16 q/k/v with b | 16 in dual
 * form on the matrix unit (b < 16: one mini-batch per zero-padded tile, as
 * above), one workgroup of four waves per (batch, head)
 * (fp32 factors as bf16 hi + lo halves, ~2^-16 relative per product);
 * otherwise token by token in fp32 arithmetic, one workgroup of 256
 * threads per (batch, head).  Outputs must not overlap each other or an
 * input; T = 0 writes dw0 = dw_T (or zeros) and zero dgamma, dbeta.
 */
ttt_status_t ttt_linear_ln_fwd_ckpt(const void* q, const void* k, const void* v,
                                   const float* eta, const float* w0,
                                   int32_t w0_per_batch, const float* ln_gamma,
                                   const float* ln_beta, float eps, int32_t B,
                                   int32_t H, int32_t T, int32_t d, int32_t b,
                                   ttt_dtype_t qkv_dtype, float* z, float* w_out,
                                   float* w_ckpt, void* stream);
ttt_status_t ttt_linear_ln_bwd(const void* q, const void* k, const void* v,
                               const float* eta, const float* w_ckpt,
                               const float* ln_gamma, const float* ln_beta,
                               float eps, int32_t B, int32_t H, int32_t T,
                               int32_t d, int32_t b, ttt_dtype_t qkv_dtype,
                               const float* dz, const float* dw_T, float* dq,
                               float* dk, float* dv, float* deta, float* dw0,
                               float* dgamma, float* dbeta, void* stream);

/*
 * Training support for TTT-MLP (§6.12, as for TTT-Linear above; §3.7, §4.4).
 * Support: d = 64, hidden = 256, fp32 or bf16 q/k/v, b | 16 or 16 | b.
 *
 * ttt_mlp_fwd_ckpt: ttt_mlp_fwd plus
 *   w1_ckpt : out [B][H][ceil(T/b)][hidden][d] fp32, W1 before each
 *             mini-batch of b tokens (w1_ckpt[..][0] = W1_0);
 *   w2_ckpt : out [B][H][ceil(T/b)][d][hidden] fp32, the same for W2.
 * It runs the kernel ttt_mlp_fwd picks for the same arguments (the bf16
 * dual-form scan for bf16 q/k/v, else the primal form), which also stores
 * each mini-batch's starting state.
 *
 * ttt_mlp_bwd: the gradient of a loss L(Z, W1_T, W2_T) with respect to the
 * scan's inputs, given
 *   dz             : [B][H][T][d] fp32, dL/dZ
 *   dw1_T, dw2_T   : [B][H][hidden][d], [B][H][d][hidden] fp32 or NULL (zero)
 *   q, k, v, eta   : the forward's inputs; w1_ckpt, w2_ckpt from
 *                    ttt_mlp_fwd_ckpt with the same b
 * and writing (fp32)
 *   dq, dk, dv : [B][H][T][d];  deta : [B][H][T]
 *   dw1_0, dw2_0 : [B][H][hidden][d], [B][H][d][hidden], per unit.
 * The mini-batches are walked in reverse, each from its checkpoint.  bf16
 * q/k/v with b | 16 run the dual form: the mini-batch's forward is recomputed
 * on MFMA and every product taken back in reverse (the adjoints of W1, W2
 * resident in registers; fp32 factors as bf16 hi + lo halves, ~2^-16
 * relative per product); for b < 16 each mini-batch takes a 16-token tile of
 * its own, the other rows zero tokens (eta = 0: no effect on the state or
 * the other tokens).  Other cases replay the mini-batch forward and take
 * its tokens back one by one in fp32, the gradient-point adjoints joining
 * the state adjoints at its first token.  Outputs must not overlap each
 * other or an input.  T = 0 writes dw*_0 = dw*_T (or zeros).  One workgroup
 * of 512 threads per (batch, head).  Besides the outputs, the kernels use
 * only their own LDS and the per-thread register spill space the compiler
 * assigns.
 */
ttt_status_t ttt_mlp_fwd_ckpt(const void* q, const void* k, const void* v,
                              const float* eta, const float* w1_0,
                              const float* w2_0, int32_t w0_per_batch, int32_t B,
                              int32_t H, int32_t T, int32_t d, int32_t hidden,
                              int32_t b, ttt_dtype_t qkv_dtype, float* z,
                              float* w1_out, float* w2_out, float* w1_ckpt,
                              float* w2_ckpt, void* stream);
ttt_status_t ttt_mlp_bwd(const void* q, const void* k, const void* v,
                         const float* eta, const float* w1_ckpt,
                         const float* w2_ckpt, int32_t B, int32_t H, int32_t T,
                         int32_t d, int32_t hidden, int32_t b,
                         ttt_dtype_t qkv_dtype, const float* dz,
                         const float* dw1_T, const float* dw2_T, float* dq,
                         float* dk, float* dv, float* deta, float* dw1_0,
                         float* dw2_0, void* stream);

/*
 * Learnable inner learning rate (§4.6): the step size of token t in head h
 * depends on the token,
 *   eta[b][h][t] = eta_base * sigmoid(theta_lr[h] . x[b][t]),
 * sigmoid(a) = 1 / (1 + exp(-a)), with x the layer's input token.  The page
 * gives theta_lr as one vector learned by the outer loop; every head runs
 * its own inner loop, so here each head has its own (H = 1 is the page's
 * single vector).  The page's eta_base is 1 for TTT-Linear and 0.1 for
 * TTT-MLP; it is an argument here.
 *
 *   x        : [B][T][dx] bf16, the layer input
 *   theta_lr : [H][dx] fp32
 *   eta_base : finite, else TTT_ERR_VALUE
 *   eta      : out [B][H][T] fp32, the scans' eta layout
 * Support: bf16 x, dx a positive multiple of 32; otherwise
 * TTT_ERR_UNSUPPORTED.  eta must not overlap x or theta_lr.  The dot
 * products are fp32 sums of exact products (theta_lr enters as three bf16
 * terms); sigmoid in fp32.  Empty work (B*T*H == 0) returns TTT_OK.
 */
ttt_status_t ttt_lr_gate(const void* x, ttt_dtype_t x_dtype,
                         const float* theta_lr, float eta_base, int32_t B,
                         int32_t T, int32_t H, int32_t dx, float* eta,
                         void* stream);

/*
 * Backward of the gate: given deta = dL/deta [B][H][T] fp32 and the gate's
 * own output eta [B][H][T] (from ttt_lr_gate with the same x, theta_lr and
 * eta_base), writes
 *   dtheta_lr [H][dx] fp32:   sum_{b,t} da[b][h][t] x[b][t]
 *   dx        [B][T][dx] fp32: sum_h da[b][h][t] theta_lr[h]
 * with da = deta * eta * (1 - eta / eta_base), the derivative of
 * eta_base * sigmoid(a) at the forward's logit a (eta_base = 0: zero).
 * dtheta_lr is deterministic (partial sums over token chunks are added in a
 * fixed order; dx's memory holds them before dx itself is written, so its
 * prior contents do not matter).  Products on the matrix unit: for
 * dtheta_lr, da as a hi + lo bf16 pair against exact bf16 x; for dx, fp32
 * products of da and theta_lr; all sums fp32.  Support and errors as
 * ttt_lr_gate, and B*T*H < 2^30 and B*T*dx < 2^31 (else TTT_ERR_SHAPE);
 * outputs must not overlap each other or an input.  x is taken to be
 * finite: a non-finite element of x makes dtheta_lr non-finite across its
 * 32-column group (x is transposed on the matrix unit by one-hot products).
 */
ttt_status_t ttt_lr_gate_bwd(const void* x, ttt_dtype_t x_dtype,
                             const float* theta_lr, float eta_base,
                             const float* eta, const float* deta, int32_t B,
                             int32_t T, int32_t H, int32_t dx,
                             float* dtheta_lr, float* dx_out, void* stream);

/*
 * The gate followed by the forward scan, on one stream: eta is computed from
 * x into the caller's eta buffer ([B][H][T] fp32, kept as an output for the
 * backward), then the scan runs with it.  All other arguments, layouts,
 * support and errors are those of ttt_lr_gate (x bf16) and of
 * ttt_linear_fwd / ttt_mlp_fwd; every check of both runs before anything is
 * launched, and eta may not overlap any tensor of the scan.
 */
ttt_status_t ttt_linear_gated_fwd(const void* q, const void* k, const void* v,
                                  const void* x, const float* theta_lr,
                                  float eta_base, int32_t dx, const float* w0,
                                  int32_t w0_per_batch, int32_t B, int32_t H,
                                  int32_t T, int32_t d, int32_t b,
                                  ttt_dtype_t qkv_dtype, float* eta, float* z,
                                  float* w_out, void* stream);
ttt_status_t ttt_mlp_gated_fwd(const void* q, const void* k, const void* v,
                               const void* x, const float* theta_lr,
                               float eta_base, int32_t dx, const float* w1_0,
                               const float* w2_0, int32_t w0_per_batch,
                               int32_t B, int32_t H, int32_t T, int32_t d,
                               int32_t hidden, int32_t b,
                               ttt_dtype_t qkv_dtype, float* eta, float* z,
                               float* w1_out, float* w2_out, void* stream);

/* Static description of a status code (never NULL). */
const char* ttt_status_str(ttt_status_t status);

/* Message for the calling thread's most recent non-OK status ("" if none). */
const char* ttt_last_error(void);

/* TTT_ABI_VERSION of the loaded library. */
int32_t ttt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
