// C ABI of libttt.so: argument validation and dispatch to the gfx950 kernels.
// Declarations, layouts and error semantics: include/ttt.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/ttt.h"
#include "../../include/ttt_tuning.h"
#include "ttt_launch.h"

namespace {

thread_local std::string g_last_error;

ttt_status_t fail(ttt_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ttt_status_t fail(ttt_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range rng(const char* name, const void* p, int64_t bytes) {
  uintptr_t lo = (uintptr_t)p;
  return Range{name, lo, p ? lo + (uintptr_t)bytes : lo};
}

bool supported_b(int32_t b) { return b >= 1 && ((b <= 16 && 16 % b == 0) || b % 16 == 0); }

// Shared checks of the two scans.  `inputs` and `outputs` list every tensor
// with its byte extent; `state_pairs` names (input index, output index)
// pairs allowed to coincide exactly when w0_per_batch = 1.
ttt_status_t check_common(const char* fn, ttt_dtype_t dt, int32_t w0_per_batch, int32_t B,
                          int32_t H, int32_t T, int32_t d, int32_t b, const Range* in, int nin,
                          const Range* out, int nout, const int (*pairs)[2], int npairs,
                          bool need_seq) {
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)dt);
  if (B < 0 || H < 0 || T < 0 || d < 0 || b < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d H=%d T=%d d=%d b=%d)", fn, B, H, T, d, b);
  if (w0_per_batch != 0 && w0_per_batch != 1)
    return fail(TTT_ERR_SHAPE, "%s: w0_per_batch must be 0 or 1, got %d", fn, w0_per_batch);
  if (d != 64) return fail(TTT_ERR_UNSUPPORTED, "%s: head dim d=%d unsupported (only 64)", fn, d);
  if (!supported_b(b))
    return fail(TTT_ERR_UNSUPPORTED, "%s: mini-batch b=%d unsupported (need b | 16 or 16 | b)", fn, b);
  const int64_t elems = (int64_t)B * H * T * d;
  if (elems >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H*T*d = %lld exceeds 2^31 - 1", fn, (long long)elems);
  if (T >= (1 << 24))  // a unit's T x 64 fp32 output stays within 32-bit byte offsets
    return fail(TTT_ERR_SHAPE, "%s: T = %d exceeds 2^24 - 1", fn, T);
  if ((int64_t)B * H == 0) return TTT_OK;
  for (int i = 0; i < nin; ++i) {
    const bool seq = i < 4;  // q, k, v, eta come first
    if (seq && !need_seq) continue;
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  for (int i = 0; i < nout; ++i) {
    if (i == 0 && !need_seq) continue;  // z is empty when T == 0
    if (!out[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[i].name);
    if (out[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[i].name);
  }
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i) {
      if (!overlap(out[o], in[i])) continue;
      bool allowed = false;
      for (int p = 0; p < npairs; ++p)
        if (pairs[p][0] == i && pairs[p][1] == o && w0_per_batch == 1 && out[o].lo == in[i].lo &&
            out[o].hi == in[i].hi)
          allowed = true;
      if (!allowed)
        return fail(TTT_ERR_ALIAS, "%s: output %s overlaps input %s%s", fn, out[o].name,
                    in[i].name,
                    w0_per_batch ? "" : " (in-place state update needs w0_per_batch = 1)");
    }
    for (int o2 = o + 1; o2 < nout; ++o2)
      if (overlap(out[o], out[o2]))
        return fail(TTT_ERR_ALIAS, "%s: outputs %s and %s overlap", fn, out[o].name, out[o2].name);
  }
  return TTT_OK;
}

// Rows of W per workgroup: one workgroup per CU when there are enough
// (batch, head) units, finer row slices (more workgroups) when there are few.
int auto_rows(int64_t units) {
  if (units >= 256) return 64;
  if (units > 64) return 32;
  return 16;
}

// Sequence chunks for the chunked scan.  With few units the chip idles
// while each unit's serial chain runs; chunking runs three passes over
// chunks of T / P tokens (two for the maps, one with outputs) at about twice
// the single pass's time per 16-token tile (256 sequences of 64 rows keep
// every CU busy), so it pays from P = 8 on: 8 or 16 chunks with
// units * P <= 256 and chunks of at least 1024 tokens, else one pass.
int auto_chunks(int64_t units, int T) {
  int P = 16;
  while (P >= 8 && (units * P > 256 || T % (16 * P) != 0 || T / P < 1024)) P /= 2;
  return P >= 8 ? P : 1;
}

// The chunk count ttt_linear_fwd picks when the caller leaves it open.
int default_chunks(ttt_dtype_t dt, int b, int64_t units, int T) {
  return (dt == TTT_BF16 && b == 16) ? auto_chunks(units, T) : 1;
}

bool chunks_supported(int P, int T, int b, ttt_dtype_t dt) {
  return P >= 2 && dt == TTT_BF16 && b == 16 && T % P == 0 && (T / P) % 16 == 0 && T / P >= 192;
}

ttt_status_t linear_impl(const void* q, const void* k, const void* v, const float* eta,
                         const float* w0, int32_t w0_per_batch, int32_t B, int32_t H, int32_t T,
                         int32_t d, int32_t b, ttt_dtype_t dt, float* z, float* w_out,
                         void* stream, int32_t rows, float* w_ckpt = nullptr,
                         const char* fn = "ttt_linear_fwd", bool dry = false, int32_t chunks = 0,
                         int32_t ring_depth = 0) {
  if (rows != 0 && rows != 16 && rows != 32 && rows != 64)
    return fail(TTT_ERR_UNSUPPORTED, "%s: rows_per_workgroup=%d (need 0, 16, 32 or 64)", fn, rows);
  if (chunks < 0) return fail(TTT_ERR_UNSUPPORTED, "%s: seq_chunks=%d must be >= 0", fn, chunks);
  const int64_t units = (int64_t)B * H;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t seq = units * T * d;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4),
                      rng("w0", w0, (w0_per_batch ? units : (int64_t)H) * d * d * 4)};
  const int64_t nck = b > 0 ? units * ((T + b - 1) / b) * d * d * 4 : 0;
  const Range out[] = {rng("z", z, seq * 4), rng("w_out", w_out, units * d * d * 4),
                       rng("w_ckpt", w_ckpt, nck)};
  const int pairs[][2] = {{4, 1}};
  ttt_status_t st = check_common(fn, dt, w0_per_batch, B, H, T, d, b, in, 5, out,
                                 w_ckpt ? 3 : 2, pairs, 1, T > 0);
  if (st != TTT_OK || units == 0) return st;
  // checkpoints for fp32 inputs: the primal-form kernel (bf16 with b < 16:
  // the b = 16 kernel, one mini-batch per zero-padded tile)
  const bool ck_primal = w_ckpt && dt != TTT_BF16;
  // chunks: 0 = automatic, 1 = one pass, P >= 2 = P sequence chunks
  int P = chunks;
  if (P == 0) P = default_chunks(dt, b, units, T);
  if (P > 1 && !chunks_supported(P, T, b, dt))
    return fail(TTT_ERR_UNSUPPORTED,
                "%s: seq_chunks=%d needs bf16 q/k/v, b = 16, and T / seq_chunks a multiple of 16 "
                "and >= 192 (T=%d)", fn, P, T);
  if (dry) return TTT_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (T == 0) {
    if (w0_per_batch && w0 == w_out) return TTT_OK;
    e = ttt::launch_copy_state(w0, w0_per_batch, (int)units, H, d * d, w_out, s);
  } else {
    ttt::LinearArgs a{q, k, v, eta, w0, z, w_out, w0_per_batch, (int)units, H, T, b, w_ckpt};
    a.ring_depth = ring_depth;
    if (w_ckpt && b < 16) a.bt = b;
    if (ck_primal)
      e = ttt::launch_linear_primal_ckpt(a, s);
    else if (P > 1)
      e = ttt::launch_linear_chunked(a, P, rows ? rows : auto_rows(units * P), s);
    else
      e = ttt::launch_linear(a, dt == TTT_F32, rows ? rows : auto_rows(units), s);
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t linear_ln_impl(const void* q, const void* k, const void* v, const float* eta,
                            const float* w0, int32_t w0_per_batch, const float* gamma,
                            const float* beta, float eps, int32_t B, int32_t H, int32_t T,
                            int32_t d, int32_t b, ttt_dtype_t dt, float* z, float* w_out,
                            void* stream, float* w_ckpt = nullptr,
                            const char* fn = "ttt_linear_ln_fwd") {
  const int64_t units = (int64_t)B * H;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t seq = units * T * d;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4),
                      rng("w0", w0, (w0_per_batch ? units : (int64_t)H) * d * d * 4),
                      rng("ln_gamma", gamma, (int64_t)H * d * 4),
                      rng("ln_beta", beta, (int64_t)H * d * 4)};
  const int64_t nck = b > 0 ? units * ((T + b - 1) / b) * d * d * 4 : 0;
  const Range out[] = {rng("z", z, seq * 4), rng("w_out", w_out, units * d * d * 4),
                       rng("w_ckpt", w_ckpt, nck)};
  const int pairs[][2] = {{4, 1}};
  ttt_status_t st = check_common(fn, dt, w0_per_batch, B, H, T, d, b, in, 7, out,
                                 w_ckpt && T > 0 ? 3 : 2, pairs, 1, T > 0);
  if (st != TTT_OK) return st;
  if (!(eps > 0.f) || eps > 3.0e38f)
    return fail(TTT_ERR_VALUE, "%s: eps=%g must be finite and > 0", fn, (double)eps);
  if (units == 0) return TTT_OK;
  // bf16 with b | 16 or 16 | b: the dual-form scan (with checkpoint stores
  // when asked; b < 16: one mini-batch per zero-padded tile); fp32: the
  // primal-form kernel
  const bool primal = dt != TTT_BF16 || (b > 16 && b % 16 != 0);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (T == 0) {
    if (w0_per_batch && w0 == w_out) return TTT_OK;
    e = ttt::launch_copy_state(w0, w0_per_batch, (int)units, H, d * d, w_out, s);
  } else {
    ttt::LinearLnArgs a{{q, k, v, eta, w0, z, w_out, w0_per_batch, (int)units, H, T, b, w_ckpt},
                        gamma, beta, eps};
    e = primal ? ttt::launch_linear_ln_primal(a, dt == TTT_F32, s) : ttt::launch_linear_ln(a, s);
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t linear_ln_bwd_impl(const void* q, const void* k, const void* v, const float* eta,
                                const float* w_ckpt, const float* gamma, const float* beta,
                                float eps, int32_t B, int32_t H, int32_t T, int32_t d, int32_t b,
                                ttt_dtype_t dt, const float* dz, const float* dw_T, float* dq,
                                float* dk, float* dv, float* deta, float* dw0, float* dgamma,
                                float* dbeta, void* stream) {
  static const char* fn = "ttt_linear_ln_bwd";
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)dt);
  if (B < 0 || H < 0 || T < 0 || d < 0 || b < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d H=%d T=%d d=%d b=%d)", fn, B, H, T, d, b);
  if (d != 64) return fail(TTT_ERR_UNSUPPORTED, "%s: head dim d=%d unsupported (only 64)", fn, d);
  if (!supported_b(b))
    return fail(TTT_ERR_UNSUPPORTED, "%s: mini-batch b=%d unsupported (need b | 16 or 16 | b)", fn, b);
  if (!(eps > 0.f) || eps > 3.0e38f)
    return fail(TTT_ERR_VALUE, "%s: eps=%g must be finite and > 0", fn, (double)eps);
  const int64_t units = (int64_t)B * H;
  const int64_t seq = units * T * d;
  if (seq >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H*T*d = %lld exceeds 2^31 - 1", fn, (long long)seq);
  if (T >= (1 << 24)) return fail(TTT_ERR_SHAPE, "%s: T = %d exceeds 2^24 - 1", fn, T);
  if (units == 0) return TTT_OK;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t nck = units * ((T + b - 1) / b) * d * d * 4;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4), rng("w_ckpt", w_ckpt, nck),
                      rng("dz", dz, seq * 4), rng("ln_gamma", gamma, (int64_t)H * d * 4),
                      rng("ln_beta", beta, (int64_t)H * d * 4),
                      rng("dw_T", dw_T, units * d * d * 4)};
  const Range out[] = {rng("dq", dq, seq * 4), rng("dk", dk, seq * 4), rng("dv", dv, seq * 4),
                       rng("deta", deta, units * T * 4), rng("dw0", dw0, units * d * d * 4),
                       rng("dgamma", dgamma, units * d * 4), rng("dbeta", dbeta, units * d * 4)};
  for (int i = 0; i < 9; ++i) {
    if ((i < 6 && T == 0) || (i == 8 && !dw_T)) continue;  // gamma, beta always
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  for (int o = 0; o < 7; ++o) {
    if (o < 4 && T == 0) continue;
    if (!out[o].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[o].name);
    if (out[o].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[o].name);
    for (int i = 0; i < 9; ++i)
      if (overlap(out[o], in[i]))
        return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, out[o].name, in[i].name);
    for (int o2 = o + 1; o2 < 7; ++o2)
      if (overlap(out[o], out[o2]))
        return fail(TTT_ERR_ALIAS, "%s: %s and %s overlap", fn, out[o].name, out[o2].name);
  }
  ttt::LinearLnBwdArgs a{q,  k,  v,  eta, w_ckpt, gamma, beta,  eps,        dz,    dw_T, dq,
                         dk, dv, deta, dw0, dgamma, dbeta, (int)units, H, T,  b};
  const hipError_t e = ttt::launch_linear_ln_bwd(a, dt == TTT_F32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

// Shared checks of the decode steps.  `in` / `out` list every tensor with its
// byte extent; states that are updated in place are listed as outputs.
ttt_status_t check_step(const char* fn, ttt_dtype_t dt, int32_t B, int32_t H, int32_t d, int32_t b,
                        const Range* in, int nin, const Range* out, int nout,
                        const bool* optional_out) {
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)dt);
  if (B < 0 || H < 0 || d < 0 || b < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d H=%d d=%d b=%d)", fn, B, H, d, b);
  if (d != 64) return fail(TTT_ERR_UNSUPPORTED, "%s: head dim d=%d unsupported (only 64)", fn, d);
  if (b < 1) return fail(TTT_ERR_UNSUPPORTED, "%s: mini-batch b=%d unsupported (need b >= 1)", fn, b);
  if ((int64_t)B * H * d * 256 >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H = %lld units is too many for one call", fn,
                (long long)B * H);
  if ((int64_t)B * H == 0) return TTT_OK;
  for (int i = 0; i < nin; ++i) {
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  for (int o = 0; o < nout; ++o) {
    if (!out[o].lo) {
      if (optional_out && optional_out[o]) continue;
      return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[o].name);
    }
    if (out[o].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[o].name);
    for (int i = 0; i < nin; ++i)
      if (overlap(out[o], in[i]))
        return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, out[o].name, in[i].name);
    for (int o2 = o + 1; o2 < nout; ++o2)
      if (overlap(out[o], out[o2]))
        return fail(TTT_ERR_ALIAS, "%s: %s and %s overlap", fn, out[o].name, out[o2].name);
  }
  return TTT_OK;
}

ttt_status_t linear_step_impl(const char* fn, const void* q, const void* k, const void* v,
                              const float* eta, float* w, float* w_gp, const int32_t* pos,
                              const float* gamma, const float* beta, float eps, bool ln,
                              int32_t B, int32_t H, int32_t d, int32_t b, ttt_dtype_t dt, float* z,
                              void* stream) {
  const int64_t units = (int64_t)B * H;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const Range in_all[] = {rng("q", q, units * d * es), rng("k", k, units * d * es),
                          rng("v", v, units * d * es), rng("eta", eta, units * 4),
                          rng("pos", pos, (int64_t)B * 4),
                          rng("ln_gamma", gamma, (int64_t)H * d * 4),
                          rng("ln_beta", beta, (int64_t)H * d * 4)};
  const Range out[] = {rng("z", z, units * d * 4), rng("w", w, units * d * d * 4),
                       rng("w_gp", w_gp, units * d * d * 4)};
  const bool optional[] = {false, false, b == 1};
  // pos only needs 4-byte alignment; check it apart from the 16-byte rule
  Range in[7];
  int nin = 0;
  for (int i = 0; i < (ln ? 7 : 5); ++i)
    if (i != 4) in[nin++] = in_all[i];
  ttt_status_t st = check_step(fn, dt, B, H, d, b, in, nin, out, 3, optional);
  if (st != TTT_OK || units == 0) return st;
  if (!w_gp && b != 1)
    return fail(TTT_ERR_NULL, "%s: w_gp is NULL (allowed only for b = 1)", fn);
  if (!pos) return fail(TTT_ERR_NULL, "%s: pos is NULL", fn);
  if ((uintptr_t)pos & 3) return fail(TTT_ERR_ALIGN, "%s: pos is not 4-byte aligned", fn);
  for (int o = 0; o < 3; ++o)
    if (overlap(out[o], in_all[4]))
      return fail(TTT_ERR_ALIAS, "%s: %s overlaps input pos", fn, out[o].name);
  if (ln && (!(eps > 0.f) || eps > 3.0e38f))
    return fail(TTT_ERR_VALUE, "%s: eps=%g must be finite and > 0", fn, (double)eps);
  ttt::StepArgs a{q, k, v, eta, w, w_gp, nullptr, nullptr, pos, z, (int)units, H, b};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = ln ? ttt::launch_linear_ln_step(a, gamma, beta, eps, dt == TTT_F32, s)
                    : ttt::launch_linear_step(a, dt == TTT_F32, s);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t mlp_step_impl(const void* q, const void* k, const void* v, const float* eta,
                           float* w1, float* w2, float* w1_gp, float* w2_gp, const int32_t* pos,
                           int32_t B, int32_t H, int32_t d, int32_t hidden, int32_t b,
                           ttt_dtype_t dt, float* z, void* stream) {
  static const char* fn = "ttt_mlp_step";
  if (hidden < 0) return fail(TTT_ERR_SHAPE, "%s: negative hidden=%d", fn, hidden);
  const int64_t units = (int64_t)B * H;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t sb = units * hidden * d * 4;
  const Range in[] = {rng("q", q, units * d * es), rng("k", k, units * d * es),
                      rng("v", v, units * d * es), rng("eta", eta, units * 4)};
  const Range out[] = {rng("z", z, units * d * 4), rng("w1", w1, sb), rng("w2", w2, sb),
                       rng("w1_gp", w1_gp, sb), rng("w2_gp", w2_gp, sb)};
  const bool optional[] = {false, false, false, b == 1, b == 1};
  ttt_status_t st = check_step(fn, dt, B, H, d, b, in, 4, out, 5, optional);
  if (st != TTT_OK) return st;
  if (hidden != 256)
    return fail(TTT_ERR_UNSUPPORTED, "%s: hidden=%d unsupported (only 256)", fn, hidden);
  if (units == 0) return TTT_OK;
  if ((!w1_gp || !w2_gp) && b != 1)
    return fail(TTT_ERR_NULL, "%s: w1_gp / w2_gp are NULL (allowed only for b = 1)", fn);
  if ((!w1_gp) != (!w2_gp))
    return fail(TTT_ERR_NULL, "%s: pass both gradient points or neither", fn);
  if (!pos) return fail(TTT_ERR_NULL, "%s: pos is NULL", fn);
  if ((uintptr_t)pos & 3) return fail(TTT_ERR_ALIGN, "%s: pos is not 4-byte aligned", fn);
  const Range rp = rng("pos", pos, (int64_t)B * 4);
  for (int o = 0; o < 5; ++o)
    if (overlap(out[o], rp)) return fail(TTT_ERR_ALIAS, "%s: %s overlaps input pos", fn, out[o].name);
  ttt::StepArgs a{q, k, v, eta, w1, w1_gp, w2, w2_gp, pos, z, (int)units, H, b};
  hipError_t e = ttt::launch_mlp_step(a, dt == TTT_F32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t linear_bwd_impl(const void* q, const void* k, const void* v, const float* eta,
                            const float* w_ckpt, int32_t B, int32_t H, int32_t T, int32_t d,
                            int32_t b, ttt_dtype_t dt, const float* dz, const float* dw_T,
                            float* dq, float* dk, float* dv, float* deta, float* dw0,
                            void* stream, int32_t chunks = 0, const char* fn = "ttt_linear_bwd") {
  const int64_t units = (int64_t)B * H;
  const int64_t seq = units * T * d;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t nck = b > 0 ? units * ((T + b - 1) / b) * d * d * 4 : 0;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4), rng("w_ckpt", w_ckpt, nck),
                      rng("dz", dz, seq * 4), rng("dw_T", dw_T, units * d * d * 4)};
  const Range out[] = {rng("dq", dq, seq * 4), rng("dk", dk, seq * 4), rng("dv", dv, seq * 4),
                       rng("deta", deta, units * T * 4), rng("dw0", dw0, units * d * d * 4)};
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)dt);
  if (B < 0 || H < 0 || T < 0 || d < 0 || b < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d H=%d T=%d d=%d b=%d)", fn, B, H, T, d, b);
  if (d != 64) return fail(TTT_ERR_UNSUPPORTED, "%s: head dim d=%d unsupported (only 64)", fn, d);
  if (!supported_b(b))
    return fail(TTT_ERR_UNSUPPORTED, "%s: mini-batch b=%d unsupported (need b | 16 or 16 | b)", fn, b);
  // bf16 with b = 16: the dual-form kernel (and its sequence chunks); bf16
  // with b < 16: the same kernel, one mini-batch per zero-padded tile; bf16
  // with b > 16: the same kernel with the gradient point held across b / 16
  // tiles; fp32 inputs: the primal-form kernel, one pass
  const bool primal = dt != TTT_BF16;
  if ((primal || b != 16) && chunks > 1)
    return fail(TTT_ERR_UNSUPPORTED, "%s: seq_chunks=%d needs bf16 q/k/v and b = 16", fn, chunks);
  if (seq >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H*T*d = %lld exceeds 2^31 - 1", fn, (long long)seq);
  if (T >= (1 << 24))  // a unit's T x 64 fp32 gradients stay within 32-bit byte offsets
    return fail(TTT_ERR_SHAPE, "%s: T = %d exceeds 2^24 - 1", fn, T);
  if (chunks < 0) return fail(TTT_ERR_UNSUPPORTED, "%s: seq_chunks=%d must be >= 0", fn, chunks);
  const int P = primal ? 1 : (chunks ? chunks : default_chunks(dt, b, units, T));
  if (P > 1 && !chunks_supported(P, T, b, dt))
    return fail(TTT_ERR_UNSUPPORTED,
                "%s: seq_chunks=%d needs T / seq_chunks a multiple of 16 and >= 192 (T=%d)", fn, P, T);
  if (units == 0) return TTT_OK;
  for (int i = 0; i < 7; ++i) {
    const bool seqt = i < 6;  // empty when T == 0
    if ((seqt && T == 0) || (i == 6 && !dw_T)) continue;
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  if (T > 0 && !w_ckpt) return fail(TTT_ERR_NULL, "%s: w_ckpt is NULL", fn);
  for (int o = 0; o < 5; ++o) {
    if ((o != 4 && T == 0)) continue;
    if (!out[o].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[o].name);
    if (out[o].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[o].name);
    for (int i = 0; i < 7; ++i)
      if (overlap(out[o], in[i]))
        return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, out[o].name, in[i].name);
    for (int o2 = o + 1; o2 < 5; ++o2)
      if (overlap(out[o], out[o2]))
        return fail(TTT_ERR_ALIAS, "%s: %s and %s overlap", fn, out[o].name, out[o2].name);
  }
  hipError_t e;
  if (primal) {
    ttt::LinearPrimalBwdArgs a{q, k, v, eta, w_ckpt, dz, dw_T, dq, dk, dv, deta, dw0, (int)units, T, b};
    e = ttt::launch_linear_primal_bwd(a, (hipStream_t)stream);
  } else {
    ttt::LinearBwdArgs a{q, k, v, eta, w_ckpt, dz, dw_T, dq, dk, dv, deta, dw0, (int)units, H, T};
    a.bt = b < 16 ? b : 16;
    a.tpm = b > 16 ? b / 16 : 1;
    e = P > 1 ? ttt::launch_linear_bwd_chunked(a, P, auto_rows(units * P), (hipStream_t)stream)
              : ttt::launch_linear_bwd(a, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t mlp_impl(const void* q, const void* k, const void* v, const float* eta,
                      const float* w1_0, const float* w2_0, int32_t w0_per_batch, int32_t B,
                      int32_t H, int32_t T, int32_t d, int32_t hidden, int32_t b,
                      ttt_dtype_t qkv_dtype, float* z, float* w1_out, float* w2_out, void* stream,
                      const char* fn = "ttt_mlp_fwd", bool dry = false, float* w1_ckpt = nullptr,
                      float* w2_ckpt = nullptr) {
  if (hidden < 0) return fail(TTT_ERR_SHAPE, "%s: negative hidden=%d", fn, hidden);
  const int64_t units = (int64_t)B * H;
  const int64_t es = qkv_dtype == TTT_F32 ? 4 : 2;
  const int64_t seq = units * T * d;
  const int64_t wn = (w0_per_batch ? units : (int64_t)H) * hidden * d * 4;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4), rng("w1_0", w1_0, wn),
                      rng("w2_0", w2_0, wn)};
  const int64_t nck = b > 0 ? units * ((T + b - 1) / b) * hidden * d * 4 : 0;
  const Range out[] = {rng("z", z, seq * 4), rng("w1_out", w1_out, units * hidden * d * 4),
                       rng("w2_out", w2_out, units * hidden * d * 4),
                       rng("w1_ckpt", w1_ckpt, nck), rng("w2_ckpt", w2_ckpt, nck)};
  const int pairs[][2] = {{4, 1}, {5, 2}};
  const bool ck = w1_ckpt != nullptr || w2_ckpt != nullptr;
  if (ck && (!w1_ckpt || !w2_ckpt) && T > 0)
    return fail(TTT_ERR_NULL, "%s: w1_ckpt and w2_ckpt must both be given", fn);
  ttt_status_t st = check_common(fn, qkv_dtype, w0_per_batch, B, H, T, d, b, in, 6, out,
                                 ck && T > 0 ? 5 : 3, pairs, 2, T > 0);
  if (st != TTT_OK) return st;
  if (hidden != 256)
    return fail(TTT_ERR_UNSUPPORTED, "%s: hidden=%d unsupported (only 256)", fn, hidden);
  if (units == 0 || dry) return TTT_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T == 0) {
    if (!(w0_per_batch && w1_0 == w1_out))
      e = ttt::launch_copy_state(w1_0, w0_per_batch, (int)units, H, hidden * d, w1_out, s);
    if (e == hipSuccess && !(w0_per_batch && w2_0 == w2_out))
      e = ttt::launch_copy_state(w2_0, w0_per_batch, (int)units, H, hidden * d, w2_out, s);
  } else {
    ttt::MlpArgs a{q, k, v, eta, w1_0, w2_0, z, w1_out, w2_out, w0_per_batch, (int)units, H, T, b,
                   w1_ckpt, w2_ckpt};
    e = ttt::launch_mlp(a, qkv_dtype == TTT_F32, s);
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t mlp_ln_impl(const void* q, const void* k, const void* v, const float* eta,
                         const float* w1_0, const float* w2_0, int32_t w0_per_batch,
                         const float* gamma, const float* beta, float eps, int32_t B, int32_t H,
                         int32_t T, int32_t d, int32_t hidden, int32_t b, ttt_dtype_t dt,
                         float* z, float* w1_out, float* w2_out, void* stream) {
  static const char* fn = "ttt_mlp_ln_fwd";
  if (hidden < 0) return fail(TTT_ERR_SHAPE, "%s: negative hidden=%d", fn, hidden);
  const int64_t units = (int64_t)B * H;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t seq = units * T * d;
  const int64_t wn = (w0_per_batch ? units : (int64_t)H) * hidden * d * 4;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4), rng("w1_0", w1_0, wn),
                      rng("w2_0", w2_0, wn), rng("ln_gamma", gamma, (int64_t)H * d * 4),
                      rng("ln_beta", beta, (int64_t)H * d * 4)};
  const Range out[] = {rng("z", z, seq * 4), rng("w1_out", w1_out, units * hidden * d * 4),
                       rng("w2_out", w2_out, units * hidden * d * 4)};
  const int pairs[][2] = {{4, 1}, {5, 2}};
  ttt_status_t st = check_common(fn, dt, w0_per_batch, B, H, T, d, b, in, 8, out, 3, pairs, 2,
                                 T > 0);
  if (st != TTT_OK) return st;
  if (hidden != 256)
    return fail(TTT_ERR_UNSUPPORTED, "%s: hidden=%d unsupported (only 256)", fn, hidden);
  if (!(eps > 0.f) || eps > 3.0e38f)
    return fail(TTT_ERR_VALUE, "%s: eps=%g must be finite and > 0", fn, (double)eps);
  if (units == 0) return TTT_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T == 0) {
    if (!(w0_per_batch && w1_0 == w1_out))
      e = ttt::launch_copy_state(w1_0, w0_per_batch, (int)units, H, hidden * d, w1_out, s);
    if (e == hipSuccess && !(w0_per_batch && w2_0 == w2_out))
      e = ttt::launch_copy_state(w2_0, w0_per_batch, (int)units, H, hidden * d, w2_out, s);
  } else {
    const ttt::MlpLnArgs a{{q, k, v, eta, w1_0, w2_0, z, w1_out, w2_out, w0_per_batch, (int)units,
                            H, T, b},
                           gamma, beta, eps};
    e = ttt::launch_mlp_ln(a, dt == TTT_F32, s);
  }
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t mlp_bwd_impl(const void* q, const void* k, const void* v, const float* eta,
                          const float* w1_ckpt, const float* w2_ckpt, int32_t B, int32_t H,
                          int32_t T, int32_t d, int32_t hidden, int32_t b, ttt_dtype_t dt,
                          const float* dz, const float* dw1_T, const float* dw2_T, float* dq,
                          float* dk, float* dv, float* deta, float* dw1_0, float* dw2_0,
                          void* stream) {
  static const char* fn = "ttt_mlp_bwd";
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)dt);
  if (B < 0 || H < 0 || T < 0 || d < 0 || b < 0 || hidden < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d H=%d T=%d d=%d hidden=%d b=%d)", fn, B, H, T,
                d, hidden, b);
  if (d != 64) return fail(TTT_ERR_UNSUPPORTED, "%s: head dim d=%d unsupported (only 64)", fn, d);
  if (hidden != 256)
    return fail(TTT_ERR_UNSUPPORTED, "%s: hidden=%d unsupported (only 256)", fn, hidden);
  if (!supported_b(b))
    return fail(TTT_ERR_UNSUPPORTED, "%s: mini-batch b=%d unsupported (need b | 16 or 16 | b)", fn, b);
  const int64_t units = (int64_t)B * H;
  const int64_t seq = units * T * d;
  if (seq >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H*T*d = %lld exceeds 2^31 - 1", fn, (long long)seq);
  if (T >= (1 << 24)) return fail(TTT_ERR_SHAPE, "%s: T = %d exceeds 2^24 - 1", fn, T);
  if (units == 0) return TTT_OK;
  const int64_t es = dt == TTT_F32 ? 4 : 2;
  const int64_t nst = units * hidden * d * 4;
  const int64_t nck = units * ((T + b - 1) / b) * hidden * d * 4;
  const Range in[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                      rng("eta", eta, units * T * 4), rng("w1_ckpt", w1_ckpt, nck),
                      rng("w2_ckpt", w2_ckpt, nck), rng("dz", dz, seq * 4),
                      rng("dw1_T", dw1_T, nst), rng("dw2_T", dw2_T, nst)};
  const Range out[] = {rng("dq", dq, seq * 4), rng("dk", dk, seq * 4), rng("dv", dv, seq * 4),
                       rng("deta", deta, units * T * 4), rng("dw1_0", dw1_0, nst),
                       rng("dw2_0", dw2_0, nst)};
  for (int i = 0; i < 9; ++i) {
    if ((i < 7 && T == 0) || (i == 7 && !dw1_T) || (i == 8 && !dw2_T)) continue;
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  for (int o = 0; o < 6; ++o) {
    if (o < 4 && T == 0) continue;
    if (!out[o].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[o].name);
    if (out[o].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[o].name);
    for (int i = 0; i < 9; ++i)
      if (overlap(out[o], in[i]))
        return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, out[o].name, in[i].name);
    for (int o2 = o + 1; o2 < 6; ++o2)
      if (overlap(out[o], out[o2]))
        return fail(TTT_ERR_ALIAS, "%s: %s and %s overlap", fn, out[o].name, out[o2].name);
  }
  ttt::MlpBwdArgs a{q,  k,  v,  eta,  w1_ckpt, w2_ckpt, dz, dw1_T, dw2_T, dq, dk, dv, deta, dw1_0,
                    dw2_0, (int)units, T, b};
  const hipError_t e = ttt::launch_mlp_bwd(a, dt == TTT_F32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}


// Checks of the learning-rate gate; `fn` names the entry point in messages.
ttt_status_t gate_check(const char* fn, const void* x, ttt_dtype_t x_dtype, const float* theta,
                        float eta_base, int32_t B, int32_t T, int32_t H, int32_t dx,
                        const float* eta) {
  if (x_dtype != TTT_F32 && x_dtype != TTT_BF16)
    return fail(TTT_ERR_DTYPE, "%s: unknown x dtype %d", fn, (int)x_dtype);
  if (B < 0 || T < 0 || H < 0 || dx < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d T=%d H=%d dx=%d)", fn, B, T, H, dx);
  if (dx == 0 || dx % 32 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "%s: dx=%d unsupported (need a positive multiple of 32)", fn, dx);
  if (x_dtype != TTT_BF16) return fail(TTT_ERR_UNSUPPORTED, "%s: only bf16 x is supported", fn);
  if (!(eta_base == eta_base) || eta_base > 3.4e38f || eta_base < -3.4e38f)
    return fail(TTT_ERR_VALUE, "%s: eta_base=%g must be finite", fn, (double)eta_base);
  const int64_t ntok = (int64_t)B * T;
  if (ntok * H >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*H*T = %lld exceeds 2^31 - 1", fn, (long long)(ntok * H));
  if (ntok * H == 0) return TTT_OK;
  const Range in[] = {rng("x", x, ntok * dx * 2), rng("theta_lr", theta, (int64_t)H * dx * 4)};
  const Range out = rng("eta", eta, ntok * H * 4);
  for (int i = 0; i < 2; ++i) {
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  if (!out.lo) return fail(TTT_ERR_NULL, "%s: eta is NULL", fn);
  if (out.lo & 15) return fail(TTT_ERR_ALIGN, "%s: eta is not 16-byte aligned", fn);
  for (int i = 0; i < 2; ++i)
    if (overlap(out, in[i])) return fail(TTT_ERR_ALIAS, "%s: eta overlaps input %s", fn, in[i].name);
  return TTT_OK;
}

ttt_status_t gate_launch(const char* fn, const void* x, const float* theta, float eta_base,
                         int32_t B, int32_t T, int32_t H, int32_t dx, float* eta, void* stream,
                         int tokens_per_workgroup = 0) {
  ttt::GateArgs a{x, theta, eta, eta_base, B, T, H, dx};
  hipError_t e = ttt::launch_lr_gate(a, tokens_per_workgroup, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

// The gate's x, theta and eta against the tensors of the scan that follows:
// eta may not overlap anything the scan reads or writes, and the scan's
// outputs may not overlap the gate's inputs.
ttt_status_t gate_scan_alias(const char* fn, const void* x, const float* theta, const float* eta,
                             int32_t B, int32_t T, int32_t H, int32_t dx, const Range* scan,
                             int nscan, int first_out) {
  const int64_t ntok = (int64_t)B * T;
  if (ntok * H == 0) return TTT_OK;
  const Range ge = rng("eta", eta, ntok * H * 4);
  const Range gi[] = {rng("x", x, ntok * dx * 2), rng("theta_lr", theta, (int64_t)H * dx * 4)};
  for (int i = 0; i < nscan; ++i) {
    if (overlap(ge, scan[i])) return fail(TTT_ERR_ALIAS, "%s: eta overlaps %s", fn, scan[i].name);
    if (i >= first_out)
      for (int j = 0; j < 2; ++j)
        if (overlap(scan[i], gi[j]))
          return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, scan[i].name, gi[j].name);
  }
  return TTT_OK;
}
}  // namespace

extern "C" {

ttt_status_t ttt_linear_fwd_ckpt(const void* q, const void* k, const void* v, const float* eta,
                                 const float* w0, int32_t w0_per_batch, int32_t B, int32_t H,
                                 int32_t T, int32_t d, int32_t b, ttt_dtype_t qkv_dtype, float* z,
                                 float* w_out, float* w_ckpt, void* stream) {
  if ((int64_t)B * H > 0 && T > 0 && !w_ckpt)
    return fail(TTT_ERR_NULL, "ttt_linear_fwd_ckpt: w_ckpt is NULL");
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     0, w_ckpt, "ttt_linear_fwd_ckpt");
}

ttt_status_t ttt_linear_bwd(const void* q, const void* k, const void* v, const float* eta,
                            const float* w_ckpt, int32_t B, int32_t H, int32_t T, int32_t d,
                            int32_t b, ttt_dtype_t qkv_dtype, const float* dz, const float* dw_T,
                            float* dq, float* dk, float* dv, float* deta, float* dw0,
                            void* stream) {
  return linear_bwd_impl(q, k, v, eta, w_ckpt, B, H, T, d, b, qkv_dtype, dz, dw_T, dq, dk, dv,
                         deta, dw0, stream);
}

ttt_status_t ttt_linear_bwd_chunked(const void* q, const void* k, const void* v, const float* eta,
                                    const float* w_ckpt, int32_t B, int32_t H, int32_t T, int32_t d,
                                    int32_t b, ttt_dtype_t qkv_dtype, const float* dz,
                                    const float* dw_T, float* dq, float* dk, float* dv, float* deta,
                                    float* dw0, void* stream, int32_t seq_chunks) {
  return linear_bwd_impl(q, k, v, eta, w_ckpt, B, H, T, d, b, qkv_dtype, dz, dw_T, dq, dk, dv,
                         deta, dw0, stream, seq_chunks, "ttt_linear_bwd_chunked");
}

ttt_status_t ttt_mlp_step(const void* q, const void* k, const void* v, const float* eta,
                          float* w1, float* w2, float* w1_gp, float* w2_gp, const int32_t* pos,
                          int32_t B, int32_t H, int32_t d, int32_t hidden, int32_t b,
                          ttt_dtype_t qkv_dtype, float* z, void* stream) {
  return mlp_step_impl(q, k, v, eta, w1, w2, w1_gp, w2_gp, pos, B, H, d, hidden, b, qkv_dtype, z,
                       stream);
}

ttt_status_t ttt_linear_step(const void* q, const void* k, const void* v, const float* eta,
                             float* w, float* w_gp, const int32_t* pos, int32_t B, int32_t H,
                             int32_t d, int32_t b, ttt_dtype_t qkv_dtype, float* z, void* stream) {
  return linear_step_impl("ttt_linear_step", q, k, v, eta, w, w_gp, pos, nullptr, nullptr, 0.f,
                          false, B, H, d, b, qkv_dtype, z, stream);
}

ttt_status_t ttt_linear_ln_step(const void* q, const void* k, const void* v, const float* eta,
                                float* w, float* w_gp, const int32_t* pos, const float* ln_gamma,
                                const float* ln_beta, float eps, int32_t B, int32_t H, int32_t d,
                                int32_t b, ttt_dtype_t qkv_dtype, float* z, void* stream) {
  return linear_step_impl("ttt_linear_ln_step", q, k, v, eta, w, w_gp, pos, ln_gamma, ln_beta,
                          eps, true, B, H, d, b, qkv_dtype, z, stream);
}


ttt_status_t ttt_linear_fwd(const void* q, const void* k, const void* v, const float* eta,
                            const float* w0, int32_t w0_per_batch, int32_t B, int32_t H,
                            int32_t T, int32_t d, int32_t b, ttt_dtype_t qkv_dtype, float* z,
                            float* w_out, void* stream) {
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     0);
}

ttt_status_t ttt_linear_fwd_tuned(const void* q, const void* k, const void* v, const float* eta,
                                  const float* w0, int32_t w0_per_batch, int32_t B, int32_t H,
                                  int32_t T, int32_t d, int32_t b, ttt_dtype_t qkv_dtype,
                                  float* z, float* w_out, void* stream,
                                  int32_t rows_per_workgroup) {
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     rows_per_workgroup, nullptr, "ttt_linear_fwd_tuned", false, 1);
}

ttt_status_t ttt_linear_fwd_ring_depth(const void* q, const void* k, const void* v,
                                       const float* eta, const float* w0, int32_t w0_per_batch,
                                       int32_t B, int32_t H, int32_t T, int32_t d, int32_t b,
                                       ttt_dtype_t qkv_dtype, float* z, float* w_out, void* stream,
                                       int32_t rows_per_workgroup, int32_t ring_depth) {
  static const char* fn = "ttt_linear_fwd_ring_depth";
  if (ring_depth != 0 && ring_depth != 1)
    return fail(TTT_ERR_UNSUPPORTED, "%s: ring_depth=%d (need 0 or 1)", fn, ring_depth);
  if (ring_depth == 1 && (qkv_dtype != TTT_BF16 || b != 16))
    return fail(TTT_ERR_UNSUPPORTED, "%s: ring_depth = 1 needs bf16 q/k/v and b = 16", fn);
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     rows_per_workgroup, nullptr, fn, false, 1, ring_depth);
}

ttt_status_t ttt_linear_fwd_plan(int32_t B, int32_t H, int32_t T, int32_t b, ttt_dtype_t qkv_dtype,
                                 int32_t* rows_per_workgroup, int32_t* seq_chunks) {
  static const char* fn = "ttt_linear_fwd_plan";
  if (!rows_per_workgroup || !seq_chunks) return fail(TTT_ERR_NULL, "%s: output pointer is NULL", fn);
  if (qkv_dtype != TTT_F32 && qkv_dtype != TTT_BF16)
    return fail(TTT_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, (int)qkv_dtype);
  if (B < 0 || H < 0 || T < 0 || b < 1)
    return fail(TTT_ERR_SHAPE, "%s: negative size or b < 1 (B=%d H=%d T=%d b=%d)", fn, B, H, T, b);
  const int64_t units = (int64_t)B * H;
  const int P = default_chunks(qkv_dtype, b, units, T);
  *seq_chunks = P;
  *rows_per_workgroup = auto_rows(units * P);
  return TTT_OK;
}

ttt_status_t ttt_linear_fwd_chunked(const void* q, const void* k, const void* v, const float* eta,
                                    const float* w0, int32_t w0_per_batch, int32_t B, int32_t H,
                                    int32_t T, int32_t d, int32_t b, ttt_dtype_t qkv_dtype,
                                    float* z, float* w_out, void* stream,
                                    int32_t rows_per_workgroup, int32_t seq_chunks) {
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     rows_per_workgroup, nullptr, "ttt_linear_fwd_chunked", false, seq_chunks);
}

ttt_status_t ttt_linear_ln_fwd(const void* q, const void* k, const void* v, const float* eta,
                               const float* w0, int32_t w0_per_batch, const float* ln_gamma,
                               const float* ln_beta, float eps, int32_t B, int32_t H, int32_t T,
                               int32_t d, int32_t b, ttt_dtype_t qkv_dtype, float* z,
                               float* w_out, void* stream) {
  return linear_ln_impl(q, k, v, eta, w0, w0_per_batch, ln_gamma, ln_beta, eps, B, H, T, d, b,
                        qkv_dtype, z, w_out, stream);
}

ttt_status_t ttt_linear_ln_fwd_ckpt(const void* q, const void* k, const void* v,
                                   const float* eta, const float* w0, int32_t w0_per_batch,
                                   const float* ln_gamma, const float* ln_beta, float eps,
                                   int32_t B, int32_t H, int32_t T, int32_t d, int32_t b,
                                   ttt_dtype_t qkv_dtype, float* z, float* w_out, float* w_ckpt,
                                   void* stream) {
  if (T > 0 && !w_ckpt) return fail(TTT_ERR_NULL, "ttt_linear_ln_fwd_ckpt: w_ckpt is NULL");
  return linear_ln_impl(q, k, v, eta, w0, w0_per_batch, ln_gamma, ln_beta, eps, B, H, T, d, b,
                        qkv_dtype, z, w_out, stream, w_ckpt, "ttt_linear_ln_fwd_ckpt");
}

ttt_status_t ttt_linear_ln_bwd(const void* q, const void* k, const void* v, const float* eta,
                               const float* w_ckpt, const float* ln_gamma, const float* ln_beta,
                               float eps, int32_t B, int32_t H, int32_t T, int32_t d, int32_t b,
                               ttt_dtype_t qkv_dtype, const float* dz, const float* dw_T,
                               float* dq, float* dk, float* dv, float* deta, float* dw0,
                               float* dgamma, float* dbeta, void* stream) {
  return linear_ln_bwd_impl(q, k, v, eta, w_ckpt, ln_gamma, ln_beta, eps, B, H, T, d, b, qkv_dtype,
                            dz, dw_T, dq, dk, dv, deta, dw0, dgamma, dbeta, stream);
}

ttt_status_t ttt_mlp_fwd_ckpt(const void* q, const void* k, const void* v, const float* eta,
                              const float* w1_0, const float* w2_0, int32_t w0_per_batch,
                              int32_t B, int32_t H, int32_t T, int32_t d, int32_t hidden,
                              int32_t b, ttt_dtype_t qkv_dtype, float* z, float* w1_out,
                              float* w2_out, float* w1_ckpt, float* w2_ckpt, void* stream) {
  if (T > 0 && (!w1_ckpt || !w2_ckpt))
    return fail(TTT_ERR_NULL, "ttt_mlp_fwd_ckpt: w1_ckpt and w2_ckpt are required");
  return mlp_impl(q, k, v, eta, w1_0, w2_0, w0_per_batch, B, H, T, d, hidden, b, qkv_dtype, z,
                  w1_out, w2_out, stream, "ttt_mlp_fwd_ckpt", false, w1_ckpt, w2_ckpt);
}

ttt_status_t ttt_mlp_bwd(const void* q, const void* k, const void* v, const float* eta,
                         const float* w1_ckpt, const float* w2_ckpt, int32_t B, int32_t H,
                         int32_t T, int32_t d, int32_t hidden, int32_t b, ttt_dtype_t qkv_dtype,
                         const float* dz, const float* dw1_T, const float* dw2_T, float* dq,
                         float* dk, float* dv, float* deta, float* dw1_0, float* dw2_0,
                         void* stream) {
  return mlp_bwd_impl(q, k, v, eta, w1_ckpt, w2_ckpt, B, H, T, d, hidden, b, qkv_dtype, dz, dw1_T,
                      dw2_T, dq, dk, dv, deta, dw1_0, dw2_0, stream);
}

ttt_status_t ttt_mlp_fwd(const void* q, const void* k, const void* v, const float* eta,
                         const float* w1_0, const float* w2_0, int32_t w0_per_batch, int32_t B,
                         int32_t H, int32_t T, int32_t d, int32_t hidden, int32_t b,
                         ttt_dtype_t qkv_dtype, float* z, float* w1_out, float* w2_out,
                         void* stream) {
  return mlp_impl(q, k, v, eta, w1_0, w2_0, w0_per_batch, B, H, T, d, hidden, b, qkv_dtype, z,
                  w1_out, w2_out, stream);
}

ttt_status_t ttt_mlp_ln_fwd(const void* q, const void* k, const void* v, const float* eta,
                            const float* w1_0, const float* w2_0, int32_t w0_per_batch,
                            const float* ln_gamma, const float* ln_beta, float eps, int32_t B,
                            int32_t H, int32_t T, int32_t d, int32_t hidden, int32_t b,
                            ttt_dtype_t qkv_dtype, float* z, float* w1_out, float* w2_out,
                            void* stream) {
  return mlp_ln_impl(q, k, v, eta, w1_0, w2_0, w0_per_batch, ln_gamma, ln_beta, eps, B, H, T, d,
                     hidden, b, qkv_dtype, z, w1_out, w2_out, stream);
}

ttt_status_t ttt_lr_gate(const void* x, ttt_dtype_t x_dtype, const float* theta_lr,
                         float eta_base, int32_t B, int32_t T, int32_t H, int32_t dx, float* eta,
                         void* stream) {
  static const char* fn = "ttt_lr_gate";
  ttt_status_t st = gate_check(fn, x, x_dtype, theta_lr, eta_base, B, T, H, dx, eta);
  if (st != TTT_OK) return st;
  return gate_launch(fn, x, theta_lr, eta_base, B, T, H, dx, eta, stream);
}

ttt_status_t ttt_lr_gate_tuned(const void* x, ttt_dtype_t x_dtype, const float* theta_lr,
                               float eta_base, int32_t B, int32_t T, int32_t H, int32_t dx,
                               float* eta, void* stream, int32_t tokens_per_workgroup) {
  static const char* fn = "ttt_lr_gate_tuned";
  if (tokens_per_workgroup != 0 && tokens_per_workgroup != 32 && tokens_per_workgroup != 64)
    return fail(TTT_ERR_UNSUPPORTED, "%s: tokens_per_workgroup=%d (need 0, 32 or 64)", fn,
                tokens_per_workgroup);
  ttt_status_t st = gate_check(fn, x, x_dtype, theta_lr, eta_base, B, T, H, dx, eta);
  if (st != TTT_OK) return st;
  return gate_launch(fn, x, theta_lr, eta_base, B, T, H, dx, eta, stream, tokens_per_workgroup);
}

ttt_status_t ttt_lr_gate_bwd(const void* x, ttt_dtype_t x_dtype, const float* theta_lr,
                             float eta_base, const float* eta, const float* deta, int32_t B,
                             int32_t T, int32_t H, int32_t dx, float* dtheta_lr, float* dx_out,
                             void* stream) {
  static const char* fn = "ttt_lr_gate_bwd";
  if (x_dtype != TTT_F32 && x_dtype != TTT_BF16)
    return fail(TTT_ERR_DTYPE, "%s: unknown x dtype %d", fn, (int)x_dtype);
  if (B < 0 || T < 0 || H < 0 || dx < 0)
    return fail(TTT_ERR_SHAPE, "%s: negative size (B=%d T=%d H=%d dx=%d)", fn, B, T, H, dx);
  if (dx == 0 || dx % 32 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "%s: dx=%d unsupported (need a positive multiple of 32)", fn, dx);
  if (x_dtype != TTT_BF16) return fail(TTT_ERR_UNSUPPORTED, "%s: only bf16 x is supported", fn);
  if (!(eta_base == eta_base) || eta_base > 3.4e38f || eta_base < -3.4e38f)
    return fail(TTT_ERR_VALUE, "%s: eta_base=%g must be finite", fn, (double)eta_base);
  const int64_t ntok = (int64_t)B * T;
  if (ntok * H >= ((int64_t)1 << 30) || ntok * dx >= ((int64_t)1 << 31))
    return fail(TTT_ERR_SHAPE, "%s: B*T*H exceeds 2^30 - 1 or B*T*dx exceeds 2^31 - 1", fn);
  const Range in[] = {rng("x", x, ntok * dx * 2), rng("theta_lr", theta_lr, (int64_t)H * dx * 4),
                      rng("eta", eta, ntok * H * 4), rng("deta", deta, ntok * H * 4)};
  const Range out[] = {rng("dtheta_lr", dtheta_lr, (int64_t)H * dx * 4),
                       rng("dx", dx_out, ntok * dx * 4)};
  const bool need[] = {ntok > 0, H > 0, ntok * H > 0, ntok * H > 0};
  for (int i = 0; i < 4; ++i) {
    if (!need[i]) continue;
    if (!in[i].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, in[i].name);
    if (in[i].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, in[i].name);
  }
  const bool needo[] = {H > 0, ntok > 0};
  for (int o = 0; o < 2; ++o) {
    if (!needo[o]) continue;
    if (!out[o].lo) return fail(TTT_ERR_NULL, "%s: %s is NULL", fn, out[o].name);
    if (out[o].lo & 15) return fail(TTT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, out[o].name);
    for (int i = 0; i < 4; ++i)
      if (overlap(out[o], in[i]))
        return fail(TTT_ERR_ALIAS, "%s: %s overlaps input %s", fn, out[o].name, in[i].name);
  }
  if (overlap(out[0], out[1])) return fail(TTT_ERR_ALIAS, "%s: dtheta_lr and dx overlap", fn);
  if ((int64_t)H * dx == 0 && ntok * dx == 0) return TTT_OK;
  ttt::GateBwdArgs a{x, theta_lr, eta, deta, dtheta_lr, dx_out, eta_base, B, T, H, dx};
  hipError_t e = ttt::launch_lr_gate_bwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return TTT_OK;
}

ttt_status_t ttt_linear_gated_fwd(const void* q, const void* k, const void* v, const void* x,
                                  const float* theta_lr, float eta_base, int32_t dx,
                                  const float* w0, int32_t w0_per_batch, int32_t B, int32_t H,
                                  int32_t T, int32_t d, int32_t b, ttt_dtype_t qkv_dtype,
                                  float* eta, float* z, float* w_out, void* stream) {
  static const char* fn = "ttt_linear_gated_fwd";
  ttt_status_t st = gate_check(fn, x, TTT_BF16, theta_lr, eta_base, B, T, H, dx, eta);
  if (st == TTT_OK)
    st = linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     0, nullptr, fn, true);
  if (st != TTT_OK) return st;
  const int64_t units = (int64_t)B * H, es = qkv_dtype == TTT_F32 ? 4 : 2, seq = units * T * d;
  const Range scan[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                        rng("w0", w0, (w0_per_batch ? units : (int64_t)H) * d * d * 4),
                        rng("z", z, seq * 4), rng("w_out", w_out, units * d * d * 4)};
  st = gate_scan_alias(fn, x, theta_lr, eta, B, T, H, dx, scan, 6, 4);
  if (st != TTT_OK) return st;
  st = gate_launch(fn, x, theta_lr, eta_base, B, T, H, dx, eta, stream);
  if (st != TTT_OK) return st;
  return linear_impl(q, k, v, eta, w0, w0_per_batch, B, H, T, d, b, qkv_dtype, z, w_out, stream,
                     0, nullptr, fn);
}

ttt_status_t ttt_mlp_gated_fwd(const void* q, const void* k, const void* v, const void* x,
                               const float* theta_lr, float eta_base, int32_t dx,
                               const float* w1_0, const float* w2_0, int32_t w0_per_batch,
                               int32_t B, int32_t H, int32_t T, int32_t d, int32_t hidden,
                               int32_t b, ttt_dtype_t qkv_dtype, float* eta, float* z,
                               float* w1_out, float* w2_out, void* stream) {
  static const char* fn = "ttt_mlp_gated_fwd";
  ttt_status_t st = gate_check(fn, x, TTT_BF16, theta_lr, eta_base, B, T, H, dx, eta);
  if (st == TTT_OK)
    st = mlp_impl(q, k, v, eta, w1_0, w2_0, w0_per_batch, B, H, T, d, hidden, b, qkv_dtype, z,
                  w1_out, w2_out, stream, fn, true);
  if (st != TTT_OK) return st;
  const int64_t units = (int64_t)B * H, es = qkv_dtype == TTT_F32 ? 4 : 2, seq = units * T * d;
  const int64_t wn = (w0_per_batch ? units : (int64_t)H) * hidden * d * 4;
  const Range scan[] = {rng("q", q, seq * es), rng("k", k, seq * es), rng("v", v, seq * es),
                        rng("w1_0", w1_0, wn), rng("w2_0", w2_0, wn), rng("z", z, seq * 4),
                        rng("w1_out", w1_out, units * hidden * d * 4),
                        rng("w2_out", w2_out, units * hidden * d * 4)};
  st = gate_scan_alias(fn, x, theta_lr, eta, B, T, H, dx, scan, 8, 5);
  if (st != TTT_OK) return st;
  st = gate_launch(fn, x, theta_lr, eta_base, B, T, H, dx, eta, stream);
  if (st != TTT_OK) return st;
  return mlp_impl(q, k, v, eta, w1_0, w2_0, w0_per_batch, B, H, T, d, hidden, b, qkv_dtype, z,
                  w1_out, w2_out, stream, fn);
}

const char* ttt_status_str(ttt_status_t s) {
  switch (s) {
    case TTT_OK: return "TTT_OK";
    case TTT_ERR_NULL: return "TTT_ERR_NULL: a required pointer is NULL";
    case TTT_ERR_SHAPE: return "TTT_ERR_SHAPE: invalid sizes";
    case TTT_ERR_DTYPE: return "TTT_ERR_DTYPE: unknown dtype";
    case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED: configuration not supported";
    case TTT_ERR_ALIAS: return "TTT_ERR_ALIAS: an output overlaps an input";
    case TTT_ERR_HIP: return "TTT_ERR_HIP: HIP runtime error";
    case TTT_ERR_ALIGN: return "TTT_ERR_ALIGN: pointer not 16-byte aligned";
    case TTT_ERR_VALUE: return "TTT_ERR_VALUE: scalar argument out of range";
    case TTT_STATUS_MAX_ENUM: break;
  }
  return "unknown ttt_status_t";
}

const char* ttt_last_error(void) { return g_last_error.c_str(); }

int32_t ttt_abi_version(void) { return TTT_ABI_VERSION; }

}  // extern "C"
