/*
 * ttt_tuning.h — launch-shape control and measurement helpers of libttt.so.
 *
 * Not needed for correctness: ttt_linear_fwd picks its launch shape itself.
 * These entry points exist so that benchmarks can sweep launch shapes and
 * calibrate hardware counters.  Same pointer, stream and error conventions
 * as include/ttt.h.
 */
#ifndef TTT_TUNING_H_
#define TTT_TUNING_H_

#include <stddef.h>
#include <stdint.h>

#include "ttt.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ttt_linear_fwd with an explicit launch shape: rows_per_workgroup rows of
 * each head's 64-row state per workgroup (16, 32 or 64; 0 = automatic), in
 * one pass over each sequence (no sequence chunks).
 * The rows of W evolve independently (the reconstruction loss is a sum over
 * output components, "论文速览 | TTT" §3.3), so any split gives the same
 * result bit for bit.  Other values: TTT_ERR_UNSUPPORTED.
 */
ttt_status_t ttt_linear_fwd_tuned(const void* q, const void* k, const void* v,
                                  const float* eta, const float* w0,
                                  int32_t w0_per_batch, int32_t B, int32_t H,
                                  int32_t T, int32_t d, int32_t b,
                                  ttt_dtype_t qkv_dtype, float* z,
                                  float* w_out, void* stream,
                                  int32_t rows_per_workgroup);

/*
 * ttt_linear_fwd_tuned with the depth of the LDS prefetch ring of the bf16
 * scan set: ring_depth = 0 is the default (about ten 16-token tiles in flight
 * ahead of the two being worked on), 1 keeps a single one.  The ring only
 * changes when tiles land, never what is computed, so results are
 * bit-identical for every depth; it exists to check that (a shallow ring
 * would expose a missing wait as a wrong result).  ring_depth = 1 needs bf16
 * q/k/v and b = 16 (one pass); other values are TTT_ERR_UNSUPPORTED.
 */
ttt_status_t ttt_linear_fwd_ring_depth(const void* q, const void* k,
                                       const void* v, const float* eta,
                                       const float* w0, int32_t w0_per_batch,
                                       int32_t B, int32_t H, int32_t T,
                                       int32_t d, int32_t b,
                                       ttt_dtype_t qkv_dtype, float* z,
                                       float* w_out, void* stream,
                                       int32_t rows_per_workgroup,
                                       int32_t ring_depth);

/*
 * ttt_linear_fwd with explicit sequence chunks (see "Sequence chunks" at
 * ttt_linear_fwd): seq_chunks = 0 picks as ttt_linear_fwd does, 1 runs one
 * pass, P >= 2 cuts each sequence into P chunks, which needs bf16 q/k/v,
 * b = 16 and T / P a multiple of 16 and at least 192 (else
 * TTT_ERR_UNSUPPORTED; negative values too).  rows_per_workgroup as in
 * ttt_linear_fwd_tuned, for every pass.
 */
ttt_status_t ttt_linear_fwd_chunked(const void* q, const void* k,
                                    const void* v, const float* eta,
                                    const float* w0, int32_t w0_per_batch,
                                    int32_t B, int32_t H, int32_t T,
                                    int32_t d, int32_t b,
                                    ttt_dtype_t qkv_dtype, float* z,
                                    float* w_out, void* stream,
                                    int32_t rows_per_workgroup,
                                    int32_t seq_chunks);

/*
 * ttt_linear_bwd with an explicit sequence-chunk count (see "Sequence
 * chunks" at ttt_linear_bwd): seq_chunks = 0 picks as ttt_linear_bwd does
 * (the count ttt_linear_fwd_plan reports), 1 runs one pass, P >= 2 cuts each
 * sequence into P chunks, which needs T / P a multiple of 16 and at least
 * 192 (else TTT_ERR_UNSUPPORTED; negative values too).  Arguments, results
 * and errors otherwise as ttt_linear_bwd.
 */
ttt_status_t ttt_linear_bwd_chunked(const void* q, const void* k,
                                    const void* v, const float* eta,
                                    const float* w_ckpt, int32_t B, int32_t H,
                                    int32_t T, int32_t d, int32_t b,
                                    ttt_dtype_t qkv_dtype, const float* dz,
                                    const float* dw_T, float* dq, float* dk,
                                    float* dv, float* deta, float* dw0,
                                    void* stream, int32_t seq_chunks);

/*
 * The launch plan ttt_linear_fwd picks for these sizes: rows of the state
 * per workgroup and the number of sequence chunks (1 = one pass; the
 * checkpointing forward and the backward chunk alike).  Host-only;
 * nothing is launched.  NULL outputs: TTT_ERR_NULL; negative sizes or b < 1:
 * TTT_ERR_SHAPE; unknown dtype: TTT_ERR_DTYPE.
 */
ttt_status_t ttt_linear_fwd_plan(int32_t B, int32_t H, int32_t T, int32_t b,
                                 ttt_dtype_t qkv_dtype,
                                 int32_t* rows_per_workgroup,
                                 int32_t* seq_chunks);

/*
 * ttt_lr_gate with an explicit launch shape: tokens_per_workgroup tokens per
 * workgroup (32 or 64; 0 = automatic).  Each token's sums are the same for
 * every value.  Other values: TTT_ERR_UNSUPPORTED.
 */
ttt_status_t ttt_lr_gate_tuned(const void* x, ttt_dtype_t x_dtype,
                               const float* theta_lr, float eta_base,
                               int32_t B, int32_t T, int32_t H, int32_t dx,
                               float* eta, void* stream,
                               int32_t tokens_per_workgroup);

/*
 * Plain streaming copy of `bytes` bytes (a multiple of 16, both pointers
 * 16-byte aligned, no overlap) from src to dst on `stream`: the reference
 * kernel whose hardware byte counters calibrate those of the scans.
 */
ttt_status_t ttt_bench_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TTT_TUNING_H_ */
