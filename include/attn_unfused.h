/*
 * attn_unfused.h -- C ABI of the unfused attention baseline (libattn_unfused.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The same operation as attn.h (its definitions, layouts, dtypes and status
 * codes apply), computed the way "Training a 100M transformer in pure Rust:
 * RustingBrain vs PyTorch and TensorFlow" computed it before fusion (section
 * "Step 1: measure before changing anything"): the [T, T] score matrix of every
 * (batch, query head) is materialised in HBM as float32 by a library GEMM and
 * read back by three softmax kernels, causal_softmax_lse (forward),
 * causal_probs_from_lse and causal_softmax_bwd (backward), around further GEMMs.
 * It exists to measure what the fused library saves on this GPU; it is not the
 * hot path.
 *
 *   forward:  S = q k^T (GEMM, float32 [T, T]);  softmax_lse: P = exp(scale S - lse)
 *             in the input dtype and lse;  o = P v (GEMM).
 *   backward: S = q k^T again;  probs_from_lse: P from S and lse;  dP = dO v^T
 *             (GEMM, float32);  softmax_bwd: dS = P (dP - sum_j P dP) in the input
 *             dtype;  per query head P^T dO and scale dS^T q (GEMMs, float32),
 *             summed over each KV group's heads in a fixed order and rounded to
 *             dv and dk;  dq = scale dS k (GEMM).
 * With causal = 1 the row kernels read only the visible part of each row and
 * write zeros past it; the GEMMs run over the whole matrix.
 *
 * GEMMs are rocBLAS strided-batched GEMMs over the query heads of each batch
 * element (k and v first repeated to the query heads; inputs in the 16-bit
 * type, float32 accumulation) with atomics disallowed, so the results are
 * bitwise run-to-run reproducible on one device like the fused library's; every
 * reduction in the library's own kernels has a fixed order.
 *
 * Unlike libattn.so this library holds state: a context owns a rocBLAS handle
 * (which allocates device memory of its own).  A context may be used by one
 * host thread at a time.  Every other buffer, including the workspace holding
 * the [T, T] matrices, is caller-owned device memory.  Only ATTN_BF16 and
 * ATTN_F16 are supported; D must be a multiple of 8 and at most 256.
 */
#ifndef REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_UNFUSED_H
#define REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_UNFUSED_H

#include <stddef.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_unfused_ctx attn_unfused_ctx;

/* Create a context on the current HIP device (creates its rocBLAS handle).
 * ATTN_ERR_INVALID_ARG for a null ctx; ATTN_ERR_HIP if rocBLAS fails. */
attn_status_t attn_unfused_create(attn_unfused_ctx** ctx);

/* Destroy a context; NULL is ignored.  Work it enqueued must be complete. */
void attn_unfused_destroy(attn_unfused_ctx* ctx);

/* Workspace bytes for attn_unfused_fwd and attn_unfused_bwd: float32 S / dP and
 * 16-bit P and dS, each [B, Hq, T, T]; float32 per-query-head dk and dv partials,
 * each [B, Hq, T, D]; then k and v repeated to the query heads, 16-bit
 * [B, T, Hq, D] each; each part rounded up to 256 bytes.  0 for invalid sizes. */
size_t attn_unfused_workspace_bytes(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype);

/* Forward: o and lse as attn_fwd.  The workspace is clobbered. */
attn_status_t attn_unfused_fwd(attn_unfused_ctx* ctx, const void* q, const void* k, const void* v,
                               void* o, float* lse, int B, int T, int Hq, int Hkv, int D,
                               float scale, int causal, attn_dtype_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Backward: dq, dk, dv as attn_bwd, from lse of either forward (o is not read:
 * the row term is sum_j P dP).  The workspace is clobbered. */
attn_status_t attn_unfused_bwd(attn_unfused_ctx* ctx, const void* q, const void* k, const void* v,
                               const float* lse, const void* dO, void* dq, void* dk, void* dv,
                               int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                               attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/* The three row kernels alone, over n_rows = B*Hq*T rows of [B, Hq, T, T]
 * matrices (row (b, h, i) starts at element ((b*Hq + h)*T + i)*T; its query
 * index is i = row % T).  s, dp: float32; p, ds: the 16-bit dtype; lse: float32
 * per row (natural log).  For timing and tests; the entry points above call
 * the same launchers. */
attn_status_t attn_unfused_softmax_lse(const float* s, void* p, float* lse, long long n_rows, int T,
                                       float scale, int causal, attn_dtype_t dtype, void* stream);
attn_status_t attn_unfused_probs_from_lse(const float* s, const float* lse, void* p,
                                          long long n_rows, int T, float scale, int causal,
                                          attn_dtype_t dtype, void* stream);
attn_status_t attn_unfused_softmax_bwd(const void* p, const float* dp, void* ds, long long n_rows,
                                       int T, int causal, attn_dtype_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_UNFUSED_H */
