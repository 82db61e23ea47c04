/*
 * attn.h -- C ABI of the reproducible fused causal attention library (libattn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is causal (optionally grouped-query) scaled-dot-product
 * attention for decoder training, forward and backward, computed without ever
 * materialising the [T, T] score matrix.  "Training a 100M transformer in pure
 * Rust: RustingBrain vs PyTorch and TensorFlow" motivates it: section "Step 1:
 * measure before changing anything" finds the cost of unfused attention in the
 * [seq_len, seq_len] fp32 matrix written and read back by causal_softmax_lse,
 * causal_softmax_bwd and causal_probs_from_lse; section "Step 2: fused flash
 * attention" removes the matrix with one fused forward and backward.  Section
 * "The setup" gives the grouped-query shape (12 query heads, 4 KV heads,
 * head_dim 64).
 *
 * Definitions (per batch element b, query head h, KV head g = h / (Hq/Hkv)):
 *   s[i][j]  = scale * sum_d q[b][i][h][d] * k[b][j][g][d]; with causal=1 key j
 *              is visible to query i iff j <= i, otherwise s = -inf;
 *   lse[i]   = ln(sum_j exp(s[i][j]))                        (natural log)
 *   P[i][j]  = exp(s[i][j] - lse[i]);   o[b][i][h][:] = sum_j P[i][j] v[b][j][g][:]
 *   delta[i] = sum_d dO[b][i][h][d] * o[b][i][h][d]
 *   dS[i][j] = P[i][j] * (sum_d dO[b][i][h][d] * v[b][j][g][d] - delta[i])
 *   dq[i] = scale * sum_j dS[i][j] k[j];  dk[j] = scale * sum_{h in group} sum_i dS[i][j] q[i];
 *   dv[j] = sum_{h in group} sum_i P[i][j] dO[i].
 *
 * Head dimension D: 64 for every dtype; 128 for ATTN_BF16 and ATTN_F16 (the same
 * kernels instantiated for 128-wide rows).
 *
 * Layouts (all row-major and contiguous; there are no stride arguments):
 *   q, o, dO, dq : [B, T, Hq,  D] elements of the input dtype
 *   k, v, dk, dv : [B, T, Hkv, D] elements of the input dtype
 *   lse, delta   : [B, Hq, T]     float32
 *
 * Ownership and execution.  Every pointer is caller-owned device memory on the
 * current HIP device.  The library allocates nothing and is safe to call from
 * several host threads; its only global state is the per-GPU delta array of
 * attn_bwd_noalloc (a fixed device array, not an allocation) and the cache of
 * that array's address on each device.  Calls enqueue work on
 * `stream` (a hipStream_t; NULL is the null stream) and return without
 * waiting for it.  Outputs are overwritten, never accumulated into, so callers
 * need not clear them first.
 *
 * Reproducibility.  For one build of the library on one device, identical
 * inputs give bitwise-identical outputs, whatever the stream, the launch order
 * or concurrent work: every reduction runs in a fixed order inside one
 * workgroup and no kernel uses atomics.  ("rust-trainer", section "The trainer
 * is not bit-identical to itself after step 1", traces the loss of bit
 * identity to a gradient accumulated with atomics.)  Bits are not promised
 * across builds, tile constants or GPU models.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued; a
 * failed validation enqueues nothing.  ATTN_ERR_INVALID_ARG: a null pointer; a
 * size <= 0; Hq not a multiple of Hkv; causal not 0 or 1; scale not finite; a
 * pointer not 16-byte aligned; an output range overlapping an input range or
 * another output; a workspace smaller than attn_bwd_workspace_bytes() (or
 * attn_bwd_rope_workspace_bytes() for attn_bwd_rope); sizes
 * beyond the limits below.  ATTN_ERR_UNSUPPORTED: D other than 64 (or 128 with
 * ATTN_BF16 / ATTN_F16), an unknown dtype, or ATTN_F32 in a rotary entry point;
 * it is reported only for calls whose other arguments pass the checks above
 * (the overlap rule included).
 * ATTN_ERR_HIP: the HIP runtime reported an error for a launch (the value of
 * hipGetLastError() after the launch; an error pending from an earlier,
 * unrelated runtime call is discarded before the launch, so it is not reported
 * as this call's failure).  Nothing aborts and no C++ exception crosses the
 * interface.
 *
 * Limits: T <= 2^24; ceil(T/64)*B*Hq < 2^23; every tensor holds fewer than
 * 2^40 elements; and one batch element of q (T*Hq*D elements) spans fewer than
 * 2^31 bytes at four bytes per element.
 */
#ifndef REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_H
#define REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_HIP = 3
} attn_status_t;

typedef enum {
  ATTN_F32 = 0,  /* float32 inputs and outputs, float32 arithmetic throughout   */
  ATTN_BF16 = 1, /* bfloat16 inputs and outputs; bf16 matrix products with fp32
                    accumulation, fp32 softmax statistics, lse and delta        */
  ATTN_F16 = 2   /* float16 inputs and outputs, otherwise as ATTN_BF16 (the same
                    kernels with fp16 matrix products and conversions)           */
} attn_dtype_t;

/* Forward.  Reads q, k, v; writes o and lse (the per-row log-sum-exp that the
 * backward uses to recompute P, as causal_probs_from_lse does in "Training a
 * 100M transformer in pure Rust: RustingBrain vs PyTorch and TensorFlow",
 * section "Step 1: measure before changing anything").  o and lse must not
 * overlap the inputs or each other. */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                       attn_dtype_t dtype, void* stream);

/* Bytes of device workspace attn_bwd needs: the float32 delta rows
 * (B*Hq*T*4 bytes) rounded up to 256 bytes.  Returns 0 for invalid sizes.
 * delta is the per-row term of the softmax backward; the unfused chain of
 * "Training a 100M transformer in pure Rust: RustingBrain vs PyTorch and
 * TensorFlow", section "Step 1: measure before changing anything", forms it
 * inside causal_softmax_bwd, the fused backward of section "Step 2: fused flash
 * attention" keeps it in this buffer between its steps. */
size_t attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype);

/* Backward of sum(o * dO): the fused flash-attention backward of "Training a
 * 100M transformer in pure Rust: RustingBrain vs PyTorch and TensorFlow",
 * section "Step 2: fused flash attention" (dq, dk, dv as defined above, with P
 * recomputed from lse as that page's causal_probs_from_lse does, section "Step
 * 1: measure before changing anything").  o and lse must be the outputs of
 * attn_fwd for the same q, k, v, scale and causal.  Enqueues, in order, attn_bwd_preprocess
 * (delta into the workspace) and attn_bwd_dkdv_dq; the results are bitwise those
 * of attn_bwd_preprocess, attn_bwd_dkdv and attn_bwd_dq called in turn.  dq, dk,
 * dv must not overlap any input, the workspace or each other; the workspace must
 * hold at least attn_bwd_workspace_bytes() bytes and is clobbered. */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Size in bytes of the device array that attn_bwd_noalloc keeps per GPU for
 * its delta rows: calls with attn_bwd_workspace_bytes() above it are refused. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)

/* attn_bwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same checks,
 * launches and results (bitwise those of attn_bwd), with delta kept in an array
 * the library holds on each GPU (ATTN_NOALLOC_SCRATCH_BYTES, i.e. B*Hq*T up to
 * 4,194,304 rows) instead of a caller workspace.  It calls no hipMalloc or
 * hipFree.  The first call on a device resolves the array's address there
 * (hipGetSymbolAddress); a failure is ATTN_ERR_HIP.  ATTN_ERR_INVALID_ARG, in
 * addition to attn_bwd's cases, when attn_bwd_workspace_bytes() exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES.  All calls on one GPU share the array and its
 * contents, so calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller; calls queued on one
 * stream are ordered and safe. */
attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dO, void* dq, void* dk, void* dv,
                               int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                               attn_dtype_t dtype, void* stream);

/* Backward step 1: delta[b][h][i] = sum_d dO[b][i][h][d] * o[b][i][h][d], accumulated
 * in float32 (the row term of the softmax backward that causal_softmax_bwd needs
 * in the unfused chain of the same page, section "Step 1").  o and dO are
 * [B, T, Hq, D]; delta is [B, Hq, T] float32 and must not overlap them. */
attn_status_t attn_bwd_preprocess(const void* o, const void* dO, float* delta,
                                  int B, int T, int Hq, int D, attn_dtype_t dtype,
                                  void* stream);

/* Backward step 2: dk and dv (definitions above): the flash_attention_dkv
 * kernel of "Training a 100M transformer in pure Rust: RustingBrain vs PyTorch
 * and TensorFlow", section "Where the time goes now".  One workgroup owns a
 * tile of keys of one KV head and visits every query head of its group and
 * every query tile that can see those keys, in a fixed order, so dk and dv are
 * summed in registers and written once, with no atomics ("rust-trainer",
 * section "The trainer is not bit-identical to itself after step 1", loses bit
 * identity to an atomically accumulated gradient).  delta is the output of
 * attn_bwd_preprocess. */
attn_status_t attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* delta, void* dk, void* dv,
                            int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                            attn_dtype_t dtype, void* stream);

/* Backward step 3: dq = scale * sum_j dS[i][j] k[j] (definitions above), the
 * query-side half of the fused backward of "Training a 100M transformer in pure
 * Rust: RustingBrain vs PyTorch and TensorFlow", section "Step 2: fused flash
 * attention".  One workgroup owns a tile of queries of one query head and
 * visits the key tiles it can see in a fixed order; each dq row has one owner,
 * so there are no atomics. */
attn_status_t attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                          const float* lse, const float* delta, void* dq,
                          int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                          attn_dtype_t dtype, void* stream);

/* Backward steps 2 and 3 co-launched in one grid (they are independent once
 * delta is known; "Training a 100M transformer in pure Rust: RustingBrain vs
 * PyTorch and TensorFlow", section "Where the time goes now", names the dk/dv
 * kernel as the remaining attention hot spot, and the page's section "The
 * result" notes that per-step overheads weigh more at small batches): one
 * workgroup per CU runs a fixed list of the dQ units of
 * attn_bwd_dq (heavy query tiles paired with light ones) and then dK/dV units
 * of attn_bwd_dkdv, so no CU waits for a second launch.  dq, dk and dv are
 * bitwise those of the two separate calls, whatever the CU count.  Arguments
 * as there; dq, dk, dv must not overlap any input or each other.  Queries the
 * current device's CU count (hipDeviceGetAttribute) to size the grid. */
attn_status_t attn_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dO,
                               const float* lse, const float* delta, void* dq, void* dk, void* dv,
                               int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                               attn_dtype_t dtype, void* stream);

/* Rotary position embedding fused into the attention (ATTN_BF16 and ATTN_F16
 * only; ATTN_F32 gives ATTN_ERR_UNSUPPORTED).  "Training a 100M transformer in
 * pure Rust: RustingBrain vs PyTorch and TensorFlow", section "The setup", puts
 * rotary positions in the model without fixing a convention; the one taken is
 * the original adjacent-pair rotation: at position t, pair i = (x[2i], x[2i+1])
 * of every query and key vector becomes
 *   (x[2i] c - x[2i+1] s,  x[2i] s + x[2i+1] c),  c = rope_cos[t][i], s = rope_sin[t][i],
 * the same positions 0 .. T-1 for queries and keys; v is not rotated.
 * rope_cos and rope_sin are [T, D/2] float32 tables that the caller fills (any
 * base or scaling); they are inputs like q.  The rotated pair is rounded to the
 * input dtype before the products, as an unfused rotation that stores its
 * result would round it.
 *
 * attn_fwd_rope: attn_fwd on the rotated q', k'.  o and lse as there. */
attn_status_t attn_fwd_rope(const void* q, const void* k, const void* v, const float* rope_cos,
                            const float* rope_sin, void* o, float* lse, int B, int T, int Hq,
                            int Hkv, int D, float scale, int causal, attn_dtype_t dtype,
                            void* stream);

/* Bytes of device workspace attn_bwd_rope needs: delta (B*Hq*T float32), then
 * the rotated q' ([B, T, Hq, D]) and k' ([B, T, Hkv, D]) in the input dtype,
 * each rounded up to 256 bytes.  Returns 0 for invalid sizes or ATTN_F32. */
size_t attn_bwd_rope_workspace_bytes(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype);

/* Backward of attn_fwd_rope: dq, dk, dv with respect to the unrotated q, k and
 * v.  o and lse must be the outputs of attn_fwd_rope for the same inputs and
 * tables.  Enqueues a preparation kernel (delta, q' and k' into the workspace,
 * rotated with the same arithmetic as the forward, so the same bits) and the
 * co-launched dK/dV + dQ grid on q', k', whose epilogues map dq and dk back
 * through the transpose of each pair's rotation:
 *   (g[2i] c + g[2i+1] s,  -g[2i] s + g[2i+1] c).
 * Ownership, overlap and workspace rules as attn_bwd; the workspace must hold
 * attn_bwd_rope_workspace_bytes() bytes and is clobbered. */
attn_status_t attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dO, const float* rope_cos,
                            const float* rope_sin, void* dq, void* dk, void* dv, int B, int T,
                            int Hq, int Hkv, int D, float scale, int causal, attn_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(attn_status_t status);

/* Static string describing the compiled library: source revision, offload
 * architecture, compiler and tile constants.  Output bits are promised
 * identical only between runs of the same compiled library ("rust-trainer", section "Build once, run
 * many", prints the resolved revision of every binary it measures). */
const char* attn_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* REPRODUCIBLE_CAUSAL_ATTENTION_ATTN_H */
