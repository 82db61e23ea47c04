// attn_api.hip -- the exported C ABI (include/attn.h): host-side validation,
// workspace sizing and kernel launches.  Validation runs entirely on the host
// and touches no HIP API, so every error path can be exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include <string>

#include "../../include/attn.h"
#include "launch.hpp"
#include "validate.hpp"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

#ifndef ATTN_GIT_REV
#define ATTN_GIT_REV "unknown"
#endif

namespace {

using namespace rca::validate;

constexpr long long kMaxT = 1LL << 24;
constexpr long long kMaxTiles = 1LL << 23;     // ceil(T/64) * B * Hq
constexpr long long kMaxElements = 1LL << 40;  // per tensor
constexpr long long kMaxBatchBytes = 1LL << 31; // one batch element of any tensor (buffer offsets are 32-bit)

#define ATTN_TRY(expr)                       \
  do {                                       \
    const attn_status_t st_ = (expr);        \
    if (st_ != ATTN_OK) return st_;          \
  } while (0)

// Sizes, shared by every entry point (Hkv = Hq where no KV tensor is involved).
attn_status_t check_sizes(int B, int T, int Hq, int Hkv, int D) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (T > kMaxT) return ATTN_ERR_INVALID_ARG;
  const long long tiles = ((long long)T + 63) / 64 * (long long)B * (long long)Hq;
  if (tiles >= kMaxTiles) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * T * Hq * (long long)D >= kMaxElements) return ATTN_ERR_INVALID_ARG;
  if ((long long)T * Hq * (long long)D * 4 >= kMaxBatchBytes) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// What the kernels implement: head dim 64 for every dtype, 128 for the 16-bit ones.
// Checked after the argument checks, so an invalid call is reported as such.
attn_status_t check_supported(int D, attn_dtype_t dtype) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  if (D != rca::kHeadDim && !(D == 128 && dtype != ATTN_F32)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t check_shape(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype) {
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  return check_supported(D, dtype);
}

rca::Problem make_problem(int B, int T, int Hq, int Hkv, float scale, int causal, int D) {
  rca::Problem p;
  p.D = D;
  p.B = B;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.causal = causal;
  return p;
}

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// hipGetLastError() returns the last error of any runtime call on this thread.
// Called once before an entry point's launches, it discards an error left by an
// earlier, unrelated call (which that call already returned to its caller), so
// the status after the launch is the launch's own.
void discard_stale_error() { (void)hipGetLastError(); }

// The rotary variants run in the 16-bit types only.
attn_status_t check_rope_dtype(attn_dtype_t dtype) {
  return dtype == ATTN_BF16 || dtype == ATTN_F16 ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}


}  // namespace

ATTN_EXPORT attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                                   attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, o, lse}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)B * T * Hq * D * es, kb = (size_t)B * T * Hkv * D * es;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb)},
                          {span_of(o, qb), span_of(lse, lb)}));
  ATTN_TRY(check_supported(D, dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16  ? rca::launch_fwd_bf16(p, q, k, v, o, lse, s)
                  : dtype == ATTN_F16 ? rca::launch_fwd_f16(p, q, k, v, o, lse, s)
                                      : rca::launch_fwd_f32(p, q, k, v, o, lse, s));
}

ATTN_EXPORT size_t attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype) {
  if (check_shape(B, T, Hq, Hkv, D, dtype) != ATTN_OK) return 0;
  return round256((size_t)B * Hq * T * sizeof(float));
}

ATTN_EXPORT attn_status_t attn_bwd_preprocess(const void* o, const void* dO, float* delta, int B,
                                              int T, int Hq, int D, attn_dtype_t dtype,
                                              void* stream) {
  ATTN_TRY(check_ptrs({o, dO, delta}));
  ATTN_TRY(check_sizes(B, T, Hq, Hq, D));
  const size_t qb = (size_t)B * T * Hq * D * elem_size(dtype);
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(o, qb), span_of(dO, qb)}, {span_of(delta, lb)}));
  ATTN_TRY(check_supported(D, dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hq, 1.0f, 1, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16  ? rca::launch_bwd_pre_bf16(p, o, dO, delta, s)
                  : dtype == ATTN_F16 ? rca::launch_bwd_pre_f16(p, o, dO, delta, s)
                                      : rca::launch_bwd_pre_f32(p, o, dO, delta, s));
}

ATTN_EXPORT attn_status_t attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                                        const float* lse, const float* delta, void* dk, void* dv,
                                        int B, int T, int Hq, int Hkv, int D, float scale,
                                        int causal, attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, dO, lse, delta, dk, dv}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)B * T * Hq * D * es, kb = (size_t)B * T * Hkv * D * es;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(dO, qb),
                           span_of(lse, lb), span_of(delta, lb)},
                          {span_of(dk, kb), span_of(dv, kb)}));
  ATTN_TRY(check_supported(D, dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16  ? rca::launch_bwd_dkdv_bf16(p, q, k, v, dO, lse, delta, dk, dv, s)
                  : dtype == ATTN_F16 ? rca::launch_bwd_dkdv_f16(p, q, k, v, dO, lse, delta, dk, dv, s)
                                      : rca::launch_bwd_dkdv_f32(p, q, k, v, dO, lse, delta, dk, dv, s));
}

ATTN_EXPORT attn_status_t attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                                      const float* lse, const float* delta, void* dq, int B, int T,
                                      int Hq, int Hkv, int D, float scale, int causal,
                                      attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, dO, lse, delta, dq}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)B * T * Hq * D * es, kb = (size_t)B * T * Hkv * D * es;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(dO, qb),
                           span_of(lse, lb), span_of(delta, lb)},
                          {span_of(dq, qb)}));
  ATTN_TRY(check_supported(D, dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16  ? rca::launch_bwd_dq_bf16(p, q, k, v, dO, lse, delta, dq, s)
                  : dtype == ATTN_F16 ? rca::launch_bwd_dq_f16(p, q, k, v, dO, lse, delta, dq, s)
                                      : rca::launch_bwd_dq_f32(p, q, k, v, dO, lse, delta, dq, s));
}

namespace rca {

// Every check of attn_bwd except those of the workspace: pointers, sizes,
// scalars, overlap of the outputs with the inputs and each other (and with
// [ws, ws + ws_bytes) when ws is not null), then the supported shapes.
attn_status_t check_bwd_args(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                             attn_dtype_t dtype, const void* ws, size_t ws_bytes) {
  ATTN_TRY(check_ptrs({q, k, v, o, lse, dO, dq, dk, dv}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)B * T * Hq * D * es, kb = (size_t)B * T * Hkv * D * es;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(o, qb),
                           span_of(lse, lb), span_of(dO, qb)},
                          {span_of(dq, qb), span_of(dk, kb), span_of(dv, kb),
                           span_of(ws, ws ? ws_bytes : 0)}));
  return check_supported(D, dtype);
}

// The launches of attn_bwd on checked arguments: the preprocess writes delta,
// then the co-launched dK/dV + dQ grid (float32: the two separate kernels).
attn_status_t enqueue_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                          int T, int Hq, int Hkv, int D, float scale, int causal,
                          attn_dtype_t dtype, float* delta, void* stream) {
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16) {
    ATTN_TRY(from_hip(rca::launch_bwd_pre_bf16(p, o, dO, delta, s)));
    return from_hip(rca::launch_bwd_dkdv_dq_bf16(p, q, k, v, dO, lse, delta, dq, dk, dv, s));
  }
  if (dtype == ATTN_F16) {
    ATTN_TRY(from_hip(rca::launch_bwd_pre_f16(p, o, dO, delta, s)));
    return from_hip(rca::launch_bwd_dkdv_dq_f16(p, q, k, v, dO, lse, delta, dq, dk, dv, s));
  }
  ATTN_TRY(from_hip(rca::launch_bwd_pre_f32(p, o, dO, delta, s)));
  ATTN_TRY(from_hip(rca::launch_bwd_dkdv_f32(p, q, k, v, dO, lse, delta, dk, dv, s)));
  return from_hip(rca::launch_bwd_dq_f32(p, q, k, v, dO, lse, delta, dq, s));
}

}  // namespace rca

ATTN_EXPORT attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                                   int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                                   attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, o, lse, dO, dq, dk, dv, workspace}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t need = attn_bwd_workspace_bytes(B, T, Hq, Hkv, D, dtype);
  if (workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
  ATTN_TRY(rca::check_bwd_args(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, D, scale, causal,
                               dtype, workspace, need));
  return rca::enqueue_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, D, scale, causal, dtype,
                          static_cast<float*>(workspace), stream);
}

ATTN_EXPORT attn_status_t attn_bwd_dkdv_dq(const void* q, const void* k, const void* v,
                                           const void* dO, const float* lse, const float* delta,
                                           void* dq, void* dk, void* dv, int B, int T, int Hq,
                                           int Hkv, int D, float scale, int causal,
                                           attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, dO, lse, delta, dq, dk, dv}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)B * T * Hq * D * es, kb = (size_t)B * T * Hkv * D * es;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(dO, qb),
                           span_of(lse, lb), span_of(delta, lb)},
                          {span_of(dq, qb), span_of(dk, kb), span_of(dv, kb)}));
  ATTN_TRY(check_supported(D, dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16)
    return from_hip(rca::launch_bwd_dkdv_dq_bf16(p, q, k, v, dO, lse, delta, dq, dk, dv, s));
  if (dtype == ATTN_F16)
    return from_hip(rca::launch_bwd_dkdv_dq_f16(p, q, k, v, dO, lse, delta, dq, dk, dv, s));
  ATTN_TRY(from_hip(rca::launch_bwd_dkdv_f32(p, q, k, v, dO, lse, delta, dk, dv, s)));
  return from_hip(rca::launch_bwd_dq_f32(p, q, k, v, dO, lse, delta, dq, s));
}

ATTN_EXPORT attn_status_t attn_fwd_rope(const void* q, const void* k, const void* v,
                                        const float* rope_cos, const float* rope_sin, void* o,
                                        float* lse, int B, int T, int Hq, int Hkv, int D,
                                        float scale, int causal, attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, rope_cos, rope_sin, o, lse}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t qb = (size_t)B * T * Hq * D * 2, kb = (size_t)B * T * Hkv * D * 2;
  const size_t lb = (size_t)B * Hq * T * sizeof(float), tb = (size_t)T * (D / 2) * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(rope_cos, tb),
                           span_of(rope_sin, tb)},
                          {span_of(o, qb), span_of(lse, lb)}));
  ATTN_TRY(check_supported(D, dtype));
  ATTN_TRY(check_rope_dtype(dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16
                      ? rca::launch_fwd_rope_bf16(p, q, k, v, rope_cos, rope_sin, o, lse, s)
                      : rca::launch_fwd_rope_f16(p, q, k, v, rope_cos, rope_sin, o, lse, s));
}

ATTN_EXPORT size_t attn_bwd_rope_workspace_bytes(int B, int T, int Hq, int Hkv, int D,
                                                 attn_dtype_t dtype) {
  if (check_shape(B, T, Hq, Hkv, D, dtype) != ATTN_OK || check_rope_dtype(dtype) != ATTN_OK)
    return 0;
  return round256((size_t)B * Hq * T * sizeof(float)) + round256((size_t)B * T * Hq * D * 2) +
         round256((size_t)B * T * Hkv * D * 2);
}

ATTN_EXPORT attn_status_t attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                                        const float* lse, const void* dO, const float* rope_cos,
                                        const float* rope_sin, void* dq, void* dk, void* dv, int B,
                                        int T, int Hq, int Hkv, int D, float scale, int causal,
                                        attn_dtype_t dtype, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  ATTN_TRY(check_ptrs({q, k, v, o, lse, dO, rope_cos, rope_sin, dq, dk, dv, workspace}));
  ATTN_TRY(check_sizes(B, T, Hq, Hkv, D));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t need = attn_bwd_rope_workspace_bytes(B, T, Hq, Hkv, D, dtype);
  if (workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * T * Hq * D * 2, kb = (size_t)B * T * Hkv * D * 2;
  const size_t lb = (size_t)B * Hq * T * sizeof(float), tb = (size_t)T * (D / 2) * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(o, qb),
                           span_of(lse, lb), span_of(dO, qb), span_of(rope_cos, tb),
                           span_of(rope_sin, tb)},
                          {span_of(dq, qb), span_of(dk, kb), span_of(dv, kb),
                           span_of(workspace, need)}));
  char* ws = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws);
  void* q_rot = ws + round256(lb);
  void* k_rot = ws + round256(lb) + round256(qb);
  ATTN_TRY(check_supported(D, dtype));
  ATTN_TRY(check_rope_dtype(dtype));
  discard_stale_error();
  const rca::Problem p = make_problem(B, T, Hq, Hkv, scale, causal, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16) {
    ATTN_TRY(from_hip(rca::launch_bwd_rope_prep_bf16(p, o, dO, q, k, rope_cos, rope_sin, delta,
                                                     q_rot, k_rot, s)));
    return from_hip(rca::launch_bwd_dkdv_dq_rope_bf16(p, q_rot, k_rot, v, dO, lse, delta, rope_cos,
                                                      rope_sin, dq, dk, dv, s));
  }
  ATTN_TRY(from_hip(rca::launch_bwd_rope_prep_f16(p, o, dO, q, k, rope_cos, rope_sin, delta, q_rot,
                                                  k_rot, s)));
  return from_hip(rca::launch_bwd_dkdv_dq_rope_f16(p, q_rot, k_rot, v, dO, lse, delta, rope_cos,
                                                   rope_sin, dq, dk, dv, s));
}

ATTN_EXPORT const char* attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: unsupported head dimension or dtype";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown attn_status_t";
}

ATTN_EXPORT const char* attn_build_info(void) {
  static const std::string info = std::string("revision=") + ATTN_GIT_REV +
                                  " arch=gfx950 compiler=clang-" + __clang_version__ + " " +
                                  rca::fwd64_tiles() + " " + rca::fwd_bf16_tiles() + " " + rca::bwd_dkdv_tiles() + " " + rca::bwd_dq_tiles() + " " +
                                  rca::f32_tiles();
  return info.c_str();
}
