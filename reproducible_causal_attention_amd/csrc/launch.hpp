// launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/attn.h"

namespace rca {

constexpr int kHeadDim = 64;  // every dtype; the 16-bit kernels also take 128

// Everything a kernel launch needs; pointers are device pointers already
// validated by the C ABI layer (contiguous, 16-byte aligned, non-overlapping).
struct Problem {
  int B, T, Hq, Hkv;
  int D;             // head dimension: 64, or 128 for the 16-bit kernels
  float scale;       // softmax scale applied to q.k
  float scale_log2;  // scale * log2(e): scores are kept in base-2 units on the GPU
  int causal;
};

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, hipStream_t s);
hipError_t launch_fwd_f16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, hipStream_t s);
// The 64-wide forward (fwd64.hip), used by the two above for D = 64.
hipError_t launch_fwd64_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                             float* lse, hipStream_t s);
hipError_t launch_fwd64_f16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                            float* lse, hipStream_t s);
hipError_t launch_bwd_pre_bf16(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s);
hipError_t launch_bwd_pre_f16(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s);
hipError_t launch_bwd_dkdv_f16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s);
hipError_t launch_bwd_dq_f16(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s);
// dK/dV and dQ in one grid; bitwise the two launches above.
hipError_t launch_bwd_dkdv_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                   const void* dO, const float* lse, const float* delta, void* dq,
                                   void* dk, void* dv, hipStream_t s);
hipError_t launch_bwd_dkdv_dq_f16(const Problem& p, const void* q, const void* k, const void* v,
                                   const void* dO, const float* lse, const float* delta, void* dq,
                                   void* dk, void* dv, hipStream_t s);

hipError_t launch_fwd_f32(const Problem& p, const void* q, const void* k, const void* v, void* o,
                          float* lse, hipStream_t s);
hipError_t launch_bwd_pre_f32(const Problem& p, const void* o, const void* dO, float* delta,
                              hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const Problem& p, const void* q, const void* k, const void* v,
                               const void* dO, const float* lse, const float* delta, void* dk,
                               void* dv, hipStream_t s);
hipError_t launch_bwd_dq_f32(const Problem& p, const void* q, const void* k, const void* v,
                             const void* dO, const float* lse, const float* delta, void* dq,
                             hipStream_t s);

// Rotary embedding (16-bit types; tables rcos, rsin: [T, D/2] float32).  The
// forward rotates q and k as it loads them; the backward's preparation writes
// delta and the rotated q', k' (q_rot, k_rot), then the co-launched dK/dV + dQ
// grid runs on q', k' and maps dq, dk back through the rotations.
hipError_t launch_fwd_rope_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* rcos, const float* rsin, void* o, float* lse,
                                hipStream_t s);
hipError_t launch_fwd_rope_f16(const Problem& p, const void* q, const void* k, const void* v,
                               const float* rcos, const float* rsin, void* o, float* lse,
                               hipStream_t s);
hipError_t launch_bwd_rope_prep_bf16(const Problem& p, const void* o, const void* dO, const void* q,
                                     const void* k, const float* rcos, const float* rsin,
                                     float* delta, void* q_rot, void* k_rot, hipStream_t s);
hipError_t launch_bwd_rope_prep_f16(const Problem& p, const void* o, const void* dO, const void* q,
                                    const void* k, const float* rcos, const float* rsin,
                                    float* delta, void* q_rot, void* k_rot, hipStream_t s);
hipError_t launch_bwd_dkdv_dq_rope_bf16(const Problem& p, const void* q_rot, const void* k_rot,
                                        const void* v, const void* dO, const float* lse,
                                        const float* delta, const float* rcos, const float* rsin,
                                        void* dq, void* dk, void* dv, hipStream_t s);
hipError_t launch_bwd_dkdv_dq_rope_f16(const Problem& p, const void* q_rot, const void* k_rot,
                                       const void* v, const void* dO, const float* lse,
                                       const float* delta, const float* rcos, const float* rsin,
                                       void* dq, void* dk, void* dv, hipStream_t s);

// attn_bwd in two parts (attn_api.hip): its argument checks other than the
// workspace's (ws, if not null, must not overlap an output), and its launches
// with delta in the given device buffer of attn_bwd_workspace_bytes() bytes.
attn_status_t check_bwd_args(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             int B, int T, int Hq, int Hkv, int D, float scale, int causal,
                             attn_dtype_t dtype, const void* ws, size_t ws_bytes);
attn_status_t enqueue_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                          int T, int Hq, int Hkv, int D, float scale, int causal,
                          attn_dtype_t dtype, float* delta, void* stream);

// Tile constants of each kernel family, reported by attn_build_info().
const char* fwd_bf16_tiles();
const char* fwd64_tiles();
const char* bwd_dkdv_tiles();
const char* bwd_dq_tiles();
const char* f32_tiles();

}  // namespace rca
