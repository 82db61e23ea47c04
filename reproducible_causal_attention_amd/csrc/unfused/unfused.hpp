// unfused.hpp -- internal launchers of the unfused attention baseline.
#pragma once

#include "../cdna4.hpp"

namespace rca {
namespace unf {

// Rows are the B*Hq*T rows of [B, Hq, T, T] matrices; row (b, h, i) starts at
// element ((b*Hq + h)*T + i)*T.  scale_log2 = scale * log2(e).
template <class E>
hipError_t softmax_lse(const float* s, void* p, float* lse, long long n_rows, int T,
                       float scale_log2, int causal, hipStream_t st);
template <class E>
hipError_t probs_from_lse(const float* s, const float* lse, void* p, long long n_rows, int T,
                          float scale_log2, int causal, hipStream_t st);
template <class E>
hipError_t softmax_bwd(const void* p, const float* dp, void* ds, long long n_rows, int T,
                       int causal, hipStream_t st);
// out[b][t][h][:] = in[b][t][h / G][:] for the Hq = Hkv*G query heads; D % 8 == 0.
hipError_t repeat_kv(const void* in, void* out, int B, int T, int Hkv, int G, int D,
                     hipStream_t st);

// out[b][j][g][d] = sum over r < G, in order, of in[b][g*G + r][j][d]; D % 4 == 0.
template <class E>
hipError_t group_sum(const float* in, void* out, int B, int T, int Hkv, int G, int D,
                     hipStream_t st);

}  // namespace unf
}  // namespace rca
