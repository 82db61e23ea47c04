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
template <class E>
hipError_t convert(const float* x, void* y, long long n, hipStream_t st);

}  // namespace unf
}  // namespace rca
