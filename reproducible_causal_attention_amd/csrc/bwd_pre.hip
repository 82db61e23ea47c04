// bwd_pre.hip -- backward preprocess of fused causal attention (bf16):
// delta_i = <dO_i, o_i> for every (batch, query head, row), accumulated in fp32.
//
// This is the row term of the softmax backward, dS = P * (dP - delta), that the
// unfused causal_softmax_bwd kernel of "Training a 100M transformer in pure
// Rust: RustingBrain vs PyTorch and TensorFlow" (section "Step 1: measure before
// changing anything") needs.  It reads o and dO once and writes one float per
// row: HBM-bound.  Eight lanes share one 64-wide row (16 bytes each, whole rows
// per wave instruction) and combine their partial dot products with a fixed
// butterfly, so the result is reproducible.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int PRE_THREADS = 256;
constexpr int PRE_ROWS = PRE_THREADS / 8;  // 8 lanes x 8 elements per 64-wide row

template <class E>
__global__ __launch_bounds__(PRE_THREADS) void attn_bwd_pre_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO, float* __restrict__ delta,
    int T, int Hq, long long n_rows) {
  const long long row = (long long)blockIdx.x * PRE_ROWS + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  if (row < n_rows) {
    const u32x4_t a = gload16(o + row * kHeadDim + part * 8);
    const u32x4_t c = gload16(dO + row * kHeadDim + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(E::lo(a[i]), E::lo(c[i]), acc);
      acc = fmaf(E::hi(a[i]), E::hi(c[i]), acc);
    }
  }
  // Fixed butterfly over the 8 lanes of the row.
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < n_rows && part == 0) {
    // row enumerates [b][t][h]; delta is [b][h][t].
    const long long bt = row / Hq;
    const int h = (int)(row - bt * Hq);
    const long long b = bt / T;
    const int t = (int)(bt - b * T);
    delta[(b * Hq + h) * T + t] = acc;
  }
}

}  // namespace

template <class E>
hipError_t launch_bwd_pre_e(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s) {
  const long long n_rows = (long long)p.B * p.T * p.Hq;
  const dim3 grid((unsigned)((n_rows + PRE_ROWS - 1) / PRE_ROWS));
  attn_bwd_pre_kernel<E><<<grid, PRE_THREADS, 0, s>>>(
      static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), delta, p.T, p.Hq, n_rows);
  return hipGetLastError();
}

hipError_t launch_bwd_pre_bf16(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s) {
  return launch_bwd_pre_e<Bf16>(p, o, dO, delta, s);
}

hipError_t launch_bwd_pre_f16(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s) {
  return launch_bwd_pre_e<F16>(p, o, dO, delta, s);
}

}  // namespace rca
