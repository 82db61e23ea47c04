// bwd_dq.hip -- launcher of the dQ kernel (a4); the work of one unit is in
// dq_body.hpp.
#include "dq_body.hpp"

namespace rca {
namespace {

template <class E, int kD>
__global__ __launch_bounds__(dqb::NTHREADS) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  __shared__ __attribute__((aligned(16))) char smem[dqb::Dims<kD>::SMEM_BYTES];
  dqb::unit_body<E, false, kD>(smem, 0, false, blockIdx.x, -1, q, k, v, dO, lse, delta, nullptr, nullptr, dq, B, T,
                           Hq, Hkv, scale, scale_log2, causal);
}

}  // namespace

template <class E>
hipError_t launch_bwd_dq_e(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s) {
  const int n_qt = (p.T + dqb::BM - 1) / dqb::BM;
  const dim3 grid((unsigned)(n_qt * p.B * p.Hq));
  auto kernel = p.D == 128 ? attn_bwd_dq_kernel<E, 128> : attn_bwd_dq_kernel<E, 64>;
  kernel<<<grid, dqb::NTHREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta,
      static_cast<uint16_t*>(dq), p.B, p.T, p.Hq, p.Hkv, p.scale, p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s) {
  return launch_bwd_dq_e<Bf16>(p, q, k, v, dO, lse, delta, dq, s);
}

hipError_t launch_bwd_dq_f16(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s) {
  return launch_bwd_dq_e<F16>(p, q, k, v, dO, lse, delta, dq, s);
}

const char* bwd_dq_tiles() { return "dq_bf16{BM=128,BN=128(D=64)|64(D=128),waves=8(4 query x 2 key),mfma=32x32x16,D=64|128,D=64: rows and first tile by lds_dma into 2 slots, next unit copied during the current}"; }

}  // namespace rca
