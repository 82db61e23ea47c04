// bwd_dkdv.hip -- launcher of the dK/dV kernel (a3); the work of one unit is in
// dkdv_body.hpp.
#include "dkdv_body.hpp"

namespace rca {
namespace {

template <class E, int kD, bool kSolo>
__global__ __launch_bounds__(dkdv::NTHREADS) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv,
    float scale, float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) char smem[dkdv::Dims<kD>::SMEM_BYTES];
  dkdv::run_unit<E, false, kD, kSolo>(smem, blockIdx.x, q, k, v, dO, lse, delta, nullptr, nullptr, dk, dv, B,
                               T, Hq, Hkv, scale, scale_log2, causal);
}

}  // namespace

template <class E>
hipError_t launch_bwd_dkdv_e(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s) {
  const int nkb = (p.T + 31) / 32;
  const dim3 grid((unsigned)(dkdv::units_per_group(p.Hq / p.Hkv, nkb, p.D) * p.B * p.Hkv));
  auto kernel = p.D == 128 ? attn_bwd_dkdv_kernel<E, 128, false>
                : dkdv::solo_units(p.Hq / p.Hkv, nkb, p.D) ? attn_bwd_dkdv_kernel<E, 64, true>
                                                            : attn_bwd_dkdv_kernel<E, 64, false>;
  kernel<<<grid, dkdv::NTHREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), p.B, p.T, p.Hq, p.Hkv, p.scale,
      p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s) {
  return launch_bwd_dkdv_e<Bf16>(p, q, k, v, dO, lse, delta, dk, dv, s);
}

hipError_t launch_bwd_dkdv_f16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s) {
  return launch_bwd_dkdv_e<F16>(p, q, k, v, dO, lse, delta, dk, dv, s);
}

const char* bwd_dkdv_tiles() {
  return "dkdv_bf16{key_block=32,waves=8,pairs=(j,n-1-j),query_step=32,mfma=32x32x16,lds_dma_x2,D=64|128(x1),"
         "per-wave pairs when G*(nkb+1)<=48 (D=64)}";
}

}  // namespace rca
