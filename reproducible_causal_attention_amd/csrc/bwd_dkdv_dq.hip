// bwd_dkdv_dq.hip -- dK/dV (a3) and dQ (a4) co-launched in one grid.
//
// After the preprocess the two backward kernels are independent, so one grid
// runs the units of both: first the dQ units, heaviest query tiles first, then
// the dK/dV units.  Under the causal mask the dQ units vary in length while the
// dK/dV units (pairs of key blocks) are all equal; a CU that finishes a short
// dQ tile takes a dK/dV unit next instead of idling until a separate dK/dV
// launch, which matters when the grids are only a few units per CU.  Every
// unit computes exactly what it computes in its own kernel (same code, same
// order), so the results are bitwise those of the two separate launches.
#include "dkdv_body.hpp"
#include "dq_body.hpp"

namespace rca {
namespace {

constexpr int kThreads = dkdv::NTHREADS;
// Unit order of the grid: the dQ units heaviest first, then the dK/dV units (all
// of equal length under the causal pairing); or, with kDkdvFirst, the dK/dV
// units first (the longest-first order, measured 1 us slower at 4 x 1024).
constexpr bool kDkdvFirst = false;
static_assert(dqb::NTHREADS == kThreads, "both bodies run 512-thread workgroups");
template <int kD>
constexpr int smem_bytes() {
  return dkdv::Dims<kD>::SMEM_BYTES > dqb::Dims<kD>::SMEM_BYTES ? dkdv::Dims<kD>::SMEM_BYTES
                                                                : dqb::Dims<kD>::SMEM_BYTES;
}

// Workgroup i < n_first runs unit i of the first kind; n_first <= i < second_base
// exit at once (padding, so that every unit of the second kind keeps the XCD,
// i % 8, it has in its own grid); then unit i - second_base of the second kind.
// kRope: q and k are the rotated q', k' and dq, dk are mapped back through the
// rotations in the epilogues (tables rcos, rsin).
template <class E, bool kRope, int kD>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv,
    float scale, float scale_log2, int causal, int n_dq, int n_kv, int second_base) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<kD>()];
  const int i = blockIdx.x;
  if (kDkdvFirst) {
    if (i < n_kv) {
      dkdv::unit_body<E, kRope, kD>(smem, i, q, k, v, dO, lse, delta, rcos, rsin, dk, dv, B, T, Hq,
                                    Hkv, scale, scale_log2, causal);
    } else if (i >= second_base) {
      dqb::unit_body<E, kRope, kD>(smem, i - second_base, q, k, v, dO, lse, delta, rcos, rsin, dq,
                                   B, T, Hq, Hkv, scale, scale_log2, causal);
    }
  } else {
    if (i < n_dq) {
      dqb::unit_body<E, kRope, kD>(smem, i, q, k, v, dO, lse, delta, rcos, rsin, dq, B, T, Hq, Hkv,
                                   scale, scale_log2, causal);
    } else if (i >= second_base) {
      dkdv::unit_body<E, kRope, kD>(smem, i - second_base, q, k, v, dO, lse, delta, rcos, rsin, dk,
                                    dv, B, T, Hq, Hkv, scale, scale_log2, causal);
    }
  }
}

}  // namespace

template <class E, bool kRope>
hipError_t launch_bwd_dkdv_dq_e(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta,
                                const float* rcos, const float* rsin, void* dq, void* dk, void* dv,
                                hipStream_t s) {
  const int n_dq = ((p.T + dqb::BM - 1) / dqb::BM) * p.B * p.Hq;
  const int nkb = (p.T + 31) / 32;
  const int n_kv = (nkb + 1) / 2 * p.B * p.Hkv;
  // The second kind's units start at a multiple of 8, so each keeps the XCD
  // (block % 8) it has in its own grid.
  const int n_first = kDkdvFirst ? n_kv : n_dq;
  const int second_base = (n_first + 7) / 8 * 8;
  const dim3 grid((unsigned)(second_base + (kDkdvFirst ? n_dq : n_kv)));
  auto kernel = p.D == 128 ? attn_bwd_dkdv_dq_kernel<E, kRope, 128> : attn_bwd_dkdv_dq_kernel<E, kRope, 64>;
  kernel<<<grid, kThreads, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta, rcos, rsin,
      static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), p.B,
      p.T, p.Hq, p.Hkv, p.scale, p.scale_log2, p.causal, n_dq, n_kv, second_base);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                   const void* dO, const float* lse, const float* delta, void* dq,
                                   void* dk, void* dv, hipStream_t s) {
  return launch_bwd_dkdv_dq_e<Bf16, false>(p, q, k, v, dO, lse, delta, nullptr, nullptr, dq, dk, dv, s);
}

hipError_t launch_bwd_dkdv_dq_f16(const Problem& p, const void* q, const void* k, const void* v,
                                  const void* dO, const float* lse, const float* delta, void* dq,
                                  void* dk, void* dv, hipStream_t s) {
  return launch_bwd_dkdv_dq_e<F16, false>(p, q, k, v, dO, lse, delta, nullptr, nullptr, dq, dk, dv, s);
}

hipError_t launch_bwd_dkdv_dq_rope_bf16(const Problem& p, const void* q_rot, const void* k_rot,
                                        const void* v, const void* dO, const float* lse,
                                        const float* delta, const float* rcos, const float* rsin,
                                        void* dq, void* dk, void* dv, hipStream_t s) {
  return launch_bwd_dkdv_dq_e<Bf16, true>(p, q_rot, k_rot, v, dO, lse, delta, rcos, rsin, dq, dk, dv, s);
}

hipError_t launch_bwd_dkdv_dq_rope_f16(const Problem& p, const void* q_rot, const void* k_rot,
                                       const void* v, const void* dO, const float* lse,
                                       const float* delta, const float* rcos, const float* rsin,
                                       void* dq, void* dk, void* dv, hipStream_t s) {
  return launch_bwd_dkdv_dq_e<F16, true>(p, q_rot, k_rot, v, dO, lse, delta, rcos, rsin, dq, dk, dv, s);
}

}  // namespace rca
