// bwd_dkdv_dq.hip -- dK/dV (a3) and dQ (a4) co-launched in one grid.
//
// After the preprocess the two backward kernels are independent, so one grid
// runs the units of both.  Under the causal mask the dQ units vary in length
// while the dK/dV units (pairs of key blocks) are all equal; a fixed number of
// workgroups, one per CU, each run a balanced list of units (dQ tiles paired
// heavy with light, then dK/dV units), so that no CU idles until a separate
// dK/dV launch and the last units do not start late on CUs that drew long
// ones.  Every unit computes exactly what it computes in its own kernel (same
// code, same order), so the results are bitwise those of the two separate
// launches.  For 64-wide heads a workgroup's consecutive dQ units alternate
// between two LDS slots, and each issues the next one's row and first-tile
// copies while it computes, so that unit starts on data already in LDS.
#include "dkdv_body.hpp"
#include "dq_body.hpp"

namespace rca {
namespace {

constexpr int kThreads = dkdv::NTHREADS;
static_assert(dqb::NTHREADS == kThreads, "both bodies run 512-thread workgroups");
template <int kD>
constexpr int smem_bytes() {
  return dkdv::Dims<kD>::SMEM_BYTES > dqb::Dims<kD>::SMEM2_BYTES ? dkdv::Dims<kD>::SMEM_BYTES
                                                                 : dqb::Dims<kD>::SMEM2_BYTES;
}

// Persistent order: P workgroups (a multiple of 8, at most one per CU; workgroup
// w runs on XCD w % 8 like unit w of a plain grid).  Workgroup w = 8l + x takes,
// among the units u = x + 8m of its XCD, first the dQ units in boustrophedon
// order over m (m = l, 2Q-1-l, 2Q+l, 4Q-1-l, ... with Q = P / 8, so a heavy
// query tile is paired with a light one), then the dK/dV units m = Q-1-l,
// 2Q-1-l, ... (from the other end, so that when there are fewer units than
// workgroups the two kinds land on different workgroups).  Every unit is taken
// exactly once, and each computes exactly what it computes in its own kernel,
// so the results do not depend on P.
template <class E, bool kRope, int kD, bool kSolo>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv,
    float scale, float scale_log2, int causal, int n_dq, int n_kv, int P) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<kD>()];
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3, Q = P >> 3;
  auto dq_unit = [&](int j) {  // the j-th dQ unit of this workgroup; m grows with j
    const int m = 2 * Q * (j >> 1) + ((j & 1) ? 2 * Q - 1 - l : l);
    return x + 8 * m;
  };
  // Unit j runs in LDS slot j % 2 and issues the copies of unit j + 1 into the
  // other slot while it computes.
  for (int j = 0, u = dq_unit(0); u < n_dq; ++j) {
    const int u_next = dq_unit(j + 1);
    dqb::unit_body<E, kRope, kD>(smem, j & 1, j > 0, u, u_next < n_dq ? u_next : -1, q, k, v, dO,
                                 lse, delta, rcos, rsin, dq, B, T, Hq, Hkv, scale, scale_log2,
                                 causal);
    lds_barrier();  // the next unit reuses the LDS (its own prologue waits for its copies)
    u = u_next;
  }
  for (int u = x + 8 * (Q - 1 - l); u < n_kv; u += 8 * Q) {
    dkdv::run_unit<E, kRope, kD, kSolo>(smem, u, q, k, v, dO, lse, delta, rcos, rsin, dk, dv, B, T, Hq,
                                 Hkv, scale, scale_log2, causal);
    lds_barrier();
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
  const int n_kv = dkdv::units_per_group(p.Hq / p.Hkv, nkb, p.D) * p.B * p.Hkv;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipGetLastError();
  // One workgroup per CU (the body's registers and LDS allow no more), or one
  // per unit with a margin of two per XCD when the units are fewer.
  const int units = n_dq + n_kv + 16;
  const int P = ((n_cu < units ? n_cu : units) + 7) / 8 * 8;
  auto kernel = p.D == 128 ? attn_bwd_dkdv_dq_kernel<E, kRope, 128, false>
                : dkdv::solo_units(p.Hq / p.Hkv, nkb, p.D) ? attn_bwd_dkdv_dq_kernel<E, kRope, 64, true>
                                                            : attn_bwd_dkdv_dq_kernel<E, kRope, 64, false>;
  kernel<<<dim3((unsigned)P), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta, rcos, rsin,
      static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), p.B,
      p.T, p.Hq, p.Hkv, p.scale, p.scale_log2, p.causal, n_dq, n_kv, P);
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
