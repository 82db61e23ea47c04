// bwd_pre.hip -- backward preprocess of fused causal attention (bf16):
// delta_i = <dO_i, o_i> for every (batch, query head, row), accumulated in fp32.
//
// This is the row term of the softmax backward, dS = P * (dP - delta), that the
// unfused causal_softmax_bwd kernel of "Training a 100M transformer in pure
// Rust: RustingBrain vs PyTorch and TensorFlow" (section "Step 1: measure before
// changing anything") needs.  It reads o and dO once and writes one float per
// row: HBM-bound.  Eight lanes share one row (16 bytes each per 64 columns,
// whole rows per wave instruction) and combine their partial dot products with
// a fixed butterfly, so the result is reproducible.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int PRE_THREADS = 256;
constexpr int PRE_ROWS = PRE_THREADS / 8;  // 8 lanes per row, 8 elements each per 64 columns

// Block blk covers positions 32*tc .. 32*tc + 31 of query head h of batch element
// b, with (b, tc, h) enumerated h fastest, so neighbouring blocks read the
// neighbouring head segments of the same tokens and each block's 32 delta values
// fill one 128-byte line of delta ([B, Hq, T]).  Lane `part` of a row's eight
// holds columns 8*part + 64c + 0..7 for c < kD/64.
template <class E, int kD>
__device__ __forceinline__ void delta_rows(int blk, const uint16_t* __restrict__ o,
                                           const uint16_t* __restrict__ dO,
                                           float* __restrict__ delta, int T, int Hq) {
  const int n_tc = (T + PRE_ROWS - 1) / PRE_ROWS;
  const int h = blk % Hq;
  const int btc = blk / Hq;
  const int b = btc / n_tc;
  const int t = (btc - b * n_tc) * PRE_ROWS + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const long long row = ((long long)b * T + t) * Hq + h;  // [b][t][h] row of o and dO
  float acc = 0.f;
  if (t < T) {
    u32x4_t a[kD / 64], c[kD / 64];
#pragma unroll
    for (int ch = 0; ch < kD / 64; ++ch) {
      a[ch] = gload16(o + row * kD + part * 8 + 64 * ch);
      c[ch] = gload16(dO + row * kD + part * 8 + 64 * ch);
    }
#pragma unroll
    for (int ch = 0; ch < kD / 64; ++ch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(E::lo(a[ch][i]), E::lo(c[ch][i]), acc);
        acc = fmaf(E::hi(a[ch][i]), E::hi(c[ch][i]), acc);
      }
    }
  }
  // Fixed butterfly over the 8 lanes of the row.
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (t < T && part == 0) delta[((long long)b * Hq + h) * T + t] = acc;
}

// Blocks of the delta part of a grid: one per (batch element, 32 positions, query head).
inline long long delta_blocks(const Problem& p) {
  return (long long)p.B * ((p.T + PRE_ROWS - 1) / PRE_ROWS) * p.Hq;
}

template <class E, int kD>
__global__ __launch_bounds__(PRE_THREADS) void attn_bwd_pre_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO, float* __restrict__ delta,
    int T, int Hq) {
  delta_rows<E, kD>(blockIdx.x, o, dO, delta, T, Hq);
}

// Backward preparation with rotary embedding: blocks [0, nd) write delta exactly
// as attn_bwd_pre_kernel does, blocks [nd, nd + nb) the rotated q rows and the
// rest the rotated k rows (rope_rotate, as the forward rotates them as it loads:
// the same bits), which the dK/dV and dQ kernels then read in place of q, k.
template <class E, int kD>
__global__ __launch_bounds__(PRE_THREADS) void attn_bwd_rope_prep_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ rcos, const float* __restrict__ rsin, float* __restrict__ delta,
    uint16_t* __restrict__ q_rot, uint16_t* __restrict__ k_rot, int T, int Hq, int Hkv,
    long long n_qrows, long long n_krows, int nd, int nb) {
  int blk = blockIdx.x;
  if (blk < nd) {
    delta_rows<E, kD>(blk, o, dO, delta, T, Hq);
    return;
  }
  blk -= nd;
  const uint16_t* src = q;
  uint16_t* dst = q_rot;
  int H = Hq;
  long long n_rows = n_qrows;
  if (blk >= nb) {
    blk -= nb;
    src = k;
    dst = k_rot;
    H = Hkv;
    n_rows = n_krows;
  }
  const long long row = (long long)blk * PRE_ROWS + (threadIdx.x >> 3);  // [b][t][h]
  const int part = threadIdx.x & 7;  // elements 8*part + 64ch .. +7, pairs 4*part + 32ch .. +3
  if (row < n_rows) {
    const int t = (int)((row / H) % T);
#pragma unroll
    for (int ch = 0; ch < kD / 64; ++ch) {
      u32x4_t x = gload16(src + row * kD + part * 8 + 64 * ch);
      const size_t ti = (size_t)t * (kD / 2) + part * 4 + 32 * ch;
      const float4 c = *reinterpret_cast<const float4*>(rcos + ti);
      const float4 s = *reinterpret_cast<const float4*>(rsin + ti);
      x[0] = rope_rotate<E>(x[0], c.x, s.x);
      x[1] = rope_rotate<E>(x[1], c.y, s.y);
      x[2] = rope_rotate<E>(x[2], c.z, s.z);
      x[3] = rope_rotate<E>(x[3], c.w, s.w);
      *reinterpret_cast<u32x4_t*>(dst + row * kD + part * 8 + 64 * ch) = x;
    }
  }
}

}  // namespace

template <class E>
hipError_t launch_bwd_pre_e(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s) {
  const dim3 grid((unsigned)delta_blocks(p));
  auto kernel = p.D == 128 ? attn_bwd_pre_kernel<E, 128> : attn_bwd_pre_kernel<E, 64>;
  kernel<<<grid, PRE_THREADS, 0, s>>>(static_cast<const uint16_t*>(o),
                                      static_cast<const uint16_t*>(dO), delta, p.T, p.Hq);
  return hipGetLastError();
}

template <class E>
hipError_t launch_bwd_rope_prep_e(const Problem& p, const void* o, const void* dO, const void* q,
                                  const void* k, const float* rcos, const float* rsin,
                                  float* delta, void* q_rot, void* k_rot, hipStream_t s) {
  const long long n_q = (long long)p.B * p.T * p.Hq, n_k = (long long)p.B * p.T * p.Hkv;
  const int nd = (int)delta_blocks(p);
  const int nb = (int)((n_q + PRE_ROWS - 1) / PRE_ROWS);
  const int nbk = (int)((n_k + PRE_ROWS - 1) / PRE_ROWS);
  const dim3 grid((unsigned)(nd + nb + nbk));
  auto kernel = p.D == 128 ? attn_bwd_rope_prep_kernel<E, 128> : attn_bwd_rope_prep_kernel<E, 64>;
  kernel<<<grid, PRE_THREADS, 0, s>>>(
      static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO),
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), rcos, rsin, delta,
      static_cast<uint16_t*>(q_rot), static_cast<uint16_t*>(k_rot), p.T, p.Hq, p.Hkv, n_q, n_k, nd, nb);
  return hipGetLastError();
}

hipError_t launch_bwd_rope_prep_bf16(const Problem& p, const void* o, const void* dO, const void* q,
                                     const void* k, const float* rcos, const float* rsin,
                                     float* delta, void* q_rot, void* k_rot, hipStream_t s) {
  return launch_bwd_rope_prep_e<Bf16>(p, o, dO, q, k, rcos, rsin, delta, q_rot, k_rot, s);
}

hipError_t launch_bwd_rope_prep_f16(const Problem& p, const void* o, const void* dO, const void* q,
                                    const void* k, const float* rcos, const float* rsin,
                                    float* delta, void* q_rot, void* k_rot, hipStream_t s) {
  return launch_bwd_rope_prep_e<F16>(p, o, dO, q, k, rcos, rsin, delta, q_rot, k_rot, s);
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
