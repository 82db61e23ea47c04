// softmax_rows.hip -- the three row kernels of the unfused attention baseline,
// which reads and writes the [T, T] score matrix in HBM between library GEMMs
// ("Training a 100M transformer in pure Rust: RustingBrain vs PyTorch and
// TensorFlow", section "Step 1: measure before changing anything": the
// causal_softmax_lse, causal_probs_from_lse and causal_softmax_bwd kernels and
// the fp32 [seq_len, seq_len] matrix they move).
//
// One 64-lane wave owns one row (b, h, i) of a [T, T] matrix; four rows per
// 256-thread workgroup.  Lane l handles columns VEC*(l + 64c) + e.  With the
// causal mask only columns j <= i are read (len = i + 1); every column of the
// output row is written, zeros past len, because the next GEMM reads the whole
// matrix.  Row reductions are per-lane partials in column order, then a fixed
// xor butterfly: the same bits in every lane and every run.
#include "unfused.hpp"

namespace rca {
namespace unf {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kThreads = 64 * kRowsPerBlock;

template <class E>
__device__ __forceinline__ uint16_t to_e16(float x) {
  return (uint16_t)(E::pack2(x, 0.f) & 0xffffu);
}
template <class E>
__device__ __forceinline__ float from_e16(uint16_t h) {
  return E::lo((uint32_t)h);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// (m, l): running maximum and sum of exp2(x - m); merged by the fixed butterfly.
__device__ __forceinline__ void wave_merge(float& m, float& l) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
    const float mn = fmaxf(m, mo);
    l = l * fast_exp2(m - mn) + lo * fast_exp2(mo - mn);
    m = mn;
  }
}

struct Row {
  size_t base;  // first element of the row in a [rows, T] matrix
  int len;      // columns read: i + 1 with the causal mask, else T
};

__device__ __forceinline__ bool row_of(long long n_rows, int T, int causal, Row& r) {
  const long long row = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= n_rows) return false;
  const int i = (int)(row % T);
  r.base = (size_t)row * (size_t)T;
  r.len = causal ? i + 1 : T;
  return true;
}

// Forward: P = exp(scale * S - lse) in the 16-bit type and lse = ln sum_j exp(scale * S_ij).
template <class E, int VEC>
__global__ __launch_bounds__(kThreads) void softmax_lse_kernel(const float* __restrict__ s,
                                                                uint16_t* __restrict__ p,
                                                                float* __restrict__ lse,
                                                                long long n_rows, int T,
                                                                float scale_log2, int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  const float* src = s + r.base;
  float m = -1e30f, l = 0.f;
  for (int j0 = VEC * lane; j0 < r.len; j0 += 64 * VEC) {
    float x[VEC];
    if (VEC == 4 && j0 + 3 < r.len) {
      const float4 v = *reinterpret_cast<const float4*>(src + j0);
      x[0] = v.x; x[VEC > 1 ? 1 : 0] = v.y; x[VEC > 2 ? 2 : 0] = v.z; x[VEC > 3 ? 3 : 0] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = j0 + e < r.len ? src[j0 + e] : -1e30f;
    }
    float mx = m;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      x[e] = j0 + e < r.len ? x[e] * scale_log2 : -1e30f;
      mx = fmaxf(mx, x[e]);
    }
    l *= fast_exp2(m - mx);
    m = mx;
#pragma unroll
    for (int e = 0; e < VEC; ++e) l += fast_exp2(x[e] - m);
  }
  wave_merge(m, l);
  const float lse2 = m + fast_log2(l);
  if (lane == 0) lse[r.base / (size_t)T] = lse2 * kLn2;
  uint16_t* dst = p + r.base;
  for (int j0 = VEC * lane; j0 < T; j0 += 64 * VEC) {
    float y[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      y[e] = j0 + e < r.len ? fast_exp2(src[j0 + e] * scale_log2 - lse2) : 0.f;
    if (VEC == 4 && j0 + 3 < T) {
      u32x2_t w;
      w[0] = E::pack2(y[0], y[VEC > 1 ? 1 : 0]);
      w[1] = E::pack2(y[VEC > 2 ? 2 : 0], y[VEC > 3 ? 3 : 0]);
      *reinterpret_cast<u32x2_t*>(dst + j0) = w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (j0 + e < T) dst[j0 + e] = to_e16<E>(y[e]);
    }
  }
}

// Backward, first step: P recomputed from the scores and the forward's lse.
template <class E, int VEC>
__global__ __launch_bounds__(kThreads) void probs_from_lse_kernel(const float* __restrict__ s,
                                                                   const float* __restrict__ lse,
                                                                   uint16_t* __restrict__ p,
                                                                   long long n_rows, int T,
                                                                   float scale_log2, int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  const float lse2 = lse[r.base / (size_t)T] * kLog2e;
  const float* src = s + r.base;
  uint16_t* dst = p + r.base;
  for (int j0 = VEC * lane; j0 < T; j0 += 64 * VEC) {
    float y[VEC];
    if (VEC == 4 && j0 + 3 < r.len) {
      const float4 v = *reinterpret_cast<const float4*>(src + j0);
      y[0] = v.x; y[VEC > 1 ? 1 : 0] = v.y; y[VEC > 2 ? 2 : 0] = v.z; y[VEC > 3 ? 3 : 0] = v.w;
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = fast_exp2(y[e] * scale_log2 - lse2);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        y[e] = j0 + e < r.len ? fast_exp2(src[j0 + e] * scale_log2 - lse2) : 0.f;
    }
    if (VEC == 4 && j0 + 3 < T) {
      u32x2_t w;
      w[0] = E::pack2(y[0], y[VEC > 1 ? 1 : 0]);
      w[1] = E::pack2(y[VEC > 2 ? 2 : 0], y[VEC > 3 ? 3 : 0]);
      *reinterpret_cast<u32x2_t*>(dst + j0) = w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (j0 + e < T) dst[j0 + e] = to_e16<E>(y[e]);
    }
  }
}

// Backward, softmax step: dS = P * (dP - sum_j P_ij dP_ij), in the 16-bit type.
template <class E, int VEC>
__global__ __launch_bounds__(kThreads) void softmax_bwd_kernel(const uint16_t* __restrict__ p,
                                                                const float* __restrict__ dp,
                                                                uint16_t* __restrict__ ds,
                                                                long long n_rows, int T,
                                                                int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* pr = p + r.base;
  const float* dpr = dp + r.base;
  auto load = [&](int j0, float (&pv)[VEC], float (&gv)[VEC]) {
    if (VEC == 4 && j0 + 3 < r.len) {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(pr + j0);
      const float4 g = *reinterpret_cast<const float4*>(dpr + j0);
      pv[0] = E::lo(w[0]); pv[VEC > 1 ? 1 : 0] = E::hi(w[0]);
      pv[VEC > 2 ? 2 : 0] = E::lo(w[1]); pv[VEC > 3 ? 3 : 0] = E::hi(w[1]);
      gv[0] = g.x; gv[VEC > 1 ? 1 : 0] = g.y; gv[VEC > 2 ? 2 : 0] = g.z; gv[VEC > 3 ? 3 : 0] = g.w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const bool in = j0 + e < r.len;
        pv[e] = in ? from_e16<E>(pr[j0 + e]) : 0.f;
        gv[e] = in ? dpr[j0 + e] : 0.f;
      }
    }
  };
  float acc = 0.f;
  for (int j0 = VEC * lane; j0 < r.len; j0 += 64 * VEC) {
    float pv[VEC], gv[VEC];
    load(j0, pv, gv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc = fmaf(pv[e], gv[e], acc);
  }
  const float delta = wave_sum(acc);
  uint16_t* dst = ds + r.base;
  for (int j0 = VEC * lane; j0 < T; j0 += 64 * VEC) {
    float pv[VEC], gv[VEC], y[VEC];
    load(j0, pv, gv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = pv[e] * (gv[e] - delta);  // 0 past len
    if (VEC == 4 && j0 + 3 < T) {
      u32x2_t w;
      w[0] = E::pack2(y[0], y[VEC > 1 ? 1 : 0]);
      w[1] = E::pack2(y[VEC > 2 ? 2 : 0], y[VEC > 3 ? 3 : 0]);
      *reinterpret_cast<u32x2_t*>(dst + j0) = w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (j0 + e < T) dst[j0 + e] = to_e16<E>(y[e]);
    }
  }
}

// Register-resident variants for T % 4 == 0 and T <= 256*CH: lane l holds
// columns 4l + 256c + 0..3 of its row for c < CH, so every load of the row is
// issued before the first use and each row is read from HBM once.
template <int CH>
__device__ __forceinline__ void load_row_f32(const float* __restrict__ src, int len, int lane,
                                             float (&x)[CH][4], float fill) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j0 = 4 * lane + 256 * c;
    if (j0 + 3 < len) {
      const float4 v = *reinterpret_cast<const float4*>(src + j0);
      x[c][0] = v.x; x[c][1] = v.y; x[c][2] = v.z; x[c][3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[c][e] = j0 + e < len ? src[j0 + e] : fill;
    }
  }
}

template <class E, int CH>
__device__ __forceinline__ void store_row_e16(uint16_t* __restrict__ dst, int T, int lane,
                                              const float (&y)[CH][4]) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j0 = 4 * lane + 256 * c;
    if (j0 < T) {  // T % 4 == 0: the whole group of four is in the row
      u32x2_t w;
      w[0] = E::pack2(y[c][0], y[c][1]);
      w[1] = E::pack2(y[c][2], y[c][3]);
      *reinterpret_cast<u32x2_t*>(dst + j0) = w;
    }
  }
}

template <class E, int CH>
__global__ __launch_bounds__(kThreads) void softmax_lse_resident(const float* __restrict__ s,
                                                                  uint16_t* __restrict__ p,
                                                                  float* __restrict__ lse,
                                                                  long long n_rows, int T,
                                                                  float scale_log2, int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  float x[CH][4];
  load_row_f32<CH>(s + r.base, r.len, lane, x, 0.f);
  float m = -1e30f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = 4 * lane + 256 * c + e < r.len;
      x[c][e] = in ? x[c][e] * scale_log2 : -1e30f;
      m = fmaxf(m, x[c][e]);
    }
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) l += fast_exp2(x[c][e] - m);
  wave_merge(m, l);
  const float lse2 = m + fast_log2(l);
  if (lane == 0) lse[r.base / (size_t)T] = lse2 * kLn2;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[c][e] = 4 * lane + 256 * c + e < r.len ? fast_exp2(x[c][e] - lse2) : 0.f;
  store_row_e16<E, CH>(p + r.base, T, lane, x);
}

template <class E, int CH>
__global__ __launch_bounds__(kThreads) void probs_from_lse_resident(const float* __restrict__ s,
                                                                     const float* __restrict__ lse,
                                                                     uint16_t* __restrict__ p,
                                                                     long long n_rows, int T,
                                                                     float scale_log2, int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  const float lse2 = lse[r.base / (size_t)T] * kLog2e;
  float x[CH][4];
  load_row_f32<CH>(s + r.base, r.len, lane, x, 0.f);
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[c][e] = 4 * lane + 256 * c + e < r.len ? fast_exp2(x[c][e] * scale_log2 - lse2) : 0.f;
  store_row_e16<E, CH>(p + r.base, T, lane, x);
}

template <class E, int CH>
__global__ __launch_bounds__(kThreads) void softmax_bwd_resident(const uint16_t* __restrict__ p,
                                                                  const float* __restrict__ dp,
                                                                  uint16_t* __restrict__ ds,
                                                                  long long n_rows, int T,
                                                                  int causal) {
  Row r;
  if (!row_of(n_rows, T, causal, r)) return;
  const int lane = threadIdx.x & 63;
  float g[CH][4], pv[CH][4];
  load_row_f32<CH>(dp + r.base, r.len, lane, g, 0.f);
  const uint16_t* pr = p + r.base;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j0 = 4 * lane + 256 * c;
    if (j0 + 3 < r.len) {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(pr + j0);
      pv[c][0] = E::lo(w[0]); pv[c][1] = E::hi(w[0]);
      pv[c][2] = E::lo(w[1]); pv[c][3] = E::hi(w[1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[c][e] = j0 + e < r.len ? from_e16<E>(pr[j0 + e]) : 0.f;
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(pv[c][e], g[c][e], acc);
  const float delta = wave_sum(acc);
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) g[c][e] = pv[c][e] * (g[c][e] - delta);  // 0 past len
  store_row_e16<E, CH>(ds + r.base, T, lane, g);
}

dim3 row_grid(long long n_rows) { return dim3((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

}  // namespace


// Chunks per lane of the register-resident kernels: 1, 2, 4 or 8 (T <= 2048,
// T % 4 == 0), else 0 (the looped kernels).
int resident_chunks(int T) {
  if (T % 4 != 0 || T > 2048) return 0;
  return T <= 256 ? 1 : T <= 512 ? 2 : T <= 1024 ? 4 : 8;
}

#define RCA_RESIDENT_DISPATCH(KERNEL, ...)                                                  \
  switch (resident_chunks(T)) {                                                            \
    case 1: KERNEL<E, 1><<<row_grid(n_rows), kThreads, 0, st>>>(__VA_ARGS__); break;      \
    case 2: KERNEL<E, 2><<<row_grid(n_rows), kThreads, 0, st>>>(__VA_ARGS__); break;      \
    case 4: KERNEL<E, 4><<<row_grid(n_rows), kThreads, 0, st>>>(__VA_ARGS__); break;      \
    default: KERNEL<E, 8><<<row_grid(n_rows), kThreads, 0, st>>>(__VA_ARGS__); break;     \
  }

template <class E>
hipError_t softmax_lse(const float* s, void* p, float* lse, long long n_rows, int T,
                       float scale_log2, int causal, hipStream_t st) {
  uint16_t* p16 = static_cast<uint16_t*>(p);
  if (resident_chunks(T) > 0) {
    RCA_RESIDENT_DISPATCH(softmax_lse_resident, s, p16, lse, n_rows, T, scale_log2, causal)
  } else if (T % 4 == 0) {
    softmax_lse_kernel<E, 4><<<row_grid(n_rows), kThreads, 0, st>>>(s, p16, lse, n_rows, T,
                                                                     scale_log2, causal);
  } else {
    softmax_lse_kernel<E, 1><<<row_grid(n_rows), kThreads, 0, st>>>(s, p16, lse, n_rows, T,
                                                                     scale_log2, causal);
  }
  return hipGetLastError();
}

template <class E>
hipError_t probs_from_lse(const float* s, const float* lse, void* p, long long n_rows, int T,
                          float scale_log2, int causal, hipStream_t st) {
  uint16_t* p16 = static_cast<uint16_t*>(p);
  if (resident_chunks(T) > 0) {
    RCA_RESIDENT_DISPATCH(probs_from_lse_resident, s, lse, p16, n_rows, T, scale_log2, causal)
  } else if (T % 4 == 0) {
    probs_from_lse_kernel<E, 4><<<row_grid(n_rows), kThreads, 0, st>>>(s, lse, p16, n_rows, T,
                                                                        scale_log2, causal);
  } else {
    probs_from_lse_kernel<E, 1><<<row_grid(n_rows), kThreads, 0, st>>>(s, lse, p16, n_rows, T,
                                                                        scale_log2, causal);
  }
  return hipGetLastError();
}

template <class E>
hipError_t softmax_bwd(const void* p, const float* dp, void* ds, long long n_rows, int T,
                       int causal, hipStream_t st) {
  const uint16_t* p16 = static_cast<const uint16_t*>(p);
  uint16_t* ds16 = static_cast<uint16_t*>(ds);
  if (resident_chunks(T) > 0) {
    RCA_RESIDENT_DISPATCH(softmax_bwd_resident, p16, dp, ds16, n_rows, T, causal)
  } else if (T % 4 == 0) {
    softmax_bwd_kernel<E, 4><<<row_grid(n_rows), kThreads, 0, st>>>(p16, dp, ds16, n_rows, T,
                                                                     causal);
  } else {
    softmax_bwd_kernel<E, 1><<<row_grid(n_rows), kThreads, 0, st>>>(p16, dp, ds16, n_rows, T,
                                                                     causal);
  }
  return hipGetLastError();
}

template hipError_t softmax_lse<Bf16>(const float*, void*, float*, long long, int, float, int, hipStream_t);
template hipError_t softmax_lse<F16>(const float*, void*, float*, long long, int, float, int, hipStream_t);
template hipError_t probs_from_lse<Bf16>(const float*, const float*, void*, long long, int, float, int, hipStream_t);
template hipError_t probs_from_lse<F16>(const float*, const float*, void*, long long, int, float, int, hipStream_t);
template hipError_t softmax_bwd<Bf16>(const void*, const float*, void*, long long, int, int, hipStream_t);
template hipError_t softmax_bwd<F16>(const void*, const float*, void*, long long, int, int, hipStream_t);

}  // namespace unf
}  // namespace rca
