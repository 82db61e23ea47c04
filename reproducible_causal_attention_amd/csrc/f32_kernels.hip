// f32_kernels.hip -- float32 instantiation of the fused causal attention path.
//
// Same algorithm and the same deterministic decomposition as the bf16 MFMA
// kernels (forward with online softmax and log-sum-exp output; backward as
// preprocess, dK/dV per key tile with a fixed loop over the group's query heads
// and the query tiles, dQ per query tile), but every product and sum is a
// float32 FMA on the vector ALUs: one thread owns one query row (forward, dQ)
// or one key row (dK/dV), with key/value or query tiles staged in LDS and read
// by all lanes at once (broadcast).  gfx950 has no reduced-precision fp32
// matrix mode, and this path is for small float32 problems where exactness
// matters more than speed.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int TB = 64;  // rows per workgroup and per LDS tile (one wave)

__device__ __forceinline__ void load_row(const float* __restrict__ src, bool valid, float* dst) {
#pragma unroll
  for (int c = 0; c < kHeadDim / 4; ++c) {
    const float4 x = valid ? reinterpret_cast<const float4*>(src)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[4 * c + 0] = x.x;
    dst[4 * c + 1] = x.y;
    dst[4 * c + 2] = x.z;
    dst[4 * c + 3] = x.w;
  }
}

__device__ __forceinline__ void tile_row_to_lds(const float* __restrict__ src, bool valid, float* dst) {
#pragma unroll
  for (int c = 0; c < kHeadDim / 4; ++c) {
    const float4 x = valid ? reinterpret_cast<const float4*>(src)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(dst)[c] = x;
  }
}

__device__ __forceinline__ float dot64(const float* a, const float* lds_row) {
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) acc = fmaf(a[d], lds_row[d], acc);
  return acc;
}

__global__ __launch_bounds__(TB) void attn_fwd_f32_kernel(const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          float* __restrict__ o, float* __restrict__ lse,
                                                          int B, int T, int Hq, int Hkv,
                                                          float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) float sK[TB * kHeadDim];
  __shared__ __attribute__((aligned(16))) float sV[TB * kHeadDim];
  const int tid = threadIdx.x;
  const int n_qt = (T + TB - 1) / TB;
  const int BH = B * Hq;
  int qt = blockIdx.x / BH;
  const int bh = blockIdx.x - qt * BH;
  if (causal) qt = n_qt - 1 - qt;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const int kvh = h / (Hq / Hkv);
  const size_t q_stride = (size_t)Hq * kHeadDim, kv_stride = (size_t)Hkv * kHeadDim;
  const int my_q = qt * TB + tid;
  const size_t qoff = ((size_t)b * T + my_q) * q_stride + (size_t)h * kHeadDim;
  const float* kbase = k + ((size_t)b * T * Hkv + kvh) * kHeadDim;
  const float* vbase = v + ((size_t)b * T * Hkv + kvh) * kHeadDim;

  float qr[kHeadDim], acc[kHeadDim];
  load_row(q + qoff, my_q < T, qr);
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) acc[d] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  const int kv_end = causal ? min(T, (qt + 1) * TB) : T;
  const int n_kv = (kv_end + TB - 1) / TB;
  for (int kt = 0; kt < n_kv; ++kt) {
    const int k0 = kt * TB;
    __syncthreads();
    tile_row_to_lds(kbase + (size_t)(k0 + tid) * kv_stride, k0 + tid < T, sK + tid * kHeadDim);
    tile_row_to_lds(vbase + (size_t)(k0 + tid) * kv_stride, k0 + tid < T, sV + tid * kHeadDim);
    __syncthreads();
    float s[TB];
    float mx = -__builtin_inff();
#pragma unroll 4
    for (int j = 0; j < TB; ++j) {
      const int key = k0 + j;
      float sv = dot64(qr, sK + j * kHeadDim) * scale_log2;
      if ((causal && key > my_q) || key >= T) sv = -__builtin_inff();
      s[j] = sv;
      mx = fmaxf(mx, sv);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) acc[d] *= alpha;
#pragma unroll 4
    for (int j = 0; j < TB; ++j) {
      const float p = fast_exp2(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) acc[d] = fmaf(p, sV[j * kHeadDim + d], acc[d]);
    }
  }
  if (my_q < T) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int c = 0; c < kHeadDim / 4; ++c)
      reinterpret_cast<float4*>(o + qoff)[c] =
          make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv);
    lse[((size_t)b * Hq + h) * T + my_q] = (m_run + fast_log2(l_run)) * kLn2;
  }
}

constexpr int PRE_THREADS = 256;
constexpr int PRE_ROWS = PRE_THREADS / 16;  // 16 lanes x 4 floats per 64-wide row

__global__ __launch_bounds__(PRE_THREADS) void attn_bwd_pre_f32_kernel(
    const float* __restrict__ o, const float* __restrict__ dO, float* __restrict__ delta, int T,
    int Hq, long long n_rows) {
  const long long row = (long long)blockIdx.x * PRE_ROWS + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (row < n_rows) {
    const float4 a = reinterpret_cast<const float4*>(o + row * kHeadDim)[part];
    const float4 c = reinterpret_cast<const float4*>(dO + row * kHeadDim)[part];
    acc = fmaf(a.x, c.x, acc);
    acc = fmaf(a.y, c.y, acc);
    acc = fmaf(a.z, c.z, acc);
    acc = fmaf(a.w, c.w, acc);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (row < n_rows && part == 0) {
    const long long bt = row / Hq;
    const int h = (int)(row - bt * Hq);
    const long long b = bt / T;
    const int t = (int)(bt - b * T);
    delta[(b * Hq + h) * T + t] = acc;
  }
}

__global__ __launch_bounds__(TB) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, int B, int T, int Hq, int Hkv, float scale,
    float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) float sQ[TB * kHeadDim];
  __shared__ __attribute__((aligned(16))) float sdO[TB * kHeadDim];
  __shared__ float sL[TB], sD[TB];
  const int tid = threadIdx.x;
  const int BG = B * Hkv;
  const int kt = blockIdx.x / BG;
  const int bg = blockIdx.x - kt * BG;
  const int b = bg / Hkv, kvh = bg - (bg / Hkv) * Hkv;
  const int G = Hq / Hkv;
  const size_t q_stride = (size_t)Hq * kHeadDim, kv_stride = (size_t)Hkv * kHeadDim;
  const int my_key = kt * TB + tid;
  const size_t koff = ((size_t)b * T + my_key) * kv_stride + (size_t)kvh * kHeadDim;

  float kr[kHeadDim], vr[kHeadDim], dka[kHeadDim], dva[kHeadDim];
  load_row(k + koff, my_key < T, kr);
  load_row(v + koff, my_key < T, vr);
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) dka[d] = dva[d] = 0.f;

  const int n_qt = (T + TB - 1) / TB;
  const int qt_begin = causal ? kt : 0;
  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    for (int qt = qt_begin; qt < n_qt; ++qt) {
      const int q0 = qt * TB;
      const int qi_load = q0 + tid;
      const size_t qoff = ((size_t)b * T + qi_load) * q_stride + (size_t)h * kHeadDim;
      __syncthreads();
      tile_row_to_lds(q + qoff, qi_load < T, sQ + tid * kHeadDim);
      tile_row_to_lds(dO + qoff, qi_load < T, sdO + tid * kHeadDim);
      sL[tid] = qi_load < T ? lse[((size_t)b * Hq + h) * T + qi_load] * kLog2e : 0.f;
      sD[tid] = qi_load < T ? delta[((size_t)b * Hq + h) * T + qi_load] : 0.f;
      __syncthreads();
      for (int i = 0; i < TB; ++i) {
        const int qi = q0 + i;
        if (qi >= T || (causal && my_key > qi)) continue;
        const float p = fast_exp2(dot64(kr, sQ + i * kHeadDim) * scale_log2 - sL[i]);
        const float ds = p * (dot64(vr, sdO + i * kHeadDim) - sD[i]);
#pragma unroll
        for (int d = 0; d < kHeadDim; ++d) {
          dva[d] = fmaf(p, sdO[i * kHeadDim + d], dva[d]);
          dka[d] = fmaf(ds, sQ[i * kHeadDim + d], dka[d]);
        }
      }
    }
  }
  if (my_key < T) {
#pragma unroll
    for (int c = 0; c < kHeadDim / 4; ++c) {
      reinterpret_cast<float4*>(dk + koff)[c] = make_float4(
          dka[4 * c] * scale, dka[4 * c + 1] * scale, dka[4 * c + 2] * scale, dka[4 * c + 3] * scale);
      reinterpret_cast<float4*>(dv + koff)[c] =
          make_float4(dva[4 * c], dva[4 * c + 1], dva[4 * c + 2], dva[4 * c + 3]);
    }
  }
}

__global__ __launch_bounds__(TB) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  __shared__ __attribute__((aligned(16))) float sK[TB * kHeadDim];
  __shared__ __attribute__((aligned(16))) float sV[TB * kHeadDim];
  const int tid = threadIdx.x;
  const int n_qt = (T + TB - 1) / TB;
  const int BH = B * Hq;
  int qt = blockIdx.x / BH;
  const int bh = blockIdx.x - qt * BH;
  if (causal) qt = n_qt - 1 - qt;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const int kvh = h / (Hq / Hkv);
  const size_t q_stride = (size_t)Hq * kHeadDim, kv_stride = (size_t)Hkv * kHeadDim;
  const int my_q = qt * TB + tid;
  const size_t qoff = ((size_t)b * T + my_q) * q_stride + (size_t)h * kHeadDim;
  const float* kbase = k + ((size_t)b * T * Hkv + kvh) * kHeadDim;
  const float* vbase = v + ((size_t)b * T * Hkv + kvh) * kHeadDim;

  float qr[kHeadDim], dor[kHeadDim], acc[kHeadDim];
  load_row(q + qoff, my_q < T, qr);
  load_row(dO + qoff, my_q < T, dor);
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) acc[d] = 0.f;
  const float L2 = my_q < T ? lse[((size_t)b * Hq + h) * T + my_q] * kLog2e : 0.f;
  const float Dl = my_q < T ? delta[((size_t)b * Hq + h) * T + my_q] : 0.f;

  const int kv_end = causal ? min(T, (qt + 1) * TB) : T;
  const int n_kv = (kv_end + TB - 1) / TB;
  for (int kt = 0; kt < n_kv; ++kt) {
    const int k0 = kt * TB;
    __syncthreads();
    tile_row_to_lds(kbase + (size_t)(k0 + tid) * kv_stride, k0 + tid < T, sK + tid * kHeadDim);
    tile_row_to_lds(vbase + (size_t)(k0 + tid) * kv_stride, k0 + tid < T, sV + tid * kHeadDim);
    __syncthreads();
    for (int j = 0; j < TB; ++j) {
      const int key = k0 + j;
      if (key >= T || (causal && key > my_q)) continue;
      const float p = fast_exp2(dot64(qr, sK + j * kHeadDim) * scale_log2 - L2);
      const float ds = p * (dot64(dor, sV + j * kHeadDim) - Dl);
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) acc[d] = fmaf(ds, sK[j * kHeadDim + d], acc[d]);
    }
  }
  if (my_q < T) {
#pragma unroll
    for (int c = 0; c < kHeadDim / 4; ++c)
      reinterpret_cast<float4*>(dq + qoff)[c] = make_float4(
          acc[4 * c] * scale, acc[4 * c + 1] * scale, acc[4 * c + 2] * scale, acc[4 * c + 3] * scale);
  }
}

}  // namespace

const char* f32_tiles() { return "f32{rows=64,valu_fma}"; }

hipError_t launch_fwd_f32(const Problem& p, const void* q, const void* k, const void* v, void* o,
                          float* lse, hipStream_t s) {
  const int n_qt = (p.T + TB - 1) / TB;
  attn_fwd_f32_kernel<<<dim3((unsigned)(n_qt * p.B * p.Hq)), TB, 0, s>>>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<float*>(o), lse, p.B, p.T, p.Hq, p.Hkv, p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_bwd_pre_f32(const Problem& p, const void* o, const void* dO, float* delta,
                              hipStream_t s) {
  const long long n_rows = (long long)p.B * p.T * p.Hq;
  attn_bwd_pre_f32_kernel<<<dim3((unsigned)((n_rows + PRE_ROWS - 1) / PRE_ROWS)), PRE_THREADS, 0, s>>>(
      static_cast<const float*>(o), static_cast<const float*>(dO), delta, p.T, p.Hq, n_rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const Problem& p, const void* q, const void* k, const void* v,
                               const void* dO, const float* lse, const float* delta, void* dk,
                               void* dv, hipStream_t s) {
  const int n_kt = (p.T + TB - 1) / TB;
  attn_bwd_dkdv_f32_kernel<<<dim3((unsigned)(n_kt * p.B * p.Hkv)), TB, 0, s>>>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(dO), lse, delta, static_cast<float*>(dk), static_cast<float*>(dv),
      p.B, p.T, p.Hq, p.Hkv, p.scale, p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const Problem& p, const void* q, const void* k, const void* v,
                             const void* dO, const float* lse, const float* delta, void* dq,
                             hipStream_t s) {
  const int n_qt = (p.T + TB - 1) / TB;
  attn_bwd_dq_f32_kernel<<<dim3((unsigned)(n_qt * p.B * p.Hq)), TB, 0, s>>>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(dO), lse, delta, static_cast<float*>(dq), p.B, p.T, p.Hq, p.Hkv,
      p.scale, p.scale_log2, p.causal);
  return hipGetLastError();
}

}  // namespace rca
