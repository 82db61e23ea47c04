// tables.hip -- helper kernels of the unfused baseline: K and V repeated to
// their query heads (so every GEMM is evenly strided over the heads), and the
// fixed-order sum of per-head dK / dV partials over each KV group.
#include "unfused.hpp"

namespace rca {
namespace unf {
namespace {

// out[b][t][h][:] = in[b][t][h / G][:], 16 bytes per thread (D % 8 == 0).
__global__ __launch_bounds__(256) void repeat_kv_kernel(const uint16_t* __restrict__ in,
                                                         uint16_t* __restrict__ out, int B, int T,
                                                         int Hkv, int G, int D) {
  const int c8 = D / 8;
  const long long n = (long long)B * T * Hkv * G * c8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % c8);
  const long long bth = i / c8;  // (b*T + t)*Hq + h
  const int Hq = Hkv * G;
  const int h = (int)(bth % Hq);
  const long long bt = bth / Hq;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(in + (bt * Hkv + h / G) * D + 8 * c);
  *reinterpret_cast<u32x4_t*>(out + bth * D + 8 * c) = x;
}

// out[b][j][g][d] = sum_{r < G} in[b][g*G + r][j][d] (r ascending), rounded to E.
template <class E>
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ in,
                                                         uint16_t* __restrict__ out, int B, int T,
                                                         int Hkv, int G, int D) {
  const long long n4 = (long long)B * T * Hkv * D / 4;
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i4 >= n4) return;
  const long long e = i4 * 4;  // element of out: ((b*T + j)*Hkv + g)*D + d
  const int d = (int)(e % D);
  const long long t1 = e / D;
  const int g = (int)(t1 % Hkv);
  const long long t2 = t1 / Hkv;
  const int j = (int)(t2 % T);
  const int b = (int)(t2 / T);
  const int Hq = Hkv * G;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = 0; r < G; ++r) {
    const float4 x = *reinterpret_cast<const float4*>(
        in + (((size_t)b * Hq + (size_t)g * G + r) * T + j) * (size_t)D + d);
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  u32x2_t w;
  w[0] = E::pack2(acc.x, acc.y);
  w[1] = E::pack2(acc.z, acc.w);
  *reinterpret_cast<u32x2_t*>(out + e) = w;
}

}  // namespace

hipError_t repeat_kv(const void* in, void* out, int B, int T, int Hkv, int G, int D,
                     hipStream_t st) {
  const long long n = (long long)B * T * Hkv * G * (D / 8);
  repeat_kv_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(
      static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), B, T, Hkv, G, D);
  return hipGetLastError();
}

template <class E>
hipError_t group_sum(const float* in, void* out, int B, int T, int Hkv, int G, int D,
                     hipStream_t st) {
  const long long n4 = (long long)B * T * Hkv * D / 4;
  group_sum_kernel<E><<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(
      in, static_cast<uint16_t*>(out), B, T, Hkv, G, D);
  return hipGetLastError();
}

template hipError_t group_sum<Bf16>(const float*, void*, int, int, int, int, int, hipStream_t);
template hipError_t group_sum<F16>(const float*, void*, int, int, int, int, int, hipStream_t);

}  // namespace unf
}  // namespace rca
