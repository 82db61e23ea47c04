// unfused_api.hip -- C ABI of the unfused baseline (include/attn_unfused.h):
// validation, workspace layout, rocBLAS GEMM calls and the row kernels.
//
// Tensors are row-major; rocBLAS is column-major, so a row-major [m, n] matrix
// with row stride ld is passed as the column-major n x m matrix with leading
// dimension ld.  With grouped heads the KV head of query head h is h / G, not
// evenly strided in h, so K and V are first repeated to the Hq query heads in
// the workspace; then every GEMM is one strided-batched call over the Hq heads
// of each batch element.  dK and dV are formed per query head in float32 and
// summed over each KV group in a fixed order.
#include <rocblas/rocblas.h>

#include "../../../include/attn_unfused.h"
#include "../validate.hpp"
#include "unfused.hpp"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

struct attn_unfused_ctx {
  rocblas_handle blas;
};

namespace {

using namespace rca::validate;

constexpr long long kMaxT = 1LL << 16;
constexpr long long kMaxMatrixBytes = 1LL << 37;  // float32 [B, Hq, T, T]

attn_status_t check_shape(int B, int T, int Hq, int Hkv, int D, attn_dtype_t dtype) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (T > kMaxT) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * Hq * (long long)T * T * 4 >= kMaxMatrixBytes) return ATTN_ERR_INVALID_ARG;
  if ((long long)T * Hq * D >= (1LL << 31)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  if (D % 8 != 0 || D > 256) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

struct Layout {
  size_t s, p, ds, dkh, dvh, krep, vrep, total;  // byte offsets into the workspace
};

Layout layout(int B, int T, int Hq, int D) {
  const size_t n = (size_t)B * Hq * T * T, m = (size_t)B * Hq * T * D;
  Layout l;
  l.s = 0;
  l.p = l.s + round256(4 * n);
  l.ds = l.p + round256(2 * n);
  l.dkh = l.ds + round256(2 * n);
  l.dvh = l.dkh + round256(4 * m);
  l.krep = l.dvh + round256(4 * m);
  l.vrep = l.krep + round256(2 * m);
  l.total = l.vrep + round256(2 * m);
  return l;
}

attn_status_t from_blas(rocblas_status st) {
  if (st == rocblas_status_success) return ATTN_OK;
  if (st == rocblas_status_not_implemented) return ATTN_ERR_UNSUPPORTED;
  return ATTN_ERR_HIP;
}

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

#define ATTN_TRY(expr)                \
  do {                                \
    const attn_status_t st_ = (expr); \
    if (st_ != ATTN_OK) return st_;   \
  } while (0)

// One strided-batched GEMM over the Hq heads of a batch element, column-major:
// C_h = alpha op(A_h) op(B_h) + beta C_h; inputs of type `ab`, output of type
// `ct`, float32 accumulation.
struct Gemm {
  rocblas_handle h;
  rocblas_datatype ab;
  int batch;
  attn_status_t operator()(rocblas_operation ta, rocblas_operation tb, int m, int n, int k,
                           float alpha, const void* a, int lda, long long sa, const void* b,
                           int ldb, long long sb, float beta, void* c, rocblas_datatype ct,
                           int ldc, long long sc) const {
    return from_blas(rocblas_gemm_strided_batched_ex(
        h, ta, tb, m, n, k, &alpha, a, ab, lda, sa, b, ab, ldb, sb, &beta, c, ct, ldc, sc, c, ct,
        ldc, sc, batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0));
  }
};

constexpr rocblas_operation N_ = rocblas_operation_none;
constexpr rocblas_operation T_ = rocblas_operation_transpose;

// Sizes of one call; element offsets of batch element b in each kind of buffer.
struct Shape {
  int B, T, Hq, Hkv, D, G;
  long long qe, tt, he;  // per batch element of q-shaped tensors; per [T, T]; per head [T, D]
  Shape(int B_, int T_, int Hq_, int Hkv_, int D_)
      : B(B_), T(T_), Hq(Hq_), Hkv(Hkv_), D(D_), G(Hq_ / Hkv_),
        qe((long long)T_ * Hq_ * D_), tt((long long)T_ * T_), he((long long)T_ * D_) {}
};

inline const char* at(const void* base, long long elems, int es) { return static_cast<const char*>(base) + elems * es; }
inline char* at(void* base, long long elems, int es) { return static_cast<char*>(base) + elems * es; }

template <class E>
struct Launch;
template <>
struct Launch<rca::Bf16> {
  static constexpr rocblas_datatype type = rocblas_datatype_bf16_r;
};
template <>
struct Launch<rca::F16> {
  static constexpr rocblas_datatype type = rocblas_datatype_f16_r;
};

// K and V of every query head: the repeated copies in the workspace, or k, v
// themselves without grouping.
struct KV {
  const void* k;
  const void* v;
};

KV repeat_kv(const Shape& z, const void* k, const void* v, char* ws, const Layout& l,
             hipStream_t st, attn_status_t& status) {
  status = ATTN_OK;
  if (z.G == 1) return KV{k, v};
  void* kr = ws + l.krep;
  void* vr = ws + l.vrep;
  status = from_hip(rca::unf::repeat_kv(k, kr, z.B, z.T, z.Hkv, z.G, z.D, st));
  if (status == ATTN_OK) status = from_hip(rca::unf::repeat_kv(v, vr, z.B, z.T, z.Hkv, z.G, z.D, st));
  return KV{kr, vr};
}

// S_h = x_h y_h^T as float32 [T, T] for every head (x, y: [B, T, Hq, D]):
// column-major (T_j x T_i) = y (T_j x D) . x^T (D x T_i).
attn_status_t scores(const Gemm& gemm, const Shape& z, const void* x, const void* y, float* s) {
  for (int b = 0; b < z.B; ++b)
    ATTN_TRY(gemm(T_, N_, z.T, z.T, z.D, 1.f, at(y, b * z.qe, 2), z.Hq * z.D, z.D,
                  at(x, b * z.qe, 2), z.Hq * z.D, z.D, 0.f, s + b * z.Hq * z.tt,
                  rocblas_datatype_f32_r, z.T, z.tt));
  return ATTN_OK;
}

template <class E>
attn_status_t run_fwd(rocblas_handle h, const Shape& z, const void* q, const void* k,
                      const void* v, void* o, float* lse, float scale, int causal, char* ws,
                      hipStream_t st) {
  const Layout l = layout(z.B, z.T, z.Hq, z.D);
  const Gemm gemm{h, Launch<E>::type, z.Hq};
  float* s = reinterpret_cast<float*>(ws + l.s);
  void* p = ws + l.p;
  attn_status_t status;
  const KV kv = repeat_kv(z, k, v, ws, l, st, status);
  ATTN_TRY(status);
  ATTN_TRY(scores(gemm, z, q, kv.k, s));
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  ATTN_TRY(from_hip(rca::unf::softmax_lse<E>(s, p, lse, (long long)z.B * z.Hq * z.T, z.T,
                                             scale_log2, causal, st)));
  // o_h = P_h v_h: column-major (D x T_i) = v^T (D x T_j) . P^T (T_j x T_i).
  for (int b = 0; b < z.B; ++b)
    ATTN_TRY(gemm(N_, N_, z.D, z.T, z.T, 1.f, at(kv.v, b * z.qe, 2), z.Hq * z.D, z.D,
                  at(p, b * z.Hq * z.tt, 2), z.T, z.tt, 0.f, at(o, b * z.qe, 2), Launch<E>::type,
                  z.Hq * z.D, z.D));
  return ATTN_OK;
}

template <class E>
attn_status_t run_bwd(rocblas_handle h, const Shape& z, const void* q, const void* k,
                      const void* v, const float* lse, const void* dO, void* dq, void* dk,
                      void* dv, float scale, int causal, char* ws, hipStream_t st) {
  const Layout l = layout(z.B, z.T, z.Hq, z.D);
  const Gemm gemm{h, Launch<E>::type, z.Hq};
  float* s = reinterpret_cast<float*>(ws + l.s);  // S, then dP
  void* p = ws + l.p;
  void* ds = ws + l.ds;
  float* dkh = reinterpret_cast<float*>(ws + l.dkh);
  float* dvh = reinterpret_cast<float*>(ws + l.dvh);
  const long long n_rows = (long long)z.B * z.Hq * z.T;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  attn_status_t status;
  const KV kv = repeat_kv(z, k, v, ws, l, st, status);
  ATTN_TRY(status);
  ATTN_TRY(scores(gemm, z, q, kv.k, s));
  ATTN_TRY(from_hip(rca::unf::probs_from_lse<E>(s, lse, p, n_rows, z.T, scale_log2, causal, st)));
  ATTN_TRY(scores(gemm, z, dO, kv.v, s));  // dP overwrites S (stream order)
  ATTN_TRY(from_hip(rca::unf::softmax_bwd<E>(p, s, ds, n_rows, z.T, causal, st)));
  for (int b = 0; b < z.B; ++b) {
    const long long mo = b * z.Hq * z.tt, ho = b * z.Hq * z.he;
    // Per query head, float32 [T, D]: dv_h = P_h^T dO_h and dk_h = scale dS_h^T q_h,
    // column-major (D x T_j) = x^T (D x T_i) . M (T_i x T_j).
    ATTN_TRY(gemm(N_, T_, z.D, z.T, z.T, 1.f, at(dO, b * z.qe, 2), z.Hq * z.D, z.D,
                  at(p, mo, 2), z.T, z.tt, 0.f, dvh + ho, rocblas_datatype_f32_r, z.D, z.he));
    ATTN_TRY(gemm(N_, T_, z.D, z.T, z.T, scale, at(q, b * z.qe, 2), z.Hq * z.D, z.D,
                  at(ds, mo, 2), z.T, z.tt, 0.f, dkh + ho, rocblas_datatype_f32_r, z.D, z.he));
    // dq_h = scale dS_h k_h: column-major (D x T_i) = k^T (D x T_j) . dS^T (T_j x T_i).
    ATTN_TRY(gemm(N_, N_, z.D, z.T, z.T, scale, at(kv.k, b * z.qe, 2), z.Hq * z.D, z.D,
                  at(ds, mo, 2), z.T, z.tt, 0.f, at(dq, b * z.qe, 2), Launch<E>::type,
                  z.Hq * z.D, z.D));
  }
  ATTN_TRY(from_hip(rca::unf::group_sum<E>(dkh, dk, z.B, z.T, z.Hkv, z.G, z.D, st)));
  return from_hip(rca::unf::group_sum<E>(dvh, dv, z.B, z.T, z.Hkv, z.G, z.D, st));
}

attn_status_t bind(attn_unfused_ctx* ctx, void* stream) {
  if (rocblas_set_stream(ctx->blas, static_cast<hipStream_t>(stream)) != rocblas_status_success)
    return ATTN_ERR_HIP;
  (void)hipGetLastError();  // discard an error left by an earlier, unrelated call
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT attn_status_t attn_unfused_create(attn_unfused_ctx** ctx) {
  if (ctx == nullptr) return ATTN_ERR_INVALID_ARG;
  *ctx = nullptr;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return ATTN_ERR_HIP;
  if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
    rocblas_destroy_handle(h);
    return ATTN_ERR_HIP;
  }
  *ctx = new attn_unfused_ctx{h};
  return ATTN_OK;
}

ATTN_EXPORT void attn_unfused_destroy(attn_unfused_ctx* ctx) {
  if (ctx == nullptr) return;
  rocblas_destroy_handle(ctx->blas);
  delete ctx;
}

ATTN_EXPORT size_t attn_unfused_workspace_bytes(int B, int T, int Hq, int Hkv, int D,
                                                attn_dtype_t dtype) {
  if (check_shape(B, T, Hq, Hkv, D, dtype) != ATTN_OK) return 0;
  return layout(B, T, Hq, D).total;
}

ATTN_EXPORT attn_status_t attn_unfused_fwd(attn_unfused_ctx* ctx, const void* q, const void* k,
                                           const void* v, void* o, float* lse, int B, int T,
                                           int Hq, int Hkv, int D, float scale, int causal,
                                           attn_dtype_t dtype, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (ctx == nullptr) return ATTN_ERR_INVALID_ARG;
  ATTN_TRY(check_ptrs({q, k, v, o, lse, workspace}));
  ATTN_TRY(check_shape(B, T, Hq, Hkv, D, dtype));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t need = layout(B, T, Hq, D).total;
  if (workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * T * Hq * D * 2, kb = (size_t)B * T * Hkv * D * 2;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb)},
                          {span_of(o, qb), span_of(lse, lb), span_of(workspace, need)}));
  ATTN_TRY(bind(ctx, stream));
  const Shape z(B, T, Hq, Hkv, D);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  return dtype == ATTN_BF16
             ? run_fwd<rca::Bf16>(ctx->blas, z, q, k, v, o, lse, scale, causal, ws, st)
             : run_fwd<rca::F16>(ctx->blas, z, q, k, v, o, lse, scale, causal, ws, st);
}

ATTN_EXPORT attn_status_t attn_unfused_bwd(attn_unfused_ctx* ctx, const void* q, const void* k,
                                           const void* v, const float* lse, const void* dO,
                                           void* dq, void* dk, void* dv, int B, int T, int Hq,
                                           int Hkv, int D, float scale, int causal,
                                           attn_dtype_t dtype, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (ctx == nullptr) return ATTN_ERR_INVALID_ARG;
  ATTN_TRY(check_ptrs({q, k, v, lse, dO, dq, dk, dv, workspace}));
  ATTN_TRY(check_shape(B, T, Hq, Hkv, D, dtype));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t need = layout(B, T, Hq, D).total;
  if (workspace_bytes < need) return ATTN_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * T * Hq * D * 2, kb = (size_t)B * T * Hkv * D * 2;
  const size_t lb = (size_t)B * Hq * T * sizeof(float);
  ATTN_TRY(check_disjoint({span_of(q, qb), span_of(k, kb), span_of(v, kb), span_of(lse, lb),
                           span_of(dO, qb)},
                          {span_of(dq, qb), span_of(dk, kb), span_of(dv, kb),
                           span_of(workspace, need)}));
  ATTN_TRY(bind(ctx, stream));
  const Shape z(B, T, Hq, Hkv, D);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  return dtype == ATTN_BF16
             ? run_bwd<rca::Bf16>(ctx->blas, z, q, k, v, lse, dO, dq, dk, dv, scale, causal, ws, st)
             : run_bwd<rca::F16>(ctx->blas, z, q, k, v, lse, dO, dq, dk, dv, scale, causal, ws, st);
}

namespace {

attn_status_t check_rows(long long n_rows, int T, attn_dtype_t dtype) {
  if (n_rows <= 0 || T <= 0 || T > kMaxT || n_rows % T != 0) return ATTN_ERR_INVALID_ARG;
  if (n_rows * (long long)T * 4 >= kMaxMatrixBytes) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT attn_status_t attn_unfused_softmax_lse(const float* s, void* p, float* lse,
                                                   long long n_rows, int T, float scale,
                                                   int causal, attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({s, p, lse}));
  ATTN_TRY(check_rows(n_rows, T, dtype));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t n = (size_t)n_rows * T;
  ATTN_TRY(check_disjoint({span_of(s, 4 * n)}, {span_of(p, 2 * n), span_of(lse, 4 * (size_t)n_rows)}));
  (void)hipGetLastError();
  const float sl2 = (float)((double)scale * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16 ? rca::unf::softmax_lse<rca::Bf16>(s, p, lse, n_rows, T, sl2, causal, st)
                                     : rca::unf::softmax_lse<rca::F16>(s, p, lse, n_rows, T, sl2, causal, st));
}

ATTN_EXPORT attn_status_t attn_unfused_probs_from_lse(const float* s, const float* lse, void* p,
                                                      long long n_rows, int T, float scale,
                                                      int causal, attn_dtype_t dtype,
                                                      void* stream) {
  ATTN_TRY(check_ptrs({s, lse, p}));
  ATTN_TRY(check_rows(n_rows, T, dtype));
  ATTN_TRY(check_scalars(scale, causal));
  const size_t n = (size_t)n_rows * T;
  ATTN_TRY(check_disjoint({span_of(s, 4 * n), span_of(lse, 4 * (size_t)n_rows)}, {span_of(p, 2 * n)}));
  (void)hipGetLastError();
  const float sl2 = (float)((double)scale * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16 ? rca::unf::probs_from_lse<rca::Bf16>(s, lse, p, n_rows, T, sl2, causal, st)
                                     : rca::unf::probs_from_lse<rca::F16>(s, lse, p, n_rows, T, sl2, causal, st));
}

ATTN_EXPORT attn_status_t attn_unfused_softmax_bwd(const void* p, const float* dp, void* ds,
                                                   long long n_rows, int T, int causal,
                                                   attn_dtype_t dtype, void* stream) {
  ATTN_TRY(check_ptrs({p, dp, ds}));
  ATTN_TRY(check_rows(n_rows, T, dtype));
  ATTN_TRY(check_scalars(1.f, causal));
  const size_t n = (size_t)n_rows * T;
  ATTN_TRY(check_disjoint({span_of(p, 2 * n), span_of(dp, 4 * n)}, {span_of(ds, 2 * n)}));
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16 ? rca::unf::softmax_bwd<rca::Bf16>(p, dp, ds, n_rows, T, causal, st)
                                     : rca::unf::softmax_bwd<rca::F16>(p, dp, ds, n_rows, T, causal, st));
}
