// bwd_bf16.hip -- fused causal attention backward for bf16 on gfx950 MFMA.
//
// The backward of the fused flash attention of "Training a 100M transformer in
// pure Rust: RustingBrain vs PyTorch and TensorFlow", section "Step 2: fused
// flash attention", in three deterministic steps:
//   1. preprocess: delta_i = <dO_i, o_i> (the row term of the softmax backward
//      that the unfused causal_softmax_bwd of section "Step 1" needs);
//   2. dK/dV: one workgroup per tile of keys of one KV head; it visits every
//      query head of the group and every query tile that can see its keys, in
//      a fixed order, recomputing P from the saved log-sum-exp (the page's
//      causal_probs_from_lse step), and writes dK, dV once -- the kernel the
//      page's section "Where the time goes now" names flash_attention_dkv;
//   3. dQ: one workgroup per tile of queries, visiting its key tiles in order.
// No step uses atomics ("rust-trainer", section "The trainer is not
// bit-identical to itself after step 1", traces lost bit identity to a
// gradient accumulated with atomics), so the results are bitwise reproducible.
//
// MFMA formulation (32x32x16 bf16, see cdna4.hpp for the register layouts):
//   dK/dV kernel, per 32-query block: S = Q K^T and dP = dO V^T with the keys on
//   the lanes; P and dS = P * (dP - delta) are packed straight from the
//   accumulators into B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//   operands (dO^T, Q^T) are transposed reads of the row-major LDS tiles.
//   dQ kernel, per 32-key block: S^T = K Q^T and dP^T = V dO^T with the queries
//   on the lanes; dS^T feeds dQ^T += K^T dS^T with K^T a transposed LDS read.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int PITCH = 72;  // LDS row pitch in bf16 elements (144 bytes)

// ---------------------------------------------------------------------------
// 1. preprocess: delta[b][h][i] = sum_d dO[b][i][h][d] * o[b][i][h][d]
// ---------------------------------------------------------------------------
constexpr int PRE_THREADS = 256;
constexpr int PRE_ROWS = PRE_THREADS / 8;  // 8 lanes x 8 elements per 64-wide row

__global__ __launch_bounds__(PRE_THREADS) void attn_bwd_pre_bf16_kernel(
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
      acc = fmaf(bf16_lo(a[i]), bf16_lo(c[i]), acc);
      acc = fmaf(bf16_hi(a[i]), bf16_hi(c[i]), acc);
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

// ---------------------------------------------------------------------------
// 2. dK / dV
// ---------------------------------------------------------------------------
constexpr int KV_BN = 128;  // keys per workgroup (4 waves x 32)
constexpr int KV_BM = 64;   // query rows per LDS step
constexpr int KV_THREADS = 256;

__global__ __launch_bounds__(KV_THREADS) void attn_bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv,
    float scale, float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[KV_BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[KV_BM * PITCH];
  __shared__ __attribute__((aligned(16))) float sL[KV_BM];  // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[KV_BM];  // delta

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int BG = B * Hkv;
  const int kt = blockIdx.x / BG;  // key tile 0 first: it sees the most queries
  const int bg = blockIdx.x - kt * BG;
  const int b = bg / Hkv;
  const int kvh = bg - b * Hkv;
  const int G = Hq / Hkv;

  const size_t q_stride = (size_t)Hq * kHeadDim;
  const size_t kv_stride = (size_t)Hkv * kHeadDim;

  const int kw0 = kt * KV_BN + wave * 32;  // first key of this wave
  const int my_key = kw0 + l32;

  // K^T and V^T as B operands (keys on the lanes): d = 16s + 8g + [0, 8).
  const uint16_t* krow = k + ((size_t)b * T * Hkv + kvh) * kHeadDim + (size_t)my_key * kv_stride;
  const uint16_t* vrow = v + ((size_t)b * T * Hkv + kvh) * kHeadDim + (size_t)my_key * kv_stride;
  u32x4_t kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s] = my_key < T ? gload16(krow + 16 * s + 8 * g) : zero4u();
    vf[s] = my_key < T ? gload16(vrow + 16 * s + 8 * g) : zero4u();
  }

  f32x16_t dk_acc[2] = {zero16(), zero16()};  // dK^T: rows d = 32*db + 8*(r/4) + 4g + r%4
  f32x16_t dv_acc[2] = {zero16(), zero16()};

  const int n_qt = (T + KV_BM - 1) / KV_BM;
  const int qt_begin = causal ? (kt * KV_BN) / KV_BM : 0;

  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const uint16_t* qbase = q + ((size_t)b * T * Hq + h) * kHeadDim;
    const uint16_t* dobase = dO + ((size_t)b * T * Hq + h) * kHeadDim;
    const float* lrow = lse + ((size_t)b * Hq + h) * T;
    const float* drow = delta + ((size_t)b * Hq + h) * T;
    for (int qt = qt_begin; qt < n_qt; ++qt) {
      const int q0 = qt * KV_BM;
      __syncthreads();  // previous step's LDS reads are done
      // Q and dO tiles: 64 rows x 8 chunks each; two chunks of each per thread.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + KV_THREADS * i;
        const int row = c >> 3, col = (c & 7) * 8;
        const int qi = q0 + row;
        const u32x4_t a = qi < T ? gload16(qbase + (size_t)qi * q_stride + col) : zero4u();
        const u32x4_t d = qi < T ? gload16(dobase + (size_t)qi * q_stride + col) : zero4u();
        lds_store16(sQ + row * PITCH + col, a);
        lds_store16(sdO + row * PITCH + col, d);
      }
      if (tid < KV_BM) {
        const int qi = q0 + tid;
        sL[tid] = qi < T ? lrow[qi] * kLog2e : 0.f;
        sD[tid] = qi < T ? drow[qi] : 0.f;
      }
      __syncthreads();

#pragma unroll
      for (int mq = 0; mq < KV_BM / 32; ++mq) {
        const int qm0 = q0 + 32 * mq;
        if (causal && kw0 > qm0 + 31) continue;  // every key of the wave is after every query
        f32x16_t sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4_t aq = lds_load16(sQ + (32 * mq + l32) * PITCH + 16 * s + 8 * g);
          const u32x4_t ad = lds_load16(sdO + (32 * mq + l32) * PITCH + 16 * s + 8 * g);
          sacc = mfma_32x32x16(aq, kf[s], sacc);
          pacc = mfma_32x32x16(ad, vf[s], pacc);
        }
        // Register r holds query qm0 + 8*(r/4) + 4g + r%4 for key my_key.
        const bool need_mask = (causal && kw0 + 31 > qm0) || (qm0 + 31 >= T);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qr = 32 * mq + 8 * j + 4 * g;  // row in the LDS tile
          const float4 L = *reinterpret_cast<const float4*>(sL + qr);
          const float4 Dl = *reinterpret_cast<const float4*>(sD + qr);
          const float Lr[4] = {L.x, L.y, L.z, L.w};
          const float Dr[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            float p = fast_exp2(sacc[r] * scale_log2 - Lr[e]);
            if (need_mask) {
              const int qi = q0 + qr + e;
              if ((causal && my_key > qi) || qi >= T) p = 0.f;
            }
            sacc[r] = p;
            pacc[r] = p * (pacc[r] - Dr[e]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4_t pb = pack_operand(sacc, 8 * ks);
          const u32x4_t sb = pack_operand(pacc, 8 * ks);
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const u32x4_t a_do = lds_operand_T(sdO, PITCH, 32 * mq + 16 * ks, 32 * db, lane);
            dv_acc[db] = mfma_32x32x16(a_do, pb, dv_acc[db]);
            const u32x4_t a_q = lds_operand_T(sQ, PITCH, 32 * mq + 16 * ks, 32 * db, lane);
            dk_acc[db] = mfma_32x32x16(a_q, sb, dk_acc[db]);
          }
        }
      }
    }
  }

  if (my_key < T) {
    const size_t off = ((size_t)b * T + my_key) * kv_stride + (size_t)kvh * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        u32x2_t wk, wv;
        wk[0] = pack_bf16x2(dk_acc[db][4 * j + 0] * scale, dk_acc[db][4 * j + 1] * scale);
        wk[1] = pack_bf16x2(dk_acc[db][4 * j + 2] * scale, dk_acc[db][4 * j + 3] * scale);
        wv[0] = pack_bf16x2(dv_acc[db][4 * j + 0], dv_acc[db][4 * j + 1]);
        wv[1] = pack_bf16x2(dv_acc[db][4 * j + 2], dv_acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2_t*>(dk + off + d) = wk;
        *reinterpret_cast<u32x2_t*>(dv + off + d) = wv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
constexpr int Q_BM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int Q_BN = 64;   // keys per LDS step
constexpr int Q_THREADS = 256;

__global__ __launch_bounds__(Q_THREADS) void attn_bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[Q_BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sV[Q_BN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int n_qt = (T + Q_BM - 1) / Q_BM;
  const int BH = B * Hq;
  int qt = blockIdx.x / BH;
  const int bh = blockIdx.x - qt * BH;
  if (causal) qt = n_qt - 1 - qt;  // heaviest query tiles first
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);

  const size_t q_stride = (size_t)Hq * kHeadDim;
  const size_t kv_stride = (size_t)Hkv * kHeadDim;
  const uint16_t* kbase = k + ((size_t)b * T * Hkv + kvh) * kHeadDim;
  const uint16_t* vbase = v + ((size_t)b * T * Hkv + kvh) * kHeadDim;

  const int qw0 = qt * Q_BM + wave * 32;
  const int my_q = qw0 + l32;
  const size_t qoff = ((size_t)b * T + my_q) * q_stride + (size_t)h * kHeadDim;

  // Q^T and dO^T as B operands (queries on the lanes).
  u32x4_t qf[4], df[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = my_q < T ? gload16(q + qoff + 16 * s + 8 * g) : zero4u();
    df[s] = my_q < T ? gload16(dO + qoff + 16 * s + 8 * g) : zero4u();
  }
  const float L2 = my_q < T ? lse[((size_t)b * Hq + h) * T + my_q] * kLog2e : 0.f;
  const float Dl = my_q < T ? delta[((size_t)b * Hq + h) * T + my_q] : 0.f;

  f32x16_t dq_acc[2] = {zero16(), zero16()};  // dQ^T: rows d = 32*db + 8*(r/4) + 4g + r%4

  const int kv_end = causal ? min(T, (qt + 1) * Q_BM) : T;
  const int n_kv = (kv_end + Q_BN - 1) / Q_BN;

  u32x4_t kreg[2], vreg[2];
  auto gload_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + Q_THREADS * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int key = kt * Q_BN + row;
      kreg[i] = key < T ? gload16(kbase + (size_t)key * kv_stride + col) : zero4u();
      vreg[i] = key < T ? gload16(vbase + (size_t)key * kv_stride + col) : zero4u();
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + Q_THREADS * i;
      const int row = c >> 3, col = (c & 7) * 8;
      lds_store16(sK + row * PITCH + col, kreg[i]);
      lds_store16(sV + row * PITCH + col, vreg[i]);
    }
  };

  gload_tile(0);
  store_tile();
  __syncthreads();

  for (int kt = 0; kt < n_kv; ++kt) {
    if (kt + 1 < n_kv) gload_tile(kt + 1);
    const int k0 = kt * Q_BN;
    const bool active = !causal || k0 <= qw0 + 31;
    if (active) {
      const bool need_mask = (causal && k0 + Q_BN - 1 > qw0) || (k0 + Q_BN > T);
      u32x4_t dsb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16_t sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4_t ak = lds_load16(sK + (32 * mb + l32) * PITCH + 16 * s + 8 * g);
          const u32x4_t av = lds_load16(sV + (32 * mb + l32) * PITCH + 16 * s + 8 * g);
          sacc = mfma_32x32x16(ak, qf[s], sacc);
          pacc = mfma_32x32x16(av, df[s], pacc);
        }
        // Register r holds key k0 + 32*mb + 8*(r/4) + 4g + r%4 for query my_q.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(sacc[r] * scale_log2 - L2);
          if (need_mask) {
            const int key = k0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((causal && key > my_q) || key >= T) p = 0.f;
          }
          pacc[r] = p * (pacc[r] - Dl);
        }
        dsb[2 * mb + 0] = pack_operand(pacc, 0);
        dsb[2 * mb + 1] = pack_operand(pacc, 8);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const u32x4_t a = lds_operand_T(sK, PITCH, 16 * ks, 32 * db, lane);
          dq_acc[db] = mfma_32x32x16(a, dsb[ks], dq_acc[db]);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < n_kv) {
      store_tile();
      __syncthreads();
    }
  }

  if (my_q < T) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2_t w;
        w[0] = pack_bf16x2(dq_acc[db][4 * j + 0] * scale, dq_acc[db][4 * j + 1] * scale);
        w[1] = pack_bf16x2(dq_acc[db][4 * j + 2] * scale, dq_acc[db][4 * j + 3] * scale);
        *reinterpret_cast<u32x2_t*>(dq + qoff + 32 * db + 8 * j + 4 * g) = w;
      }
    }
  }
}

}  // namespace

const char* bwd_bf16_tiles() {
  return "bwd_bf16{pre_rows=32,dkdv_BN=128,dkdv_BM=64,dq_BM=128,dq_BN=64,waves=4,mfma=32x32x16}";
}

hipError_t launch_bwd_pre_bf16(const Problem& p, const void* o, const void* dO, float* delta,
                               hipStream_t s) {
  const long long n_rows = (long long)p.B * p.T * p.Hq;
  const dim3 grid((unsigned)((n_rows + PRE_ROWS - 1) / PRE_ROWS));
  attn_bwd_pre_bf16_kernel<<<grid, PRE_THREADS, 0, s>>>(
      static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), delta, p.T, p.Hq, n_rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s) {
  const int n_kt = (p.T + KV_BN - 1) / KV_BN;
  const dim3 grid((unsigned)(n_kt * p.B * p.Hkv));
  attn_bwd_dkdv_bf16_kernel<<<grid, KV_THREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), p.B, p.T, p.Hq, p.Hkv, p.scale,
      p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dO, const float* lse, const float* delta, void* dq,
                              hipStream_t s) {
  const int n_qt = (p.T + Q_BM - 1) / Q_BM;
  const dim3 grid((unsigned)(n_qt * p.B * p.Hq));
  attn_bwd_dq_bf16_kernel<<<grid, Q_THREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta,
      static_cast<uint16_t*>(dq), p.B, p.T, p.Hq, p.Hkv, p.scale, p.scale_log2, p.causal);
  return hipGetLastError();
}

}  // namespace rca
