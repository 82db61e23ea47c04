// fwd_bf16.hip -- fused causal attention forward for bf16 on gfx950 MFMA.
//
// This is the fused flash-attention forward of "Training a 100M transformer in
// pure Rust: RustingBrain vs PyTorch and TensorFlow", section "Step 2: fused
// flash attention": the [seq_len, seq_len] score matrix that section "Step 1:
// measure before changing anything" found written and read back by the unfused
// causal_softmax_lse kernel never leaves registers.  The per-row log-sum-exp is
// written instead, so the backward can recompute probabilities from it (that
// page's causal_probs_from_lse).
//
// Work decomposition (MI355X-first, not the page's Ampere design):
//   * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//     each wave owns 32 query rows for the whole kernel;
//   * key/value tiles of 64 rows are staged row-major in LDS (pitch 72 bf16,
//     so 16-byte column reads of 32 consecutive rows hit distinct banks);
//   * the wave computes S^T = K Q^T (keys x queries) with 32x32x16 bf16 MFMA, so
//     every lane holds one query's scores: the row max and row sum need a single
//     half-wave exchange (v_permlane32_swap), and the O^T = V^T P^T product takes
//     the probabilities straight from the accumulators (packed to bf16, round to
//     nearest even) with V^T read from the row-major tile by ds_read_b64_tr_b16;
//   * scores are kept in base-2 units (scale * log2 e folded in) so every
//     exponential is one v_exp_f32;
//   * query tiles are issued heaviest first (the causal loop length grows with
//     the tile index).
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int BM = 128;     // query rows per workgroup
constexpr int BN = 64;      // key rows per LDS tile
constexpr int PITCH = 72;   // LDS row pitch in bf16 elements (144 bytes)
constexpr int NTHREADS = 256;

__global__ __launch_bounds__(NTHREADS) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int T, int Hq, int Hkv,
    float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int n_qt = (T + BM - 1) / BM;
  const int BH = B * Hq;
  int qt = blockIdx.x / BH;
  const int bh = blockIdx.x - qt * BH;
  if (causal) qt = n_qt - 1 - qt;  // heaviest query tiles first
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);

  const size_t q_stride = (size_t)Hq * kHeadDim;   // elements between tokens of q / o
  const size_t kv_stride = (size_t)Hkv * kHeadDim;  // elements between tokens of k / v
  const uint16_t* qbase = q + ((size_t)b * T * Hq + h) * kHeadDim;
  const uint16_t* kbase = k + ((size_t)b * T * Hkv + kvh) * kHeadDim;
  const uint16_t* vbase = v + ((size_t)b * T * Hkv + kvh) * kHeadDim;

  const int qw0 = qt * BM + wave * 32;  // first query row of this wave
  const int my_q = qw0 + l32;           // the query row this lane accumulates

  // Q^T as the B operand of S^T = K Q^T: lane holds query my_q, d = 16s + 8g + [0, 8).
  u32x4_t qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qf[s] = my_q < T ? gload16(qbase + (size_t)my_q * q_stride + 16 * s + 8 * g) : zero4u();

  f32x16_t oacc[2] = {zero16(), zero16()};  // O^T: rows d = 32*db + 8*(r/4) + 4g + r%4
  float m_run = -1e30f;                     // running max (base-2 units)
  float l_run = 0.f;                        // this lane's share of the running sum

  const int kv_end = causal ? min(T, (qt + 1) * BM) : T;
  const int n_kv = (kv_end + BN - 1) / BN;

  // Cooperative tile load: 64 rows x 8 chunks of 16 bytes per tensor, two chunks
  // of each tensor per thread; a wave instruction covers 8 whole rows.
  u32x4_t kreg[2], vreg[2];
  auto gload_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + NTHREADS * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int key = kt * BN + row;
      kreg[i] = key < T ? gload16(kbase + (size_t)key * kv_stride + col) : zero4u();
      vreg[i] = key < T ? gload16(vbase + (size_t)key * kv_stride + col) : zero4u();
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + NTHREADS * i;
      const int row = c >> 3, col = (c & 7) * 8;
      lds_store16(sK + row * PITCH + col, kreg[i]);
      lds_store16(sV + row * PITCH + col, vreg[i]);
    }
  };

  gload_tile(0);
  store_tile();
  __syncthreads();

  for (int kt = 0; kt < n_kv; ++kt) {
    if (kt + 1 < n_kv) gload_tile(kt + 1);  // next tile's loads overlap this tile's math
    const int k0 = kt * BN;
    const bool active = !causal || k0 <= qw0 + 31;
    if (active) {
      // S^T (64 keys x 32 queries) as two 32x32 blocks.
      f32x16_t sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4_t a = lds_load16(sK + (32 * mb + l32) * PITCH + 16 * s + 8 * g);
          sacc[mb] = mfma_32x32x16(a, qf[s], sacc[mb]);
        }
      }
      const bool need_mask = (causal && k0 + BN - 1 > qw0) || (k0 + BN > T);
      float mx = -__builtin_inff();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = sacc[mb][r] * scale_log2;
          if (need_mask) {
            const int key = k0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((causal && key > my_q) || key >= T) sv = -__builtin_inff();
          }
          sacc[mb][r] = sv;
          mx = fmaxf(mx, sv);
        }
      }
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[mb][r] - m_new);
          sacc[mb][r] = p;
          rs += p;
        }
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      // O^T += V^T P^T over the four 16-key steps of the tile.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t pb = pack_operand(sacc[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const u32x4_t a = lds_operand_T(sV, PITCH, 16 * ks, 32 * db, lane);
          oacc[db] = mfma_32x32x16(a, pb, oacc[db]);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < n_kv) {
      store_tile();
      __syncthreads();
    }
  }

  const float l_tot = halves_sum(l_run);
  if (my_q < T) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = o + ((size_t)b * T + my_q) * q_stride + (size_t)h * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2_t w;
        w[0] = pack_bf16x2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + 32 * db + 8 * j + 4 * g) = w;
      }
    }
    if (g == 0) lse[((size_t)b * Hq + h) * T + my_q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace

const char* fwd_bf16_tiles() {
  return "fwd_bf16{BM=128,BN=64,waves=4,mfma=32x32x16}";
}

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, hipStream_t s) {
  const int n_qt = (p.T + BM - 1) / BM;
  const dim3 grid((unsigned)(n_qt * p.B * p.Hq));
  attn_fwd_bf16_kernel<<<grid, NTHREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, p.B, p.T, p.Hq, p.Hkv,
      p.scale_log2, p.causal);
  return hipGetLastError();
}

}  // namespace rca
