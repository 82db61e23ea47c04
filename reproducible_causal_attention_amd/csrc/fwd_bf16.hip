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
// Decomposition (MI355X-first, not the page's Ampere design):
//   * a workgroup of 8 waves owns 128 query rows of one (batch, query head):
//     four 32-row query blocks times two key halves;
//   * key/value tiles of 64 rows (128 when the grid fits the
//     GPU in one round: half the barriers) are staged row-major in LDS (pitch
//     72 bf16, so 16-byte column reads of 32 consecutive rows hit distinct
//     banks) and double-buffered; wave (qb, kh) runs an online softmax over the
//     32-key blocks kh, kh + 2, kh + 4, ... (keys 64j + 32kh .. +31 of each
//     64-key half of a tile), so each K/V row in LDS feeds four waves and the
//     tile size does not change the result;
//   * the wave computes S^T = K Q^T (keys x queries) with 32x32x16 bf16 MFMA, so
//     every lane holds one query's scores: the row max and row sum need a single
//     half-wave exchange (v_permlane32_swap), and O^T += V^T P^T takes the
//     probabilities straight from the accumulators (packed to bf16, round to
//     nearest even) with V^T read from the row-major tile by ds_read_b64_tr_b16;
//   * the running max moves lazily (only when a row's maximum grew by more than
//     2^8), so the output rescale runs a few times per row instead of per tile;
//     the row sums are accumulated from the packed bf16 probabilities with
//     v_dot2c_f32_bf16;
//   * scores are kept in base-2 units (scale * log2 e folded in) so every
//     exponential is one v_exp_f32;
//   * the two key halves' states (max, sum, O) are merged in a fixed order;
//   * query tiles are issued heaviest first, and the tiles of one
//     (batch, KV head) group run on one XCD so they share its L2.
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int BM = 128;    // query rows per workgroup
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr float kSlack = 8.0f;   // lazy-rescale threshold, base-2 units

// Head-dimension dependent sizes (kD = 64 or 128).
template <int kD, int kBN>
struct Dims {
  static constexpr int BN = kBN;                 // key rows per LDS tile (64 or 128)
  static constexpr int NB = BN / 64;             // 32-key blocks per wave per tile
  static constexpr int PITCH = kD + 8;           // LDS row pitch in elements (144 / 272 bytes)
  static constexpr int TILE = BN * PITCH;        // one K or V tile
  static constexpr int PART_STRIDE = kD / 2 + 4;  // floats per lane in the merge buffer (O, m, l)
  static constexpr int NQ = kD / 16;             // 16-wide chunks of d: MFMA k-steps of S
  static constexpr int ND = kD / 32;             // 32-row blocks of O^T
  static constexpr int NL = kD / 64;             // 16-byte tile loads per thread per tensor
  static_assert(4 * 64 * PART_STRIDE * 4 <= 4 * TILE * 2, "merge buffer must fit");
};

// kRope: q and k are rotated as they are loaded (rotary tables rcos, rsin:
// [T, kD/2] float32, pair i of position t at t*kD/2 + i), v is not.
// kBN: key rows per LDS tile.  With 128 each wave takes two 32-key blocks of a
// tile (the same blocks in the same order as with 64, so the same bits) and
// meets half the barriers; it pays off where a grid fits the GPU in one round
// and is used there without rotary positions (whose second row of tables would
// cost the second 64-wide workgroup per CU).
template <bool kPosScale, class E, bool kRope, int kD, int kBN>
__global__ __launch_bounds__(NTHREADS) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ o,
    float* __restrict__ lse, int B, int T, int Hq, int Hkv, float scale_log2, int causal) {
  using Dm = Dims<kD, kBN>;
  constexpr int PITCH = Dm::PITCH, TILE = Dm::TILE, NQ = Dm::NQ, ND = Dm::ND, NL = Dm::NL;
  constexpr int BN = Dm::BN, NB = Dm::NB;
  constexpr uint32_t kHalf = kD / 2;  // rotary pairs per row
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int qb = wave & 3;
  const int kh = wave >> 2;

  const int G = Hq / Hkv;
  const int n_qt = (T + BM - 1) / BM;
  int gi, rank;
  // Two 64-wide workgroups fit a CU (the paired order assumes it); one 128-wide.
  if (kD == 64)
    decode_unit_paired(blockIdx.x, gridDim.x, B * Hkv, gi, rank);
  else
    decode_unit(blockIdx.x, B * Hkv, gi, rank);
  const int b = gi / Hkv;
  const int kvh = gi - b * Hkv;
  const int hh = rank % G;
  const int qt = causal ? n_qt - 1 - rank / G : rank / G;  // heaviest tiles first
  const int h = kvh * G + hh;

  // Per-batch-element buffers; byte offsets below are within one batch element.
  const uint32_t q_row = (uint32_t)Hq * kD * 2;   // bytes between tokens of q / o
  const uint32_t kv_row = (uint32_t)Hkv * kD * 2;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * kD, ke = (size_t)T * Hkv * kD;
  const rsrc_t rk = make_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rv = make_rsrc(v + b * ke, (uint32_t)T * kv_row);

  const int qw0 = qt * BM + 32 * qb;  // first query row of this wave
  const int my_q = qw0 + l32;         // the query row this lane accumulates
  const uint32_t qoff = (uint32_t)my_q * q_row + (uint32_t)h * kD * 2;  // bytes

  // Q^T as the B operand of S^T = K Q^T: lane holds query my_q, d = 16s + 8g + [0, 8).
  const rsrc_t rq = make_rsrc(q + b * qe, (uint32_t)T * q_row);
  const rsrc_t ro = make_rsrc(o + b * qe, (uint32_t)T * q_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  u32x4_t qf[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) qf[s] = bload16(rq, qoff + 32 * s + 16 * g);
  // Rotary tables (rows past the sequence end read as zero, like their q and k rows).
  const rsrc_t rtc = make_rsrc(rcos, kRope ? (uint32_t)T * kHalf * 4u : 0u);
  const rsrc_t rts = make_rsrc(rsin, kRope ? (uint32_t)T * kHalf * 4u : 0u);
  u32x4_t qc[NQ], qsn[NQ];
  if (kRope) {  // lane's pairs of chunk s: i = 8s + 4g + 0..3 of row my_q
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      qc[s] = bload16(rtc, ((uint32_t)my_q * kHalf + 8 * s + 4 * g) * 4);
      qsn[s] = bload16(rts, ((uint32_t)my_q * kHalf + 8 * s + 4 * g) * 4);
    }
  }
  // Tile loads: thread -> rows ld_row + 64rr for rr < NB, columns ld_col + 64c + 0..7
  // for c < NL.
  const int ld_row = tid >> 3, ld_col = (tid & 7) * 8;
  const uint32_t ld_off = (uint32_t)ld_row * kv_row + (uint32_t)kvh * kD * 2 + 2 * ld_col;
  u32x4_t kreg[NB][NL], vreg[NB][NL], kc[NB][NL], ksn[NB][NL];
  // Loads of tile kt; rows past the sequence end read as zero, and with
  // present == false every access is out of range (zeros, no memory traffic).
  auto gload_tile = [&](int kt, bool present = true) {
#pragma unroll
    for (int rr = 0; rr < NB; ++rr) {
      const uint32_t off = present ? ld_off + (uint32_t)(kt * BN + 64 * rr) * kv_row : 0x80000000u;
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        kreg[rr][c] = bload16(rk, off + 128 * c);
        vreg[rr][c] = bload16(rv, off + 128 * c);
      }
      if (kRope) {  // pairs ld_col/2 + 32c + 0..3 of key row kt*BN + 64rr + ld_row
        const uint32_t toff =
            present ? ((uint32_t)(kt * BN + 64 * rr + ld_row) * kHalf + ld_col / 2) * 4 : 0x80000000u;
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          kc[rr][c] = bload16(rtc, toff + 128 * c);
          ksn[rr][c] = bload16(rts, toff + 128 * c);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < NB; ++rr) {
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        if (kRope) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            kreg[rr][c][e] = rope_rotate<E>(kreg[rr][c][e], bits_to_float(kc[rr][c][e]),
                                            bits_to_float(ksn[rr][c][e]));
        }
        const int at = (ld_row + 64 * rr) * PITCH + ld_col + 64 * c;
        lds_store16(smem + (2 * buf) * TILE + at, kreg[rr][c]);
        lds_store16(smem + (2 * buf + 1) * TILE + at, vreg[rr][c]);
      }
    }
  };

  gload_tile(0);  // in flight together with the Q rows
  wait_loads();
  if (kRope) {
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qf[s][e] = rope_rotate<E>(qf[s][e], bits_to_float(qc[s][e]), bits_to_float(qsn[s][e]));
    }
  }

  f32x16_t oacc[ND];  // O^T: rows d = 32*db + 8*(r/4) + 4g + r%4
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = zero16();
  float m_run = -1e30f;                     // running max (base-2 units)
  float l_run = 0.f;                        // this lane's share of the running sum

  const int kv_end = causal ? min(T, (qt + 1) * BM) : T;
  const int n_kv = (kv_end + BN - 1) / BN;

  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_kv; ++kt) {
    const int cur = kt & 1;
    // The next tile's loads overlap this tile's math; after the last tile they are
    // empty and its store fills the unused buffer with zeros, so neither needs a
    // branch that would split the loop body's scheduling regions.
    gload_tile(kt + 1, kt + 1 < n_kv);
    const uint16_t* sK = smem + (2 * cur) * TILE;
    const uint16_t* sV = smem + (2 * cur + 1) * TILE;
    // Wave kh takes keys 64sb + 32kh .. +31 of the tile, so over the tiles it
    // visits the 32-key blocks kh, kh + 2, kh + 4, ... in order.
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      const int krow = 64 * sb + 32 * kh;  // first tile row of this 32-key block
      const int kb0 = kt * BN + krow;
      const bool active = kb0 < T && (!causal || kb0 <= qw0 + 31);
      if (active) {
        f32x16_t sacc = zero16();
#pragma unroll
        for (int s = 0; s < NQ; ++s)
          sacc = E::mfma(lds_load16(sK + (krow + l32) * PITCH + 16 * s + 8 * g), qf[s], sacc);
        // Register r holds key kb0 + 8*(r/4) + 4g + r%4 against query my_q.  The
        // tile maximum is taken over the raw scores (the scale is positive; for a
        // negative scale the minimum) and scaled once.
        const bool edge = (causal && kb0 + 31 > qw0) || kb0 + 32 > T;
        bool keep[16];
        float mraw;
        if (edge) {
          // Diagonal tile or sequence tail: keys after the query or past the end
          // take no part in the maximum and get probability 0.
          mraw = kPosScale ? -__builtin_inff() : __builtin_inff();
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 8 * (r >> 2) + 4 * g + (r & 3);
            keep[r] = !((causal && key > my_q) || key >= T);
            const float x = keep[r] ? sacc[r] : (kPosScale ? -__builtin_inff() : __builtin_inff());
            mraw = kPosScale ? fmaxf(mraw, x) : fminf(mraw, x);
          }
        } else {
          mraw = sacc[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mraw = kPosScale ? fmaxf(mraw, sacc[r]) : fminf(mraw, sacc[r]);
        }
        const float mx = halves_max(mraw * scale_log2);
        // Lazy rescale: the running max only moves when some row's maximum grew by
        // more than kSlack (base-2 units), so probabilities stay below 2^kSlack
        // (exact in bf16 and fp32) and O is rescaled a few times per row, not per tile.
        const float m_cand = fmaxf(m_run, mx);
        if (__any(m_cand > m_run + kSlack)) {
          const float alpha = fast_exp2(m_run - m_cand);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < ND; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          }
          m_run = m_cand;
        }
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[r], scale_log2, -m_run));
            sacc[r] = keep[r] ? p : 0.f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], scale_log2, -m_run));
        }
        const u32x4_t pb0 = pack_operand_e<E>(sacc, 0), pb1 = pack_operand_e<E>(sacc, 8);
        // Row sum of the bf16 probabilities that enter O (two per v_dot2c_f32_bf16).
#pragma unroll
        for (int i = 0; i < 4; ++i) l_run = E::add_pair(pb1[i], E::add_pair(pb0[i], l_run));
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          oacc[db] = E::mfma(lds_operand_T(sV, PITCH, krow, 32 * db, lane), pb0, oacc[db]);
          oacc[db] = E::mfma(lds_operand_T(sV, PITCH, krow + 16, 32 * db, lane), pb1, oacc[db]);
        }
      }
    }
    store_tile(cur ^ 1);
    __syncthreads();
  }

  // Merge the key halves: (m, l, O) of half 1 into half 0, in that order.
  float* part = reinterpret_cast<float*>(smem);
  float* slot = part + (qb * 64 + lane) * Dm::PART_STRIDE;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        *reinterpret_cast<float4*>(slot + 16 * db + r) =
            make_float4(oacc[db][r], oacc[db][r + 1], oacc[db][r + 2], oacc[db][r + 3]);
    }
    slot[kD / 2] = m_run;
    slot[kD / 2 + 1] = l_run;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = slot[kD / 2], l1 = slot[kD / 2 + 1];
    const float m = fmaxf(m_run, m1);
    const float a0 = fast_exp2(m_run - m), a1 = fast_exp2(m1 - m);
    const float l_tot = halves_sum(l_run * a0 + l1 * a1);
    // Rows past the sequence end are dropped by the buffer range check.
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = *reinterpret_cast<const float4*>(slot + 16 * db + 4 * j);
        u32x2_t w;
        w[0] = E::pack2((oacc[db][4 * j + 0] * a0 + x.x * a1) * inv,
                           (oacc[db][4 * j + 1] * a0 + x.y * a1) * inv);
        w[1] = E::pack2((oacc[db][4 * j + 2] * a0 + x.z * a1) * inv,
                           (oacc[db][4 * j + 3] * a0 + x.w * a1) * inv);
        bstore8(ro, qoff + 2 * (32 * db + 8 * j + 4 * g), w);
      }
    }
    if (g == 0 && my_q < T) bstore_f32(rl, ((uint32_t)h * T + my_q) * 4, (m + fast_log2(l_tot)) * kLn2);
  }
}

}  // namespace

const char* fwd_bf16_tiles() {
  return "fwd_bf16{BM=128,BN=64|128(grids<=512),waves=8(4 query x 2 key),mfma=32x32x16,D=64|128}";
}

template <class E, bool kRope>
hipError_t launch_fwd_e(const Problem& p, const void* q, const void* k, const void* v,
                        const float* rcos, const float* rsin, void* o, float* lse, hipStream_t s) {
  const int n_qt = (p.T + BM - 1) / BM;
  const dim3 grid((unsigned)(n_qt * p.B * p.Hq));
  const bool pos = p.scale_log2 >= 0.f;
  auto kernel = p.D == 128 ? (pos ? attn_fwd_kernel<true, E, kRope, 128, 64>
                                  : attn_fwd_kernel<false, E, kRope, 128, 64>)
                           : (pos ? attn_fwd_kernel<true, E, kRope, 64, 64>
                                  : attn_fwd_kernel<false, E, kRope, 64, 64>);
  if constexpr (!kRope) {
    if (p.D == 64 && grid.x <= 512)  // the grid fits the GPU in one round
      kernel = pos ? attn_fwd_kernel<true, E, false, 64, 128> : attn_fwd_kernel<false, E, false, 64, 128>;
    if (p.D == 128 && grid.x <= 512)
      kernel = pos ? attn_fwd_kernel<true, E, false, 128, 128> : attn_fwd_kernel<false, E, false, 128, 128>;
  }
  kernel<<<grid, NTHREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), rcos, rsin, static_cast<uint16_t*>(o), lse, p.B, p.T, p.Hq,
      p.Hkv, p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_fwd_rope_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* rcos, const float* rsin, void* o, float* lse,
                                hipStream_t s) {
  return launch_fwd_e<Bf16, true>(p, q, k, v, rcos, rsin, o, lse, s);
}

hipError_t launch_fwd_rope_f16(const Problem& p, const void* q, const void* k, const void* v,
                               const float* rcos, const float* rsin, void* o, float* lse,
                               hipStream_t s) {
  return launch_fwd_e<F16, true>(p, q, k, v, rcos, rsin, o, lse, s);
}

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, hipStream_t s) {
  if (p.D == 64) return launch_fwd64_bf16(p, q, k, v, o, lse, s);
  return launch_fwd_e<Bf16, false>(p, q, k, v, nullptr, nullptr, o, lse, s);
}

hipError_t launch_fwd_f16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, hipStream_t s) {
  if (p.D == 64) return launch_fwd64_f16(p, q, k, v, o, lse, s);
  return launch_fwd_e<F16, false>(p, q, k, v, nullptr, nullptr, o, lse, s);
}

}  // namespace rca
