// dq_body.hpp -- dQ of fused causal attention, bf16 on gfx950 MFMA.
//
// For a block of query rows, recompute P from the saved log-sum-exp (the
// causal_probs_from_lse step of "Training a 100M transformer in pure Rust:
// RustingBrain vs PyTorch and TensorFlow", section "Step 1: measure before
// changing anything"), form dS = P * (dP - delta) and accumulate
// dQ = scale * sum_j dS_ij k_j over the keys the rows can see.  dQ has one owner
// per row, so there are no atomics and the sum order is fixed.
//
// Decomposition (MI355X-first):
//   * a workgroup of 8 waves owns 128 query rows of one (batch, query head):
//     four 32-row query blocks times two key halves;
//   * key/value tiles of 128 rows (64 for 128-wide heads) go straight from HBM
//     into double-buffered LDS (buffer_load ... lds, eight whole rows per
//     instruction, XOR-swizzled 16-byte chunks; the next tile's copy is in
//     flight while the current one is used); wave (query block qb, key half kh)
//     uses the kh-th half of each tile in blocks of 32 keys, so every K/V row in
//     LDS feeds four waves;
//   * S^T = K Q^T and dP^T = V dO^T put the queries on the lanes, so lse and
//     delta are one register per lane, the dP accumulator starts at -delta
//     (the MFMA adds dO.v to it), and dS^T feeds dQ^T += K^T dS^T directly from
//     the accumulators with K^T read by ds_read_b64_tr_b16;
//   * the two key halves' fp32 partials are added in a fixed order through LDS;
//   * query tiles are issued heaviest first, and the tiles of one
//     (batch, KV head) group run on one XCD so they share its L2;
//   * for 64-wide heads a unit's q and dO rows, lse, delta and first K/V tile
//     reach LDS by load-to-LDS copies (each row copied once, not once per key
//     half into registers), and a workgroup that runs several units issues the
//     next unit's copies into a second LDS slot while the current unit is still
//     computing, so the next unit starts on data already in LDS.
#pragma once

#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace dqb {

constexpr int BM = 128;  // query rows per workgroup
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;

// Sizes for head dim kD.  A K or V tile of BN keys is kD/64 column halves one
// after the other, each BN swizzled rows of 64 elements; wave (qb, kh) takes
// keys kh*BN/2 .. +BN/2-1 of every tile as NB blocks of 32.  64-wide heads use
// 128-key tiles (half the tiles and barriers per key); 128-wide heads, whose
// registers are full, 64-key tiles.
//
// 64-wide heads (STAGED) keep a unit in an LDS slot: K/V buffers 0 and 1, then
// lse and delta of the 128 rows.  Before the loop the q and dO rows sit in
// buffer 1 (the loop refills it only after they have been read into
// registers).  A workgroup running a list of units alternates between two
// slots and fills the next unit's slot during the current unit's last tiles.
// 128-wide heads (whose rows do not fit one buffer) load the rows into
// registers and use one slot.
template <int kD>
struct Dims {
  static constexpr int BN = kD == 64 ? 128 : 64;
  static constexpr int NB = BN / 64;                 // 32-key blocks per wave per tile
  static constexpr int HALF_BYTES = BN * 128;
  static constexpr int TILE_BYTES = (kD / 64) * HALF_BYTES;
  static constexpr int NQ = kD / 16, ND = kD / 32, NH = kD / 64;
  static constexpr bool STAGED = kD == 64;
  static constexpr int STAT_OFF = 4 * TILE_BYTES;             // [buffer][K, V], then statistics
  static constexpr int SLOT_BYTES = STAT_OFF + (STAGED ? 2 * BM * 4 : 0);
  static constexpr int SMEM_BYTES = SLOT_BYTES;                    // one unit per workgroup
  static constexpr int SMEM2_BYTES = (STAGED ? 2 : 1) * SLOT_BYTES;  // a list of units
  static constexpr int STAGE_COPIES = 8;  // load-to-LDS rows and tile copies per wave (+1 for waves 0-3)
  static_assert(4 * (4 * ND) * 64 * 16 <= STAT_OFF, "reduction buffer must fit");
  static_assert(!STAGED || 2 * BM * kD * 2 == 2 * TILE_BYTES, "q and dO rows fill K/V buffer 1");
};

// Where unit `unit` lies: batch element b, KV head kvh, query head h, query tile
// qt, and the number of K/V tiles its rows see.
struct UnitPos {
  int b, kvh, h, qt, n_kv;
};
template <int kD>
__device__ __forceinline__ UnitPos unit_pos(int unit, int B, int T, int Hq, int Hkv, int causal) {
  const int G = Hq / Hkv;
  const int n_qt = (T + BM - 1) / BM;
  int gi, rank;
  decode_unit(unit, B * Hkv, gi, rank);
  UnitPos u;
  u.b = gi / Hkv;
  u.kvh = gi - u.b * Hkv;
  u.qt = causal ? n_qt - 1 - rank / G : rank / G;  // heaviest tiles first
  u.h = u.kvh * G + rank % G;
  const int kv_end = causal ? min(T, (u.qt + 1) * BM) : T;
  u.n_kv = (kv_end + Dims<kD>::BN - 1) / Dims<kD>::BN;
  return u;
}

// Issues the load-to-LDS copies of unit `unit` (64-wide heads) into slot `slot`:
// its 128 q rows and 128 dO rows into K/V buffer 1, its first K/V tile into
// buffer 0 and its lse and delta after the buffers (rows past the sequence end
// read as zero).  Each wave issues STAGE_COPIES copies, waves 0-3 one more first.
template <int kD>
__device__ __forceinline__ void stage_unit(char* __restrict__ smem, int slot, int unit,
                                           const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const uint16_t* __restrict__ dO,
                                           const float* __restrict__ lse,
                                           const float* __restrict__ delta, int B, int T, int Hq,
                                           int Hkv, int causal) {
  using Dm = Dims<kD>;
  static_assert(Dm::STAGED, "64-wide heads only");
  constexpr int TILE_BYTES = Dm::TILE_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const UnitPos u = unit_pos<kD>(unit, B, T, Hq, Hkv, causal);
  char* const base = smem + slot * Dm::SLOT_BYTES;
  const uint32_t q_row = (uint32_t)Hq * kD * 2, kv_row = (uint32_t)Hkv * kD * 2;
  const size_t qe = (size_t)T * Hq * kD, ke = (size_t)T * Hkv * kD;
  if (wave < 4) {  // statistics: wave w copies rows 64*(w%2) .. +63 of lse (w < 2) or delta
    const u32x4_t st_src = raw_rsrc((wave < 2 ? lse : delta) + (size_t)u.b * Hq * T, (uint32_t)Hq * T * 4);
    const int row = u.qt * BM + 64 * (wave & 1) + lane;
    dma4s(st_src, base + Dm::STAT_OFF + 4 * 64 * wave,
          row < T ? ((uint32_t)u.h * T + row) * 4 : 0xffffffffu, 0);
  }
  // Pass p: wave w copies rows 64p + 8w .. +7; lane fills slot lane % 8 of row
  // 8w + lane / 8 of the pass (rows past the sequence end read as zero).
  const int cp_row = 8 * wave + (lane >> 3);
  const uint32_t chunk = 16u * (uint32_t)swz_slot(cp_row, lane & 7);
  const u32x4_t q_src = raw_rsrc(q + u.b * qe, (uint32_t)T * q_row);
  const u32x4_t do_src = raw_rsrc(dO + u.b * qe, (uint32_t)T * q_row);
  const u32x4_t k_src = raw_rsrc(k + u.b * ke, (uint32_t)T * kv_row);
  const u32x4_t v_src = raw_rsrc(v + u.b * ke, (uint32_t)T * kv_row);
  const uint32_t q_off = (uint32_t)cp_row * q_row + chunk;
  const uint32_t kv_off = (uint32_t)cp_row * kv_row + (uint32_t)u.kvh * kD * 2 + chunk;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t q_soff = (uint32_t)(u.qt * BM + 64 * p) * q_row + (uint32_t)u.h * kD * 2;
    char* const dst = base + 8192 * p + 1024 * wave;
    dma16s(q_src, dst + 2 * TILE_BYTES, q_off, q_soff);
    dma16s(do_src, dst + 3 * TILE_BYTES, q_off, q_soff);
    dma16s(k_src, dst, kv_off, (uint32_t)(64 * p) * kv_row);
    dma16s(v_src, dst + TILE_BYTES, kv_off, (uint32_t)(64 * p) * kv_row);
  }
}

// The work of unit `unit` (one 128-row query tile of one (batch, query head),
// see decode_unit) for a 512-thread workgroup.  For 64-wide heads it runs in
// LDS slot `slot` (smem holds Dims<kD>::SMEM_BYTES for slot 0, SMEM2_BYTES for both);
// `staged`: its copies were issued by stage_unit already; next >= 0: the unit
// that follows in this workgroup, whose copies it issues into the other slot.
// kRope: q and k are the rotated q', k' (rotary embedding); the epilogue maps
// dQ back through each pair's rotation transpose with the tables rcos, rsin
// ([T, kD/2] float32), so dq is the gradient with respect to the unrotated q.
template <class E, bool kRope, int kD>
__device__ __forceinline__ void unit_body(
    char* __restrict__ smem, int slot, bool staged, int unit, int next, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dq,
    int B, int T, int Hq, int Hkv, float scale, float scale_log2, int causal) {
  using Dm = Dims<kD>;
  constexpr int TILE_BYTES = Dm::TILE_BYTES, NQ = Dm::NQ, ND = Dm::ND, NH = Dm::NH;
  constexpr int BN = Dm::BN, NB = Dm::NB, HALF_BYTES = Dm::HALF_BYTES;
  constexpr uint32_t kHalf = kD / 2;  // rotary pairs per row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int qb = wave & 3;   // query block within the tile
  const int kh = wave >> 2;  // key half within each K/V tile

  const UnitPos up = unit_pos<kD>(unit, B, T, Hq, Hkv, causal);
  const int b = up.b, kvh = up.kvh, h = up.h, qt = up.qt, n_kv = up.n_kv;
  char* const base = smem + (Dm::STAGED ? slot * Dm::SLOT_BYTES : 0);

  // Per-batch-element buffers; byte offsets below are within one batch element.
  const uint32_t q_row = (uint32_t)Hq * kD * 2;   // bytes between tokens of q / o
  const uint32_t kv_row = (uint32_t)Hkv * kD * 2;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * kD, ke = (size_t)T * Hkv * kD;
  const u32x4_t k_src = raw_rsrc(k + b * ke, (uint32_t)T * kv_row);  // load-to-LDS sources
  const u32x4_t v_src = raw_rsrc(v + b * ke, (uint32_t)T * kv_row);

  const int qw0 = qt * BM + 32 * qb;  // first query row of this wave
  const int my_q = qw0 + l32;
  const uint32_t qoff = (uint32_t)my_q * q_row + (uint32_t)h * kD * 2;  // bytes

  const rsrc_t rdq = make_rsrc(dq + b * qe, (uint32_t)T * q_row);

  // Tile copy: in pass p wave w copies rows 64p + 8w .. +7 of every 64-column
  // half of the K tile and of the V tile; lane fills slot lane % 8 of row
  // 64p + 8w + lane / 8 (rows past the sequence end read as zero).
  const int cp_row = 8 * wave + (lane >> 3);
  const uint32_t cp_off = (uint32_t)cp_row * kv_row + (uint32_t)kvh * kD * 2 +
                          16u * (uint32_t)swz_slot(cp_row, lane & 7);
  auto copy_tile = [&](int kt, int buf) {
#pragma unroll
    for (int p = 0; p < BN / 64; ++p) {
      const uint32_t soff = (uint32_t)(kt * BN + 64 * p) * kv_row;  // scalar
      char* dst = base + (2 * buf) * TILE_BYTES + 8192 * p + 1024 * wave;
#pragma unroll
      for (int c = 0; c < NH; ++c) {
        dma16s(k_src, dst + c * HALF_BYTES, cp_off + 128 * c, soff);
        dma16s(v_src, dst + TILE_BYTES + c * HALF_BYTES, cp_off + 128 * c, soff);
      }
    }
  };

  // Q^T and dO^T as B operands (queries on the lanes), lse and delta of the
  // lane's row.  Rows past the sequence end read lse = delta = 0 and are never
  // stored.
  u32x4_t qf[NQ], df[NQ];
  float lse_raw, Dl;
  if constexpr (Dm::STAGED) {
    if (!staged) stage_unit<kD>(smem, slot, unit, q, k, v, dO, lse, delta, B, T, Hq, Hkv, causal);
    // A staged unit's copies were issued before the previous unit's dQ stores (4 * ND
    // per key-half-0 wave), which may stay in flight.
    if (staged && kh == 0)
      wait_vmem_but<4 * ND>();
    else
      wait_vmem();
    __syncthreads();
    const uint16_t* sQr = reinterpret_cast<const uint16_t*>(base + 2 * TILE_BYTES);
    const uint16_t* sdOr = reinterpret_cast<const uint16_t*>(base + 3 * TILE_BYTES);
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      qf[s] = lds_load16_swz(sQr, 32 * qb + l32, 16 * s + 8 * g);
      df[s] = lds_load16_swz(sdOr, 32 * qb + l32, 16 * s + 8 * g);
    }
    const float* stat = reinterpret_cast<const float*>(base + Dm::STAT_OFF);
    lse_raw = stat[32 * qb + l32];
    Dl = stat[BM + 32 * qb + l32];
    lds_barrier();  // every wave has its rows before buffer 1 is refilled
  } else {
    const rsrc_t rq = make_rsrc(q + b * qe, (uint32_t)T * q_row);
    const rsrc_t rdo = make_rsrc(dO + b * qe, (uint32_t)T * q_row);
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      qf[s] = bload16(rq, qoff + 32 * s + 16 * g);
      df[s] = bload16(rdo, qoff + 32 * s + 16 * g);
    }
    const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
    const rsrc_t rdl = make_rsrc(delta + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
    const uint32_t stat_off = ((uint32_t)h * T + my_q) * 4;
    lse_raw = bload_f32(rl, my_q < T ? stat_off : 0xffffffffu);
    Dl = bload_f32(rdl, my_q < T ? stat_off : 0xffffffffu);
    copy_tile(0, 0);  // in flight together with the row loads above
    wait_loads();
    __syncthreads();
  }
  const float L2 = lse_raw * kLog2e;
  f32x16_t neg_delta;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_delta[r] = -Dl;

  f32x16_t dq_acc[ND];  // dQ^T: rows d = 32*db + 8*(r/4) + 4g + r%4
#pragma unroll
  for (int db = 0; db < ND; ++db) dq_acc[db] = zero16();

  // The next unit's copies go out with the second-to-last tile's own copy (or
  // with the only tile); from then on the loop waits for its own copies only.
  const bool pf = Dm::STAGED && next >= 0;
  const int pf_at = n_kv >= 2 ? n_kv - 2 : 0;

  for (int kt = 0; kt < n_kv; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_kv) copy_tile(kt + 1, cur ^ 1);  // that buffer was last read before the previous barrier
    if constexpr (Dm::STAGED) {
      if (pf && kt == pf_at) stage_unit<kD>(smem, slot ^ 1, next, q, k, v, dO, lse, delta, B, T, Hq, Hkv, causal);
    }
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(base + (2 * cur) * TILE_BYTES);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(base + (2 * cur + 1) * TILE_BYTES);
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      const int krow = kh * (BN / 2) + 32 * sb;  // first tile row of this 32-key block
      const int kb0 = kt * BN + krow;            // its first key
      const bool active = kb0 < T && (!causal || kb0 <= qw0 + 31);
      if (active) {
        f32x16_t sacc = zero16(), pacc = neg_delta;  // dP^T - delta accumulates from -delta
        // Register r holds key kb0 + 8*(r/4) + 4g + r%4 against query my_q.
        const bool masked = (causal && kb0 + 31 > qw0) || kb0 + 32 > T;
        if constexpr (kD == 64) {
          // The block's LDS operands are read up front; the S chain runs first,
          // then dP's products interleaved with the exponentials, then the mask
          // (diagonal block or sequence tail), dS and dQ's products.
          u32x4_t av[NQ], at[ND][2];
          u32x4_t ak[NQ];  // K operands first, so each S product waits for its own
#pragma unroll
          for (int c = 0; c < NQ; ++c) ak[c] = lds_load16_swz(sK, krow + l32, 16 * c + 8 * g);
#pragma unroll
          for (int c = 0; c < NQ; ++c) av[c] = lds_load16_swz(sV, krow + l32, 16 * c + 8 * g);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < NQ; ++c) sacc = E::mfma(ak[c], qf[c], sacc);
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            at[db][0] = lds_operand_T_swz(sK, krow, 32 * db, lane);
            at[db][1] = lds_operand_T_swz(sK, krow + 16, 32 * db, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < NQ; ++c) pacc = E::mfma(av[c], df[c], pacc);
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], scale_log2, -L2));
#pragma unroll
          for (int i = 0; i < NQ; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU
          }
          __builtin_amdgcn_sched_barrier(0);
          if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb0 + 8 * (r >> 2) + 4 * g + (r & 3);
              if ((causal && key > my_q) || key >= T) sacc[r] = 0.f;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) pacc[r] *= sacc[r];
          const u32x4_t ds0 = pack_operand_e<E>(pacc, 0), ds1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            dq_acc[db] = E::mfma(at[db][0], ds0, dq_acc[db]);
            dq_acc[db] = E::mfma(at[db][1], ds1, dq_acc[db]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < NQ; ++s) {  // first product adds to a literal zero
            const int hoff = (s >> 2) * (HALF_BYTES / 2);  // elements to the 64-column half
            const u32x4_t ak = lds_load16_swz(sK + hoff, krow + l32, 16 * (s & 3) + 8 * g);
            const u32x4_t av = lds_load16_swz(sV + hoff, krow + l32, 16 * (s & 3) + 8 * g);
            sacc = E::mfma(ak, qf[s], sacc);
            pacc = E::mfma(av, df[s], pacc);
          }
          if (masked) {
            // Diagonal block or sequence tail: zero P where the key is after the
            // query or past the end.
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb0 + 8 * (r >> 2) + 4 * g + (r & 3);
              const float p = fast_exp2(fmaf(sacc[r], scale_log2, -L2));
              pacc[r] *= ((causal && key > my_q) || key >= T) ? 0.f : p;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) pacc[r] *= fast_exp2(fmaf(sacc[r], scale_log2, -L2));
          }
          const u32x4_t ds0 = pack_operand_e<E>(pacc, 0), ds1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const uint16_t* sKh = sK + (db >> 1) * (HALF_BYTES / 2);
            dq_acc[db] = E::mfma(lds_operand_T_swz(sKh, krow, 32 * (db & 1), lane), ds0, dq_acc[db]);
            dq_acc[db] = E::mfma(lds_operand_T_swz(sKh, krow + 16, 32 * (db & 1), lane), ds1, dq_acc[db]);
          }
        }
      }
    }
    if (pf && kt >= pf_at) {  // the next unit's copies stay in flight
      if (kt + 1 < n_kv) wait_vmem_but<Dm::STAGE_COPIES>();  // the next tile has landed in LDS
      lds_barrier();
    } else {
      wait_loads();  // the next tile has landed in LDS
      __syncthreads();
    }
  }

  // dQ = key half 0 + key half 1, in that order.  Partial of half 1 in LDS as
  // [query block][float4 index f = 4*db + j][lane] (consecutive lanes, no bank
  // conflicts); every wave is past its reads of the last tile.
  float4* part = reinterpret_cast<float4*>(base) + qb * (4 * ND) * 64 + lane;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part[(4 * db + j) * 64] = make_float4(dq_acc[db][4 * j], dq_acc[db][4 * j + 1],
                                              dq_acc[db][4 * j + 2], dq_acc[db][4 * j + 3]);
    }
  }
  lds_barrier();
  if (kh == 0) {  // rows past the sequence end are dropped by the buffer range check
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = part[(4 * db + j) * 64];
        u32x2_t w;
        float g0 = (dq_acc[db][4 * j + 0] + x.x) * scale, g1 = (dq_acc[db][4 * j + 1] + x.y) * scale;
        float g2 = (dq_acc[db][4 * j + 2] + x.z) * scale, g3 = (dq_acc[db][4 * j + 3] + x.w) * scale;
        if (kRope) {  // d = 32db + 8j + 4g + 0..3: pairs 16db + 4j + 2g + 0, 1 of row my_q
          const rsrc_t rtc = make_rsrc(rcos, (uint32_t)T * kHalf * 4u);
          const rsrc_t rts = make_rsrc(rsin, (uint32_t)T * kHalf * 4u);
          const uint32_t toff = ((uint32_t)my_q * kHalf + 16 * db + 4 * j + 2 * g) * 4;
          rope_rotate_back(g0, g1, bload_f32(rtc, toff), bload_f32(rts, toff));
          rope_rotate_back(g2, g3, bload_f32(rtc, toff + 4), bload_f32(rts, toff + 4));
        }
        w[0] = E::pack2(g0, g1);
        w[1] = E::pack2(g2, g3);
        bstore8(rdq, qoff + 2 * (32 * db + 8 * j + 4 * g), w);
      }
    }
  }
}

}  // namespace dqb
}  // namespace rca
