// fwd64.hip -- fused causal attention forward for 64-wide heads in bf16 / fp16 on
// gfx950 MFMA: the workhorse of the headline shape (head_dim 64, "Training a 100M
// transformer in pure Rust: RustingBrain vs PyTorch and TensorFlow", section "The
// setup").
//
// It computes what the forward of section "Step 2: fused flash attention" of that
// page computes -- o = softmax(scale q k^T + causal mask) v and the per-row
// log-sum-exp -- without the [seq_len, seq_len] score matrix that section "Step 1:
// measure before changing anything" found written and read back.
//
// Decomposition (chosen for the CU's budgets, not taken from the page's Ampere
// kernel): at head_dim 64 a 32x32 score block costs as much vector work (the
// softmax: one exponential per score) as matrix work, and a wave that owns only 32
// queries re-reads every K/V row from LDS for each 32 queries, so the forward was
// bound by LDS reads and by matrix and vector work that did not overlap.  Here:
//   * a workgroup owns the query rows of one (batch, query head), split between
//     two key halves and, within each, between query groups: on grids that fit
//     the GPU in one round (at most twice the CU count in 128-row tiles) 8 waves
//     of 32 rows each (128 rows), two workgroups per CU (126 registers), so a
//     heavy query tile's softmax (vector work a single wave issues slowly) is
//     spread over eight waves; on grids of at most half the CU count 4 waves of
//     32 rows each (64 rows), one workgroup per CU, so no wave shares its SIMD;
//     on larger grids 4 waves of 64 rows each (128 rows), two workgroups per CU,
//     so every K/V operand read from LDS feeds two products.  A row's arithmetic
//     is the same in every form, so all forms give the same bits;
//   * K/V tiles of 128 keys go straight from HBM into double-buffered LDS
//     (buffer_load ... lds, no staging registers; 16-byte chunks XOR-swizzled so
//     row reads and transposed reads are free of bank conflicts), and the per-lane
//     LDS offsets are computed once; the workgroup's Q rows arrive the same way
//     (each row copied once, where both key halves' waves read it);
//   * wave (query group, key half kh) takes keys 64s + 32kh .. +31 of every tile
//     (s = 0, 1: its blocks A and B); S^T = K Q^T puts one query per lane, so a
//     row's max and sum take one half-wave exchange, and P goes from the
//     accumulators straight into O^T += V^T P^T (V^T by ds_read_b64_tr_b16);
//   * a block's probabilities are computed against the running max without
//     first taking the block's own maximum (one fma, one exponential, half a pack
//     and half a pair-sum per score); a block where some lane's share of a row
//     sum exceeds 2^8 (its max grew, or the row had none yet) is redone, per
//     32-row query block, with its max taken, the running max moved up to an
//     integer and O and the row sum multiplied by the exact power of two; its
//     P V products are issued only after that check;
//   * within a tile the products of one block are interleaved with the
//     exponentials of the other (block B's score products with block A's softmax,
//     block A's P V products with block B's softmax), so the matrix and vector
//     units work at the same time;
//   * the two key halves' (max, sum, O) are merged in a fixed order; query tiles
//     run heaviest first, the tiles of one (batch, KV head) on one XCD.
// Every sum has a fixed order, so results are bitwise reproducible, and a row's
// result does not depend on T beyond its own keys, on the batch or on the grid.
#include <type_traits>

#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int BN = 128;                 // keys per K/V tile
constexpr int TBYTES = BN * 128;        // one tile of one tensor: 128 rows of 128 bytes
constexpr int BUF_BYTES = 2 * TBYTES;   // K then V
constexpr int SMEM = 2 * BUF_BYTES;     // double-buffered
constexpr float kSumLimit = 256.0f;     // a block is redone when a row's block sum exceeds 2^8

__device__ __forceinline__ int swz_of(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }

// One 32x32 MFMA operand of V^T: rows d = 32db + (lane%32), keys row0 + 8*(e/4) + 4g + e%4,
// from a swizzled V tile; lo / hi are the lane's precomputed byte offsets for the
// key rows row0 + 0..7 and row0 + 8..15 (row0 a multiple of 16).
__device__ __forceinline__ u32x4_t vt_operand(const char* base, uint32_t lo, uint32_t hi) {
  const u32x2_t a = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + lo));
  const u32x2_t b = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + hi));
  u32x4_t o;
  o[0] = a[0];
  o[1] = a[1];
  o[2] = b[0];
  o[3] = b[1];
  return o;
}

// Load-to-LDS of one 16-byte chunk per lane (as dma16s in cdna4.hpp) into the LDS
// byte address m0; the descriptor, m0 and the scalar offset pass through
// readfirstlane so they are scalar registers whatever the allocator did.
__device__ __forceinline__ void dma_rows(const u32x4_t& r, uint32_t m0, uint32_t off, uint32_t soff) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)soff);
  u32x4_t rs;
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)r[i]);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m), "v"(off), "s"(rs), "s"(so)
      : "memory", "m0");
}

// Keys visible to a lane in an edge block: register r of a 32x32 score block is
// key kb0 + 4g + off(r), off(r) = 8*(r/4) + r%4, and is visible iff off(r) <= lim.
// The limit passes through an empty asm so that each use recomputes its compares
// right where they are consumed, instead of the compiler keeping 32 masks alive.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
constexpr int key_off(int r) { return 8 * (r >> 2) + (r & 3); }

// kQB: 32-row query blocks per wave; kNQG: query groups per workgroup (each with
// two waves, one per key half), so a workgroup owns 32 * kQB * kNQG query rows;
// kWaves: waves per SIMD the kernel's registers must allow.  Each row is computed
// the same way in every instantiation (same products, same order, its own slow
// path), so all of them give the same bits.
template <int kNQG>
constexpr int threads_of() { return 128 * kNQG; }
template <bool kPosScale, class E, int kQB, int kNQG, int kWaves>
__global__ __launch_bounds__(threads_of<kNQG>(), kWaves) void attn_fwd64_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int B, int T, int Hq, int Hkv,
    float scale_log2, int causal) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;
  // The lane index read again from the work-item id where it is needed after the
  // loops (the empty asm keeps the compiler from holding it, or values derived
  // from it, in registers across them): with 32-row waves the 8-wave form then fits
  // 128 registers without spills.  With 64-row waves the registers are there and
  // the lane index stays in one.
  auto fresh_lane = [&]() { return kQB == 1 ? opaque((int)(threadIdx.x & 63)) : lane; };
  constexpr int QB = kQB;
  constexpr int NQG = kNQG;        // query groups (32*QB rows each) per workgroup
  constexpr int NW = 2 * NQG;      // waves per workgroup
  constexpr int BM = 32 * QB * NQG;  // query rows per workgroup
  const int qg = wave % NQG;       // query group: rows 32*QB*qg .. of the tile
  const int kh = wave / NQG;       // key half: blocks 32kh and 64 + 32kh of every tile

  const int G = Hq / Hkv;
  const int n_qt = (T + BM - 1) / BM;
  int gi, rank;
  decode_unit_paired(blockIdx.x, gridDim.x, B * Hkv, gi, rank);
  const int b = gi / Hkv;
  const int kvh = gi - b * Hkv;
  const int hh = rank % G;
  const int qt = causal ? n_qt - 1 - rank / G : rank / G;  // heaviest tiles first
  const int h = kvh * G + hh;

  const uint32_t q_row = (uint32_t)Hq * 128;   // bytes between tokens of q / o
  const uint32_t kv_row = (uint32_t)Hkv * 128;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * 64, ke = (size_t)T * Hkv * 64;
  const rsrc_t ro = make_rsrc(o + b * qe, (uint32_t)T * q_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  const u32x4_t k_src = raw_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const u32x4_t v_src = raw_rsrc(v + b * ke, (uint32_t)T * kv_row);

  const int qw0 = qt * BM + 32 * QB * qg;  // first query row of this wave
  // Q^T as B operands: lane holds query qw0 + 32qb + l32, d = 16s + 8g + [0, 8).
  u32x4_t qf[QB][4];
  // byte offset of this lane's row of q / o (recomputed where used, to keep it out of
  // the registers live across the loops)
  auto row_off = [&](int qb) { return (uint32_t)(qw0 + 32 * qb + (fresh_lane() & 31)) * q_row + (uint32_t)h * 128; };

  // Tile copy: instruction (tensor, group of 8 rows) with group = wave + NW*m, so a
  // wave's groups all have the parity of `wave` and one per-lane offset serves
  // them: lane fills slot lane%8 of row 8*group + lane/8, i.e. fetches chunk
  // (lane%8) ^ swz(row).
  const int r8 = lane >> 3;
  const uint32_t dma_lane = (uint32_t)r8 * kv_row + (uint32_t)kvh * 128 +
                            16u * (uint32_t)((lane & 7) ^ swz_of(8 * (wave & 1) + r8));
  const int kv_end = causal ? min(T, (qt + 1) * BM) : T;
  const int n_kv = (kv_end + BN - 1) / BN;
  // LDS byte address of smem (uniform).
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)smem));
  auto copy_tile = [&](int t, int buf) {
    const bool present = t < n_kv;
#pragma unroll
    for (int m = 0; m < 16 / NW; ++m) {
      const int grp = wave + NW * m;
      // out of range (zeros, no traffic) after the last tile
      const uint32_t soff = present ? (uint32_t)(t * BN + 8 * grp) * kv_row : 0x80000000u;
      const uint32_t dst = lds0 + (uint32_t)(buf * BUF_BYTES + grp * 1024);
      dma_rows(k_src, dst, dma_lane, soff);
      dma_rows(v_src, dst + TBYTES, dma_lane, soff);
    }
  };

  // Per-lane LDS byte offsets within a tile (block rows are multiples of 32, so
  // the swizzle of a row depends only on its offset within the block).
  // K as the A operand of S^T: row l32, chunk 2s + g.
  const int swz_l = swz_of(l32);
  uint32_t ka[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ka[s] = (uint32_t)l32 * 128 + 16u * (uint32_t)((2 * s + g) ^ swz_l);
  // V^T operands: 16-lane group gq, lane s16 in it reads row 4*(gq/2) + s16/4 (+8),
  // columns 32db + 16*(gq%2) + 4*(s16%4) .. +3.
  uint32_t va[2][2];
  {
    const int gq = lane >> 4, s16 = lane & 15;
    const int rl = 4 * (gq >> 1) + (s16 >> 2);
    const int cl = 2 * (gq & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int row = rl + 8 * h8;
        va[db][h8] = (uint32_t)row * 128 + 16u * (uint32_t)((4 * db + cl) ^ swz_of(row)) +
                     8u * (uint32_t)(s16 & 1);
      }
    }
  }

  // The workgroup's 128 Q rows are copied once into K/V buffer 1 (as a tile's
  // rows, 8 per instruction, same swizzle; rows past T read as zero) and each
  // wave reads its B operands from there; buffer 1 is refilled only after the
  // barrier that follows those reads.
  {
    const u32x4_t q_src = raw_rsrc(q + b * qe, (uint32_t)T * q_row);
    const uint32_t q_lane = (uint32_t)r8 * q_row + (uint32_t)h * 128 +
                            16u * (uint32_t)((lane & 7) ^ swz_of(8 * (wave & 1) + r8));
#pragma unroll
    for (int m = 0; m < BM / 8 / NW; ++m) {
      const int grp = wave + NW * m;
      dma_rows(q_src, lds0 + (uint32_t)(BUF_BYTES + grp * 1024), q_lane, (uint32_t)(qt * BM + 8 * grp) * q_row);
    }
  }
  copy_tile(0, 0);  // in flight together with the Q rows
  wait_vmem();
  __syncthreads();
  {
    const char* sQ = smem + BUF_BYTES + 32 * QB * qg * 128;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[qb][s] = *reinterpret_cast<const u32x4_t*>(sQ + 32 * qb * 128 + ka[s]);
    }
  }
  lds_barrier();

  f32x16_t oacc[2][QB];  // O^T [db][qb]: rows d = 32db + 8*(r/4) + 4g + r%4, column = query
#pragma unroll
  for (int db = 0; db < 2; ++db)
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = zero16();
  float m_run[QB];  // running max per query (base-2 units; an integer once set)
  float l_run[QB];        // this lane's share of the running sum
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -1e30f; l_run[qb] = 0.f; }

  // The largest key offset a lane may see in the block at kb0 for query block qb:
  // keys up to the lane's query (causal) and below T.
  auto edge_limit = [&](int kb0, int qb) {
    const int ln = fresh_lane();
    const int last = causal ? min(qw0 + 32 * qb + (ln & 31), T - 1) : T - 1;
    return last - kb0 - 4 * (ln >> 5);
  };
  // Score products of one 32-key block (tile rows krow .. +31): for every query
  // block, or (s_one) for query block qb alone.
  auto k_operands = [&](const char* sK, int krow, u32x4_t (&kop)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kop[s] = *reinterpret_cast<const u32x4_t*>(sK + krow * 128 + ka[s]);
  };
  auto s_one = [&](const u32x4_t (&kop)[4], int qb, f32x16_t& acc) {
    acc = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = E::mfma(kop[s], qf[qb][s], acc);
  };
  auto s_block = [&](const char* sK, int krow, f32x16_t (&sacc)[QB]) {
    u32x4_t kop[4];
    k_operands(sK, krow, kop);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s_one(kop, qb, sacc[qb]);
  };
  // P V products of one block: O^T[db][qb] += V^T(keys krow..) P^T.
  auto pv_block = [&](const char* sV, int krow, const u32x4_t (&p)[QB][2]) {
    u32x4_t vop[2][2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vop[db][ks] = vt_operand(sV + (krow + 16 * ks) * 128, va[db][0], va[db][1]);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        oacc[db][qb] = E::mfma(vop[db][0], p[qb][0], oacc[db][qb]);
        oacc[db][qb] = E::mfma(vop[db][1], p[qb][1], oacc[db][qb]);
      }
    }
  };
  // Probabilities of a block against the current running max, packed as the B
  // operands of the P V products.  Register r of sacc[qb] is key
  // kb0 + 8*(r/4) + 4g + r%4 against query qw0 + 32qb + l32; kEdge: the block
  // crosses the diagonal or the sequence end, so keys after the query or past T
  // get probability 0.
  auto exp_one = [&](f32x16_t& acc, int kb0, auto edge_c, int qb, u32x4_t (&p)[2]) {
    constexpr bool kEdge = decltype(edge_c)::value;
    const int lim = kEdge ? opaque(edge_limit(kb0, qb)) : 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(fmaf(acc[r], scale_log2, -m_run[qb]));
      acc[r] = (kEdge && key_off(r) > lim) ? 0.f : pr;
    }
    p[0] = pack_operand_e<E>(acc, 0);
    p[1] = pack_operand_e<E>(acc, 8);
  };
  auto exp_block = [&](f32x16_t (&sacc)[QB], int kb0, auto edge_c, u32x4_t (&p)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) exp_one(sacc[qb], kb0, edge_c, qb, p[qb]);
  };
  // This lane's share (its 16 of the block's 32 keys) of each query's sum of the
  // packed probabilities of a block (the values that enter O), two per
  // v_dot2c_f32 against ones.
  auto sum_one = [&](const u32x4_t (&p)[2]) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = E::add_pair(p[1][i], E::add_pair(p[0][i], acc));
    return acc;
  };
  auto sum_block = [&](const u32x4_t (&p)[QB][2], float (&bs)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bs[qb] = sum_one(p[qb]);
  };
  // Row maxima of a block's scores (masked as in exp_block) and the move of the
  // running max: a row whose maximum exceeds it moves it up to the next integer at
  // or above that maximum, and its O and running sum are multiplied by the exact
  // power of two 2^(m_old - m_new) (0 at the first visible block).
  auto max_rescale_one = [&](const f32x16_t& acc, int kb0, auto edge_c, int qb) {
    constexpr bool kEdge = decltype(edge_c)::value;
    float mraw = kPosScale ? -__builtin_inff() : __builtin_inff();
    const int lim = kEdge ? opaque(edge_limit(kb0, qb)) : 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = acc[r];
      if (kEdge && key_off(r) > lim) x = kPosScale ? -__builtin_inff() : __builtin_inff();
      mraw = kPosScale ? fmaxf(mraw, x) : fminf(mraw, x);
    }
    const float mx = halves_max(mraw * scale_log2);
    const float m_new = mx > m_run[qb] ? ceilf(mx) : m_run[qb];
    const float d = m_run[qb] - m_new;  // 0, a negative integer, or about -1e30 at the start
    const float alpha = d < -126.f ? 0.f : __builtin_ldexpf(1.0f, (int)d);
    m_run[qb] = m_new;
    l_run[qb] *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
    }
  };
  // A block's probabilities were computed against the running max without looking
  // at the block's own maximum.  If some lane's share of a row's block sum exceeds
  // 2^8 (so some probability may exceed 2^8, or overflowed, or the row had no
  // running max yet) the block is redone for that 32-row query block (whichever
  // wave holds it): its scores recomputed, the running max
  // moved and O rescaled, its probabilities and sums recomputed.  Then the sums
  // are added.
  // Its P V products are issued only after this, so O stays consistent.
  auto settle_block = [&](const char* sK, int krow, int kb0, auto edge_c, u32x4_t (&p)[QB][2],
                          float (&bs)[QB]) {
    bool any_big = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any_big = any_big || !(bs[qb] <= kSumLimit);
    if (__any(any_big)) {  // rare: one branch in the common case
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {  // each 32-row query block on its own
        if (__any(!(bs[qb] <= kSumLimit))) {
          u32x4_t kop[4];
          f32x16_t acc;
          k_operands(sK, krow, kop);
          s_one(kop, qb, acc);
          max_rescale_one(acc, kb0, edge_c, qb);
          exp_one(acc, kb0, edge_c, qb, p[qb]);
          bs[qb] = sum_one(p[qb]);
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += bs[qb];
  };

  // One tile: blocks A (keys 32kh) and B (keys 64 + 32kh) of the tile in buffer BUF.
  // The next tile's copies go to the other buffer, last read before the previous
  // barrier.  Waves of 64 rows issue them first; waves of 32 rows after block A's
  // softmax, where the wave waits for A's row sums anyway (issued first, they held
  // up A's score products).
  constexpr bool kCopyFirst = QB == 2;
  auto tile = [&](int t, auto buf_c, auto edge_c) {
    constexpr int BUF = decltype(buf_c)::value;
    if (kCopyFirst) copy_tile(t + 1, BUF ^ 1);
    const char* sK = smem + BUF * BUF_BYTES;
    const char* sV = sK + TBYTES;
    const int krA = 32 * kh, krB = 64 + 32 * kh;
    const int kbA = t * BN + krA, kbB = t * BN + krB;
    f32x16_t sA[QB], sB[QB];
    u32x4_t pA[QB][2], pB[QB][2];
    float bsA[QB], bsB[QB];
    s_block(sK, krA, sA);
    __builtin_amdgcn_sched_barrier(0);
    // block B's score products with block A's exponentials
    s_block(sK, krB, sB);
    exp_block(sA, kbA, edge_c, pA);
    sum_block(pA, bsA);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // twelve VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!kCopyFirst) {
      copy_tile(t + 1, BUF ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    settle_block(sK, krA, kbA, edge_c, pA, bsA);
    __builtin_amdgcn_sched_barrier(0);
    // block A's P V products with block B's exponentials
    pv_block(sV, krA, pA);
    exp_block(sB, kbB, edge_c, pB);
    sum_block(pB, bsB);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    settle_block(sK, krB, kbB, edge_c, pB, bsB);
    __builtin_amdgcn_sched_barrier(0);
    pv_block(sV, krB, pB);
    wait_vmem();  // this wave's part of the next tile has landed
    __syncthreads();
  };
  // Tiles before n_plain need no masking for this wave (the causal diagonal and the
  // sequence end come later, and the wave's blocks of every later tile are edge
  // blocks); the two kinds run in loops of their own (one loop holding both kinds
  // of tile body needs more registers than either).
  const int n_plain = min(min(n_kv, T / BN), causal ? (qw0 + 1) / BN : n_kv);
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t + 1 < n_plain; t += 2) {
    tile(t, B0{}, std::false_type{});
    tile(t + 1, B1{}, std::false_type{});
  }
  if (t < n_plain) {
    tile(t, B0{}, std::false_type{});
    ++t;
  }
  if ((t & 1) && t < n_kv) {
    tile(t, B1{}, std::true_type{});
    ++t;
  }
  for (; t < n_kv; t += 2) {
    tile(t, B0{}, std::true_type{});
    if (t + 1 < n_kv) tile(t + 1, B1{}, std::true_type{});
  }

  // Merge the key halves: (m, l, O) of half 1 into half 0, in that order.  Half 1
  // parks its state as [query block][float4 index f][lane] (f < NF: O^T registers
  // 4(f%4) .. +3 of oacc[f/(4QB)][(f/4)%QB]; f = NF: the first and last query
  // block's m, then their l).
  constexpr int NF = 2 * QB * 4;  // float4 per lane of O^T
  float4* part = reinterpret_cast<float4*>(smem) + qg * (NF + 1) * 64 + fresh_lane();
  if (kh == 1) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const f32x16_t& a = oacc[f / (4 * QB)][(f / 4) % QB];
      const int r = 4 * (f & 3);
      part[f * 64] = make_float4(a[r], a[r + 1], a[r + 2], a[r + 3]);
    }
    part[NF * 64] = make_float4(m_run[0], m_run[QB - 1], l_run[0], l_run[QB - 1]);
  }
  __syncthreads();
  if (kh == 0) {
    const float4 st = part[NF * 64];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m1 = qb == 0 ? st.x : st.y, l1 = qb == 0 ? st.z : st.w;
      const float m = fmaxf(m_run[qb], m1);
      const float a0 = fast_exp2(m_run[qb] - m), a1 = fast_exp2(m1 - m);
      const float l_tot = halves_sum(l_run[qb] * a0 + l1 * a1);
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 x = part[(4 * QB * db + 4 * qb + j) * 64];
          u32x2_t w;
          w[0] = E::pack2((oacc[db][qb][4 * j + 0] * a0 + x.x * a1) * inv,
                          (oacc[db][qb][4 * j + 1] * a0 + x.y * a1) * inv);
          w[1] = E::pack2((oacc[db][qb][4 * j + 2] * a0 + x.z * a1) * inv,
                          (oacc[db][qb][4 * j + 3] * a0 + x.w * a1) * inv);
          bstore8(ro, row_off(qb) + 2 * (32 * db + 8 * j + 4 * (fresh_lane() >> 5)), w);  // rows past T are dropped
        }
      }
      const int ln = fresh_lane();
      const int my_q = qw0 + 32 * qb + (ln & 31);
      if (ln < 32 && my_q < T) bstore_f32(rl, ((uint32_t)h * T + my_q) * 4, (m + fast_log2(l_tot)) * kLn2);
    }
  }
}

}  // namespace

const char* fwd64_tiles() {
  return "fwd64{BN=128,128-row tiles<=CUs/2: BM=64,waves=4(2 query blocks of 32 x 2 key halves),"
         "1 workgroup/CU; <=2*CUs: BM=128,waves=8(4 query blocks of 32 x 2 key halves),"
         "2 workgroups/CU; larger grids: BM=128,waves=4(2 query groups of 64 x 2 key halves),"
         "2 workgroups/CU;lds_dma_x2 K/V tiles,q rows by lds_dma,mfma=32x32x16}";
}

template <class E>
hipError_t launch_fwd64_e(const Problem& p, const void* q, const void* k, const void* v, void* o,
                          float* lse, hipStream_t s) {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipGetLastError();
  // The forms give the same bits; the choice is speed only.  With W = the number of
  // 128-row query tiles:
  //  * 2W <= CUs: 4-wave workgroups of 64 rows (two query groups of 32-row waves),
  //    one per CU, so each wave has its SIMD to itself and a heavy query tile's
  //    chain of products and exponentials runs without a second wave beside it;
  //  * W <= 2 * CUs (the grid fits the GPU in one round): 8-wave workgroups of 128
  //    rows, two per CU (at most 128 registers), spreading the heavy tiles' softmax
  //    over more waves;
  //  * larger grids: 4-wave workgroups of 128 rows in 64-row waves, whose K/V
  //    operands each feed two products.
  using K = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*, int,
                     int, int, int, float, int);
  const bool pos = p.scale_log2 >= 0.f;
  const long long W = (long long)((p.T + 127) / 128) * p.B * p.Hq;
  K kernel;
  int threads, rows;
  if (2 * W <= n_cu) {
    kernel = pos ? attn_fwd64_kernel<true, E, 1, 2, 2> : attn_fwd64_kernel<false, E, 1, 2, 2>;
    threads = threads_of<2>();
    rows = 64;
  } else if (W <= 2LL * n_cu) {
    kernel = pos ? attn_fwd64_kernel<true, E, 1, 4, 4> : attn_fwd64_kernel<false, E, 1, 4, 4>;
    threads = threads_of<4>();
    rows = 128;
  } else {
    kernel = pos ? attn_fwd64_kernel<true, E, 2, 2, 2> : attn_fwd64_kernel<false, E, 2, 2, 2>;
    threads = threads_of<2>();
    rows = 128;
  }
  const dim3 grid((unsigned)((long long)((p.T + rows - 1) / rows) * p.B * p.Hq));
  kernel<<<grid, threads, 0, s>>>(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                  static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                  p.B, p.T, p.Hq, p.Hkv, p.scale_log2, p.causal);
  return hipGetLastError();
}

hipError_t launch_fwd64_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                             float* lse, hipStream_t s) {
  return launch_fwd64_e<Bf16>(p, q, k, v, o, lse, s);
}

hipError_t launch_fwd64_f16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                            float* lse, hipStream_t s) {
  return launch_fwd64_e<F16>(p, q, k, v, o, lse, s);
}

}  // namespace rca
