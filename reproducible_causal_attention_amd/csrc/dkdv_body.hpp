// dkdv_body.hpp -- dK and dV of fused causal attention, bf16 on gfx950 MFMA.
//
// This is the kernel that "Training a 100M transformer in pure Rust: RustingBrain
// vs PyTorch and TensorFlow", section "Where the time goes now", calls
// flash_attention_dkv: for a block of keys it recomputes the probabilities from
// the saved log-sum-exp (that page's causal_probs_from_lse step), forms
// dS = P * (dP - delta) (its causal_softmax_bwd step) and accumulates
//   dV = sum_i P_ij dO_i   and   dK = scale * sum_i dS_ij q_i
// over every query row i >= j of every query head of the key's group.  No
// atomics: each partial sum has one owner and the partials are combined in a
// fixed order ("rust-trainer", section "The trainer is not bit-identical to
// itself after step 1", loses bit identity to an atomically accumulated
// gradient).
//
// Decomposition (MI355X-first):
//   * a workgroup of 8 waves owns two 32-key blocks j and n-1-j of one
//     (batch, KV head), so under the causal mask every workgroup has the same
//     amount of work (the two blocks see n-j and j+1 query blocks);
//   * the work of one key block is a fixed list of steps (query head of the
//     group, 32-query block); for 64-wide heads the two blocks run at once, the
//     waves split into two groups sized to the blocks' step counts, and wave w
//     of a group of W takes its block's steps w, w+W, w+2W, ..., keeping its own
//     fp32 partial dK^T, dV^T in accumulator registers;
//   * the 32 query rows of q and dO of a step go straight from HBM into a
//     wave-private, double-buffered LDS region (buffer_load ... lds, eight whole
//     rows per instruction, XOR-swizzled 16-byte chunks), issued one step
//     ahead; lse and delta of the rows travel through registers and are stored
//     next to them, delta negated, so the dP accumulator starts at -delta and
//     the products leave dP - delta directly;
//   * S = Q K^T and dP = dO V^T put the keys on the lanes; P and dS are packed
//     from the accumulators into B operands, and dO^T P and Q^T dS are added into
//     dV^T and dK^T with the transposed A operands read by ds_read_b64_tr_b16;
//   * K and V of the key block are staged once through LDS and held in
//     registers as the B operands of S and dP;
//   * each wave parks its partial in its own LDS region; a block's partials
//     (those of its wave group) are summed in wave order and written once (dK
//     scaled by the softmax scale), in bf16 with round to nearest even.
// With 128-wide heads the rows of a step are twice as long, so each wave has
// one step buffer instead of two (the next step's copy is issued once the
// current one has been read), K^T and V^T are read from LDS at every step
// instead of being held in registers, the dK and dV partials are parked and
// summed one after the other, and the two key blocks take one pass each with
// all eight waves (both blocks' K and V do not fit in LDS besides the rows).
#pragma once

#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace dkdv {

constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int HALF_BYTES = 32 * 128;  // 32 swizzled rows of 64 elements

// Head-dimension dependent layout (kD = 64 or 128): a block of 32 rows is kD/64
// swizzled 64-column halves one after the other.
template <int kD>
struct Dims {
  static constexpr int NH = kD / 64, NQ = kD / 16, ND = kD / 32;
  static constexpr int ROWS_BYTES = NH * HALF_BYTES;
  static constexpr int BUF_BYTES = 2 * ROWS_BYTES + 256;  // q rows, dO rows, 64 row statistics
  static constexpr int NBUF = kD == 64 ? 2 : 1;           // step buffers per wave
  static constexpr int WAVE_BYTES = NBUF * BUF_BYTES;
  static constexpr int KV_OFF = NWAVES * WAVE_BYTES;      // staging of the blocks' K and V rows
  static constexpr bool TOGETHER = kD == 64;              // both key blocks of a unit at once
  static constexpr int SMEM_BYTES = KV_OFF + (TOGETHER ? 4 : 2) * ROWS_BYTES;
  static constexpr bool KV_REGS = kD == 64;               // K^T, V^T held in registers
  static constexpr int PASSES = kD == 64 ? 1 : 2;         // dK and dV parked together or in turn
  static_assert(2 * ND * 4 * 64 * 16 / PASSES <= WAVE_BYTES, "a wave's parked partial must fit its region");
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget of one CU");
};

// The work of unit `unit` (a pair of key blocks of one (batch, KV head), see
// decode_unit) for a 512-thread workgroup; smem holds Dims<kD>::SMEM_BYTES.
// kRope: q and k are the rotated q', k' (rotary embedding); the epilogue maps
// dK back through each pair's rotation transpose with the tables rcos, rsin
// ([T, kD/2] float32), so dk is the gradient with respect to the unrotated k.
template <class E, bool kRope, int kD>
__device__ __forceinline__ void unit_body(
    char* __restrict__ smem, int unit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  using Dm = Dims<kD>;
  constexpr int NH = Dm::NH, NQ = Dm::NQ, ND = Dm::ND, ROWS_BYTES = Dm::ROWS_BYTES;
  constexpr int BUF_BYTES = Dm::BUF_BYTES, WAVE_BYTES = Dm::WAVE_BYTES, KV_OFF = Dm::KV_OFF;
  constexpr int HALF_ELEMS = HALF_BYTES / 2;
  constexpr uint32_t kHalf = kD / 2;  // rotary pairs per row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int nkb = (T + 31) / 32;  // 32-row blocks of keys (and of queries)
  int bg, pair;
  decode_unit(unit, B * Hkv, bg, pair);  // every pair has the same work
  const int b = bg / Hkv;
  const int kvh = bg - b * Hkv;
  const int G = Hq / Hkv;

  // Per-batch-element buffers; byte offsets below are within one batch element.
  const uint32_t q_row = (uint32_t)Hq * kD * 2;   // bytes between tokens of q / dO
  const uint32_t kv_row = (uint32_t)Hkv * kD * 2;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * kD, ke = (size_t)T * Hkv * kD;
  const rsrc_t rdk = make_rsrc(dk + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdv = make_rsrc(dv + b * ke, (uint32_t)T * kv_row);
  const u32x4_t q_src = raw_rsrc(q + b * qe, (uint32_t)T * q_row);   // load-to-LDS sources
  const u32x4_t do_src = raw_rsrc(dO + b * qe, (uint32_t)T * q_row);
  const u32x4_t k_src = raw_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const u32x4_t v_src = raw_rsrc(v + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  const rsrc_t rd = make_rsrc(delta + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);

  char* const my_region = smem + wave * WAVE_BYTES;
  // Load-to-LDS lane mapping: lane fills slot lane % 8 of row 8i + lane / 8 of an
  // instruction's eight rows, i.e. it fetches chunk swz_slot(row, lane % 8).
  const int dma_row = lane >> 3;
  auto dma_chunk_bytes = [&](int row) { return 16u * (uint32_t)swz_slot(row, lane & 7); };
  // Per-lane part of the source offset of instruction i of a step (row 8i + lane/8
  // of the 32, chunk by the swizzle); the step's part is wave-uniform.
  uint32_t row_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) row_off[i] = (uint32_t)(8 * i + dma_row) * q_row + dma_chunk_bytes(8 * i + dma_row);

  // The unit's key blocks jA = pair and jB = nkb - 1 - pair.  For 64-wide heads
  // both are processed in one pass: waves [0, w0) take block jA's steps and waves
  // [w0, 8) block jB's, w0 chosen so the two groups' step counts per wave are as
  // equal as possible.  For 128-wide heads (no room in LDS for both blocks' K
  // and V) the blocks take one pass each with all eight waves, as does the
  // middle block of an odd count.
  const int jA = pair, jB = nkb - 1 - pair;
  const bool together = Dm::TOGETHER && jA != jB;
  const int n_pass = (jA == jB || together) ? 1 : 2;
  auto steps_of = [&](int jb) { return G * (nkb - (causal ? jb : 0)); };
  for (int ps = 0; ps < n_pass; ++ps) {
    const int nb = together ? 2 : 1;       // blocks in this pass
    const int jfirst = ps == 0 ? jA : jB;  // block of wave group 0
    int w0 = NWAVES;                       // waves of group 0
    if (together) {
      const int s0 = steps_of(jA), s1 = steps_of(jB);
      int best = 1 << 30;
      for (int w = 1; w < NWAVES; ++w) {
        const int c = max((s0 + w - 1) / w, (s1 + NWAVES - w - 1) / (NWAVES - w));
        if (c < best) { best = c; w0 = w; }
      }
    }
    const int my_b = wave >= w0 ? 1 : 0;
    const int j = my_b == 0 ? jfirst : jB;
    const int gw = wave - (my_b ? w0 : 0);            // rank in the wave group
    const int gs = my_b ? NWAVES - w0 : w0;           // size of the wave group
    const int k0 = 32 * j;
    const int my_key = k0 + l32;

    const int qb0 = causal ? j : 0;  // first query block that sees key block j
    const int per_head = nkb - qb0;
    const int nsteps = G * per_head;
    const uint16_t* const sK = reinterpret_cast<const uint16_t*>(smem + KV_OFF + my_b * 2 * ROWS_BYTES);
    const uint16_t* const sV = sK + ROWS_BYTES / 2;

    // Step s: rows 32*qb .. +31 of query head h of the group.  Issues the copy
    // of its q and dO rows into buffer buf of this wave's region, and returns
    // the loads of the rows' lse and delta.
    auto issue_step = [&](int s, int buf, float& l_raw, float& d_raw) {
      const int hh = s / per_head;  // scalar
      const int qb = qb0 + (s - hh * per_head);
      const int h = kvh * G + hh;
      char* dst = my_region + buf * BUF_BYTES;
      const uint32_t step_off = (uint32_t)(32 * qb) * q_row + (uint32_t)h * kD * 2;  // scalar
#pragma unroll
      for (int c = 0; c < NH; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dma16s(q_src, dst + c * HALF_BYTES + 1024 * i, row_off[i] + 128 * c, step_off);
          dma16s(do_src, dst + ROWS_BYTES + c * HALF_BYTES + 1024 * i, row_off[i] + 128 * c, step_off);
        }
      }
      const uint32_t soff = ((uint32_t)h * T + 32 * qb + l32) * 4;
      l_raw = bload_f32(rl, soff);
      d_raw = bload_f32(rd, soff);
    };

    // Prologue: K and V rows of the pass's blocks (copy instruction i = (block,
    // tensor, 64-column half, group of eight rows) is issued by wave i % 8) and
    // this wave's first step.
    float l_raw = 0.f, d_raw = 0.f;
#pragma unroll
    for (int i = wave; i < nb * 8 * NH; i += NWAVES) {
      const int bb = i / (8 * NH), ii = i % (8 * NH);
      const int t = ii / (4 * NH), c = (ii / 4) % NH, rg = ii % 4;
      const int r = 8 * rg + dma_row;
      const int kb = 32 * (bb == 0 ? jfirst : jB);
      const uint32_t off = (uint32_t)(kb + r) * kv_row + (uint32_t)kvh * kD * 2 + 128 * c + dma_chunk_bytes(r);
      char* dst = smem + KV_OFF + bb * 2 * ROWS_BYTES + t * ROWS_BYTES + c * HALF_BYTES + 1024 * rg;
      dma16(t == 0 ? k_src : v_src, dst, off);
    }
    if (gw < nsteps) issue_step(gw, 0, l_raw, d_raw);
    wait_loads();
    __syncthreads();

    // K^T and V^T as B operands (keys on the lanes): d = 16c + 8g + [0, 8), held in
    // registers for 64-wide heads, read from LDS at every step otherwise.
    auto k_operand = [&](int c) { return lds_load16_swz(sK + (c >> 2) * HALF_ELEMS, l32, 16 * (c & 3) + 8 * g); };
    auto v_operand = [&](int c) { return lds_load16_swz(sV + (c >> 2) * HALF_ELEMS, l32, 16 * (c & 3) + 8 * g); };
    u32x4_t kf[Dm::KV_REGS ? NQ : 1], vf[Dm::KV_REGS ? NQ : 1];
    if (Dm::KV_REGS) {
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        kf[c] = k_operand(c);
        vf[c] = v_operand(c);
      }
    }
    f32x16_t dk_acc[ND], dv_acc[ND];  // dK^T: rows d = 32*db + 8*(r/4) + 4g + r%4
#pragma unroll
    for (int db = 0; db < ND; ++db) dk_acc[db] = dv_acc[db] = zero16();

    int buf = 0;
    for (int s = gw; s < nsteps; s += gs, buf ^= 1) {
      const int hh = s / per_head;
      const int q0 = 32 * (qb0 + (s - hh * per_head));
      char* cur = my_region + (Dm::NBUF == 2 ? buf : 0) * BUF_BYTES;
      const uint16_t* sQ = reinterpret_cast<const uint16_t*>(cur);
      const uint16_t* sdO = reinterpret_cast<const uint16_t*>(cur + ROWS_BYTES);
      float* stat = reinterpret_cast<float*>(cur + 2 * ROWS_BYTES);  // [0,32): lse*log2e, [32,64): -delta

      wait_loads();  // this step's rows and statistics (issued one step ago)
      stat[lane] = g == 0 ? l_raw * kLog2e : -d_raw;
      if (Dm::NBUF == 2 && s + gs < nsteps) issue_step(s + gs, buf ^ 1, l_raw, d_raw);
      wave_lds_fence();

      // Register r of a 32x32 accumulator is query q0 + 8*(r/4) + 4g + r%4
      // against key my_key, so float4 jj of the statistics fills registers 4jj..4jj+3.
      f32x16_t pacc, Lr;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 d4 = *reinterpret_cast<const float4*>(stat + 32 + 8 * jj + 4 * g);
        const float4 l4 = *reinterpret_cast<const float4*>(stat + 8 * jj + 4 * g);
        pacc[4 * jj + 0] = d4.x; pacc[4 * jj + 1] = d4.y; pacc[4 * jj + 2] = d4.z; pacc[4 * jj + 3] = d4.w;
        Lr[4 * jj + 0] = l4.x; Lr[4 * jj + 1] = l4.y; Lr[4 * jj + 2] = l4.z; Lr[4 * jj + 3] = l4.w;
      }
      f32x16_t sacc = zero16();
      if constexpr (Dm::KV_REGS) {
        // 64-wide heads: the step's LDS operands are all read up front; the S
        // chain runs first, then dP's products interleaved with the
        // exponentials, then dV's products interleaved with dS, then dK's.
        u32x4_t da[NQ], ta[ND][4];
#pragma unroll
        for (int c = 0; c < NQ; ++c) da[c] = lds_load16_swz(sdO, l32, 16 * c + 8 * g);
#pragma unroll
        for (int c = 0; c < NQ; ++c) sacc = E::mfma(lds_load16_swz(sQ, l32, 16 * c + 8 * g), kf[c], sacc);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          ta[db][0] = lds_operand_T_swz(sdO, 0, 32 * db, lane);
          ta[db][1] = lds_operand_T_swz(sdO, 16, 32 * db, lane);
          ta[db][2] = lds_operand_T_swz(sQ, 0, 32 * db, lane);
          ta[db][3] = lds_operand_T_swz(sQ, 16, 32 * db, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NQ; ++c) pacc = E::mfma(da[c], vf[c], pacc);  // dP - delta
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        if ((causal && q0 == k0) || q0 + 31 >= T) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((causal && my_key > qi) || qi >= T) sacc[r] = 0.f;
          }
        }
        const u32x4_t pb0 = pack_operand_e<E>(sacc, 0), pb1 = pack_operand_e<E>(sacc, 8);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          dv_acc[db] = E::mfma(ta[db][0], pb0, dv_acc[db]);
          dv_acc[db] = E::mfma(ta[db][1], pb1, dv_acc[db]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] *= sacc[r];
        const u32x4_t sb0 = pack_operand_e<E>(pacc, 0), sb1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          dk_acc[db] = E::mfma(ta[db][2], sb0, dk_acc[db]);
          dk_acc[db] = E::mfma(ta[db][3], sb1, dk_acc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);  // pack P
#pragma unroll
        for (int i = 0; i < 2 * ND; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // a dV product
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);  // dS and its packing
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * ND, 1);  // dK's products
      } else {
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          const int ho = (c >> 2) * HALF_ELEMS, col = 16 * (c & 3) + 8 * g;
          sacc = E::mfma(lds_load16_swz(sQ + ho, l32, col), k_operand(c), sacc);
          pacc = E::mfma(lds_load16_swz(sdO + ho, l32, col), v_operand(c), pacc);
        }
        // pacc now holds dP - delta.  P = exp2(S scale log2e - lse log2e), then on
        // the diagonal block or the sequence tail P = 0 where the key is after the
        // query or the query row does not exist; then dS = P (dP - delta).
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
        if ((causal && q0 == k0) || q0 + 31 >= T) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((causal && my_key > qi) || qi >= T) sacc[r] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] *= sacc[r];
        const u32x4_t pb0 = pack_operand_e<E>(sacc, 0), pb1 = pack_operand_e<E>(sacc, 8);
        const u32x4_t sb0 = pack_operand_e<E>(pacc, 0), sb1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const uint16_t* sdOh = sdO + (db >> 1) * HALF_ELEMS;
          const uint16_t* sQh = sQ + (db >> 1) * HALF_ELEMS;
          const int c0 = 32 * (db & 1);
          dv_acc[db] = E::mfma(lds_operand_T_swz(sdOh, 0, c0, lane), pb0, dv_acc[db]);
          dk_acc[db] = E::mfma(lds_operand_T_swz(sQh, 0, c0, lane), sb0, dk_acc[db]);
          dv_acc[db] = E::mfma(lds_operand_T_swz(sdOh, 16, c0, lane), pb1, dv_acc[db]);
          dk_acc[db] = E::mfma(lds_operand_T_swz(sQh, 16, c0, lane), sb1, dk_acc[db]);
        }
      }
      wave_lds_fence();  // this buffer's reads complete before it is refilled
      if (Dm::NBUF == 1 && s + gs < nsteps) issue_step(s + gs, 0, l_raw, d_raw);
    }

    // Sum each block's partials and write dK (scaled) and dV once.
    // Each wave stores its partial in its own region as soon as its last step
    // is done: [float4 index f][lane], float4 f of a tensor being accumulator
    // registers 4f .. 4f+3 of the flat 16*ND; for 64-wide heads dK at f and dV
    // at 4*ND + f in one pass, otherwise dK in the first pass and dV in the second.
#pragma unroll
    for (int pass = 0; pass < Dm::PASSES; ++pass) {
      if (pass > 0) __syncthreads();  // every wave has read the first pass's partials
      float4* mine = reinterpret_cast<float4*>(my_region);
#pragma unroll
      for (int f = 0; f < 4 * ND; ++f) {
        const int r = 4 * (f & 3);
        if (Dm::PASSES == 1 || pass == 0) {
          const f32x16_t& a = dk_acc[f >> 2];
          mine[f * 64 + lane] = make_float4(a[r], a[r + 1], a[r + 2], a[r + 3]);
        }
        if (Dm::PASSES == 1 || pass == 1) {
          const f32x16_t& c = dv_acc[f >> 2];
          mine[((Dm::PASSES == 1 ? 4 * ND : 0) + f) * 64 + lane] = make_float4(c[r], c[r + 1], c[r + 2], c[r + 3]);
        }
      }
      __syncthreads();
      // Thread -> (key kk, d = 4*c4 .. 4*c4+3), which is registers 16*db + r0 .. +3
      // of lane kk + 32*(c4 % 2) with db = c4 / 8, r0 = 4*((c4 % 8) / 2).  One wave
      // covers the 64 lanes of one float4 index, so its LDS reads are consecutive.
      // Block bb's partials are those of its wave group, summed in wave order.
      const int src_lane = tid & 63;
      const int kk = tid & 31;
      for (int bb = 0; bb < nb; ++bb) {
        const int w_lo = bb == 0 ? 0 : w0, w_hi = bb == 0 ? w0 : NWAVES;
        const int kb = 32 * (bb == 0 ? jfirst : jB);
#pragma unroll
        for (int it = 0; it < NH; ++it) {
          const int c4 = 2 * (wave + NWAVES * it) + ((tid >> 5) & 1);
          const int f = 4 * (c4 >> 3) + ((c4 & 7) >> 1);
          const uint32_t out_off = (uint32_t)(kb + kk) * kv_row + (uint32_t)kvh * kD * 2 + 8 * c4;
#pragma unroll
          for (int t = 0; t < 2; ++t) {  // 0: dK, 1: dV
            if (Dm::PASSES == 2 && t != pass) continue;
            const int fi = (Dm::PASSES == 1 ? t * 4 * ND : 0) + f;
            float4 acc = reinterpret_cast<const float4*>(smem + w_lo * WAVE_BYTES)[fi * 64 + src_lane];
            for (int w = w_lo + 1; w < w_hi; ++w) {
              const float4 x = reinterpret_cast<const float4*>(smem + w * WAVE_BYTES)[fi * 64 + src_lane];
              acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
            }
            u32x2_t out;
            if (t == 0) {
              float g0 = acc.x * scale, g1 = acc.y * scale, g2 = acc.z * scale, g3 = acc.w * scale;
              if (kRope) {  // d = 4*c4 .. +3: pairs 2*c4, 2*c4 + 1 of key kb + kk
                const rsrc_t rtc = make_rsrc(rcos, (uint32_t)T * kHalf * 4u);
                const rsrc_t rts = make_rsrc(rsin, (uint32_t)T * kHalf * 4u);
                const uint32_t toff = ((uint32_t)(kb + kk) * kHalf + 2 * c4) * 4;
                rope_rotate_back(g0, g1, bload_f32(rtc, toff), bload_f32(rts, toff));
                rope_rotate_back(g2, g3, bload_f32(rtc, toff + 4), bload_f32(rts, toff + 4));
              }
              out[0] = E::pack2(g0, g1);
              out[1] = E::pack2(g2, g3);
              bstore8(rdk, out_off, out);  // rows past the sequence end are dropped
            } else {
              out[0] = E::pack2(acc.x, acc.y);
              out[1] = E::pack2(acc.z, acc.w);
              bstore8(rdv, out_off, out);
            }
          }
        }
      }
    }
    lds_barrier();  // the regions are refilled by the next block; its stores need not have landed
  }
}


// ---------------------------------------------------------------------------
// Per-wave units (64-wide heads).  When a pair of key blocks has few steps --
// G * (nkb + 1) <= kSoloMaxSteps, e.g. multi-head attention at T = 1024 has 33 --
// splitting them over eight waves leaves each wave a handful of steps behind
// the unit's shared prologue (K/V staging, a barrier) and epilogue (partials
// parked in LDS, a barrier, a sum over the waves).  Then each wave owns a pair
// (j, n-1-j) of key blocks outright: it loads a block's K and V operands
// straight into registers, runs all of the block's steps (query heads of the
// group, then query blocks, in order) with its own double-buffered row copies,
// and writes dK (scaled) and dV from its accumulators, one block after the
// other.  No barrier, no cross-wave sum.  Workgroup unit u of a (batch, KV head)
// group takes pairs 8u + w (w = wave); the choice depends only on G and T, so
// batch and group slicing keep their bits.
constexpr int kSoloMaxSteps = 48;
__host__ __device__ constexpr bool solo_units(int G, int nkb, int D) {
  return D == 64 && G * (nkb + 1) <= kSoloMaxSteps;
}
// Workgroup units of dK/dV work: pairs of key blocks (split design) or groups of
// eight pairs (per-wave design), per (batch, KV head).
__host__ __device__ constexpr int units_per_group(int G, int nkb, int D) {
  return solo_units(G, nkb, D) ? ((nkb + 1) / 2 + NWAVES - 1) / NWAVES : (nkb + 1) / 2;
}

template <class E, bool kRope>
__device__ __forceinline__ void solo_body(
    char* __restrict__ smem, int unit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  constexpr int kD = 64;
  using Dm = Dims<kD>;
  constexpr int NQ = Dm::NQ, ND = Dm::ND, ROWS_BYTES = Dm::ROWS_BYTES;
  constexpr int BUF_BYTES = Dm::BUF_BYTES, WAVE_BYTES = Dm::WAVE_BYTES;
  constexpr uint32_t kHalf = kD / 2;  // rotary pairs per row
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int nkb = (T + 31) / 32;
  const int npairs = (nkb + 1) / 2;
  const int G = Hq / Hkv;
  int bg, r;
  decode_unit(unit, B * Hkv, bg, r);  // r: workgroup unit within the group
  const int pair = NWAVES * r + wave;
  if (pair >= npairs) return;  // a group's last workgroup unit may hold fewer pairs
  const int b = bg / Hkv;
  const int kvh = bg - b * Hkv;

  const uint32_t q_row = (uint32_t)Hq * kD * 2;
  const uint32_t kv_row = (uint32_t)Hkv * kD * 2;
  const size_t qe = (size_t)T * Hq * kD, ke = (size_t)T * Hkv * kD;
  const rsrc_t rk = make_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rv = make_rsrc(v + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdk = make_rsrc(dk + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdv = make_rsrc(dv + b * ke, (uint32_t)T * kv_row);
  const u32x4_t q_src = raw_rsrc(q + b * qe, (uint32_t)T * q_row);
  const u32x4_t do_src = raw_rsrc(dO + b * qe, (uint32_t)T * q_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  const rsrc_t rd = make_rsrc(delta + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);

  char* const my_region = smem + wave * WAVE_BYTES;
  const int dma_row = lane >> 3;
  uint32_t row_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    row_off[i] = (uint32_t)(8 * i + dma_row) * q_row + 16u * (uint32_t)swz_slot(8 * i + dma_row, lane & 7);

  const int jA = pair, jB = nkb - 1 - pair;
  for (int pass = 0; pass < (jA == jB ? 1 : 2); ++pass) {
    const int j = pass == 0 ? jA : jB;
    const int k0 = 32 * j;
    const int my_key = k0 + l32;
    const int qb0 = causal ? j : 0;
    const int per_head = nkb - qb0;
    const int nsteps = G * per_head;

    // Step s: rows 32*qb .. +31 of query head h of the group into buffer buf.
    auto issue_step = [&](int s, int buf, float& l_raw, float& d_raw) {
      const int hh = s / per_head;
      const int qb = qb0 + (s - hh * per_head);
      const int h = kvh * G + hh;
      char* dst = my_region + buf * BUF_BYTES;
      const uint32_t step_off = (uint32_t)(32 * qb) * q_row + (uint32_t)h * kD * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16s(q_src, dst + 1024 * i, row_off[i], step_off);
        dma16s(do_src, dst + ROWS_BYTES + 1024 * i, row_off[i], step_off);
      }
      const uint32_t soff = ((uint32_t)h * T + 32 * qb + l32) * 4;
      l_raw = bload_f32(rl, soff);
      d_raw = bload_f32(rd, soff);
    };

    // K and V of the block as B operands (keys on the lanes, d = 16c + 8g + [0, 8)),
    // straight from memory; rows past T read as zero.
    u32x4_t kf[NQ], vf[NQ];
    const uint32_t kv_off = (uint32_t)my_key * kv_row + (uint32_t)kvh * kD * 2 + 16u * (uint32_t)g;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      kf[c] = bload16(rk, kv_off + 32 * c);
      vf[c] = bload16(rv, kv_off + 32 * c);
    }
    float l_raw = 0.f, d_raw = 0.f;
    issue_step(0, 0, l_raw, d_raw);  // every block has at least one step
    f32x16_t dk_acc[ND], dv_acc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) dk_acc[db] = dv_acc[db] = zero16();

    int buf = 0;
    for (int s = 0; s < nsteps; ++s, buf ^= 1) {
      const int hh = s / per_head;
      const int q0 = 32 * (qb0 + (s - hh * per_head));
      char* cur = my_region + buf * BUF_BYTES;
      const uint16_t* sQ = reinterpret_cast<const uint16_t*>(cur);
      const uint16_t* sdO = reinterpret_cast<const uint16_t*>(cur + ROWS_BYTES);
      float* stat = reinterpret_cast<float*>(cur + 2 * ROWS_BYTES);  // [0,32): lse*log2e, [32,64): -delta

      wait_vmem();  // this step's rows and statistics (issued one step ago), and K/V
      stat[lane] = g == 0 ? l_raw * kLog2e : -d_raw;
      if (s + 1 < nsteps) issue_step(s + 1, buf ^ 1, l_raw, d_raw);
      wave_lds_fence();

      f32x16_t pacc, Lr;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 d4 = *reinterpret_cast<const float4*>(stat + 32 + 8 * jj + 4 * g);
        const float4 l4 = *reinterpret_cast<const float4*>(stat + 8 * jj + 4 * g);
        pacc[4 * jj + 0] = d4.x; pacc[4 * jj + 1] = d4.y; pacc[4 * jj + 2] = d4.z; pacc[4 * jj + 3] = d4.w;
        Lr[4 * jj + 0] = l4.x; Lr[4 * jj + 1] = l4.y; Lr[4 * jj + 2] = l4.z; Lr[4 * jj + 3] = l4.w;
      }
      f32x16_t sacc = zero16();
      u32x4_t da[NQ], ta[ND][4];
#pragma unroll
      for (int c = 0; c < NQ; ++c) da[c] = lds_load16_swz(sdO, l32, 16 * c + 8 * g);
#pragma unroll
      for (int c = 0; c < NQ; ++c) sacc = E::mfma(lds_load16_swz(sQ, l32, 16 * c + 8 * g), kf[c], sacc);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        ta[db][0] = lds_operand_T_swz(sdO, 0, 32 * db, lane);
        ta[db][1] = lds_operand_T_swz(sdO, 16, 32 * db, lane);
        ta[db][2] = lds_operand_T_swz(sQ, 0, 32 * db, lane);
        ta[db][3] = lds_operand_T_swz(sQ, 16, 32 * db, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NQ; ++c) pacc = E::mfma(da[c], vf[c], pacc);  // dP - delta
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[rr] = fast_exp2(fmaf(sacc[rr], scale_log2, -Lr[rr]));
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Register rr is query q0 + 8*(rr/4) + 4g + rr%4 against key my_key: P = 0 where
      // the key is after the query (diagonal block) or the query row does not exist.
      if ((causal && q0 == k0) || q0 + 31 >= T) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int qi = q0 + 8 * (rr >> 2) + 4 * g + (rr & 3);
          if ((causal && my_key > qi) || qi >= T) sacc[rr] = 0.f;
        }
      }
      const u32x4_t pb0 = pack_operand_e<E>(sacc, 0), pb1 = pack_operand_e<E>(sacc, 8);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        dv_acc[db] = E::mfma(ta[db][0], pb0, dv_acc[db]);
        dv_acc[db] = E::mfma(ta[db][1], pb1, dv_acc[db]);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) pacc[rr] *= sacc[rr];
      const u32x4_t sb0 = pack_operand_e<E>(pacc, 0), sb1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        dk_acc[db] = E::mfma(ta[db][2], sb0, dk_acc[db]);
        dk_acc[db] = E::mfma(ta[db][3], sb1, dk_acc[db]);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * ND, 1);
      wave_lds_fence();  // this buffer's reads complete before it is refilled
    }

    // dK^T, dV^T: lane holds key my_key, d = 32db + 8jj + 4g + 0..3 in registers 4jj..4jj+3.
    // Rows past the sequence end are dropped by the buffer range check.
    const uint32_t out_row = (uint32_t)my_key * kv_row + (uint32_t)kvh * kD * 2;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * db + 8 * jj + 4 * g;
        float g0 = dk_acc[db][4 * jj] * scale, g1 = dk_acc[db][4 * jj + 1] * scale;
        float g2 = dk_acc[db][4 * jj + 2] * scale, g3 = dk_acc[db][4 * jj + 3] * scale;
        if (kRope) {  // pairs d0/2 and d0/2 + 1 of key my_key
          const rsrc_t rtc = make_rsrc(rcos, (uint32_t)T * kHalf * 4u);
          const rsrc_t rts = make_rsrc(rsin, (uint32_t)T * kHalf * 4u);
          const uint32_t toff = ((uint32_t)my_key * kHalf + d0 / 2) * 4;
          rope_rotate_back(g0, g1, bload_f32(rtc, toff), bload_f32(rts, toff));
          rope_rotate_back(g2, g3, bload_f32(rtc, toff + 4), bload_f32(rts, toff + 4));
        }
        u32x2_t wk, wv;
        wk[0] = E::pack2(g0, g1);
        wk[1] = E::pack2(g2, g3);
        wv[0] = E::pack2(dv_acc[db][4 * jj], dv_acc[db][4 * jj + 1]);
        wv[1] = E::pack2(dv_acc[db][4 * jj + 2], dv_acc[db][4 * jj + 3]);
        bstore8(rdk, out_row + 2 * d0, wk);
        bstore8(rdv, out_row + 2 * d0, wv);
      }
    }
  }
}

// Workgroup unit u of the dK/dV work in the design the launcher chose
// (kSolo == solo_units(G, nkb, kD), decided on the host).
template <class E, bool kRope, int kD, bool kSolo>
__device__ __forceinline__ void run_unit(
    char* __restrict__ smem, int unit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
  if constexpr (kSolo && kD == 64)
    solo_body<E, kRope>(smem, unit, q, k, v, dO, lse, delta, rcos, rsin, dk, dv, B, T, Hq, Hkv,
                        scale, scale_log2, causal);
  else
    unit_body<E, kRope, kD>(smem, unit, q, k, v, dO, lse, delta, rcos, rsin, dk, dv, B, T, Hq, Hkv,
                            scale, scale_log2, causal);
}

}  // namespace dkdv
}  // namespace rca
