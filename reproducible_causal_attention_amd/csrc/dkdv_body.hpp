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
//     group, 32-query block); wave w takes steps w, w+8, w+16, ... and keeps its
//     own fp32 partial dK^T, dV^T in accumulator registers;
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
//   * each wave parks its partial in its own LDS region; the eight partials are
//     summed in wave order 0..7 and written once (dK scaled by the softmax
//     scale), in bf16 with round to nearest even.
#pragma once

#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace dkdv {

constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int ROWS_BYTES = 32 * 128;                   // 32 swizzled rows of 64 bf16
constexpr int BUF_BYTES = 2 * ROWS_BYTES + 256;        // q rows, dO rows, 64 row statistics
constexpr int WAVE_BYTES = 2 * BUF_BYTES;              // double-buffered
constexpr int KV_OFF = NWAVES * WAVE_BYTES;            // staging of the block's K and V rows
constexpr int SMEM_BYTES = KV_OFF + 2 * ROWS_BYTES;
static_assert(16 * 64 * 16 <= WAVE_BYTES, "a wave's partial dK, dV must fit its region");
static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget of one CU");

// The work of unit `unit` (a pair of key blocks of one (batch, KV head), see
// decode_unit) for a 512-thread workgroup; smem holds SMEM_BYTES.
// kRope: q and k are the rotated q', k' (rotary embedding); the epilogue maps
// dK back through each pair's rotation transpose with the tables rcos, rsin
// ([T, 32] float32), so dk is the gradient with respect to the unrotated k.
template <class E, bool kRope>
__device__ __forceinline__ void unit_body(
    char* __restrict__ smem, int unit, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ rcos, const float* __restrict__ rsin, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv, float scale, float scale_log2,
    int causal) {
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
  const uint32_t q_row = (uint32_t)Hq * kHeadDim * 2;   // bytes between tokens of q / dO
  const uint32_t kv_row = (uint32_t)Hkv * kHeadDim * 2;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * kHeadDim, ke = (size_t)T * Hkv * kHeadDim;
  const rsrc_t rdk = make_rsrc(dk + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdv = make_rsrc(dv + b * ke, (uint32_t)T * kv_row);
  const u32x4_t q_src = raw_rsrc(q + b * qe, (uint32_t)T * q_row);   // load-to-LDS sources
  const u32x4_t do_src = raw_rsrc(dO + b * qe, (uint32_t)T * q_row);
  const u32x4_t k_src = raw_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const u32x4_t v_src = raw_rsrc(v + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  const rsrc_t rd = make_rsrc(delta + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);

  char* const my_region = smem + wave * WAVE_BYTES;
  const uint16_t* const sK = reinterpret_cast<const uint16_t*>(smem + KV_OFF);
  const uint16_t* const sV = reinterpret_cast<const uint16_t*>(smem + KV_OFF + ROWS_BYTES);
  // Load-to-LDS lane mapping: lane fills slot lane % 8 of row 8i + lane / 8 of an
  // instruction's eight rows, i.e. it fetches chunk swz_slot(row, lane % 8).
  const int dma_row = lane >> 3;
  auto dma_chunk_bytes = [&](int row) { return 16u * (uint32_t)swz_slot(row, lane & 7); };
  // Per-lane part of the source offset of instruction i of a step (row 8i + lane/8
  // of the 32, chunk by the swizzle); the step's part is wave-uniform.
  uint32_t row_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) row_off[i] = (uint32_t)(8 * i + dma_row) * q_row + dma_chunk_bytes(8 * i + dma_row);

  for (int half = 0; half < 2; ++half) {
    const int j = half == 0 ? pair : nkb - 1 - pair;
    if (half == 1 && j == pair) break;  // middle block of an odd count: once only
    const int k0 = 32 * j;
    const int my_key = k0 + l32;

    const int qb0 = causal ? j : 0;  // first query block that sees key block j
    const int per_head = nkb - qb0;
    const int nsteps = G * per_head;

    // Step s: rows 32*qb .. +31 of query head h of the group.  Issues the copy
    // of its q and dO rows into buffer buf of this wave's region, and returns
    // the loads of the rows' lse and delta.
    auto issue_step = [&](int s, int buf, float& l_raw, float& d_raw) {
      const int hh = s / per_head;  // scalar
      const int qb = qb0 + (s - hh * per_head);
      const int h = kvh * G + hh;
      char* dst = my_region + buf * BUF_BYTES;
      const uint32_t step_off = (uint32_t)(32 * qb) * q_row + (uint32_t)h * kHeadDim * 2;  // scalar
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16s(q_src, dst + 1024 * i, row_off[i], step_off);
        dma16s(do_src, dst + ROWS_BYTES + 1024 * i, row_off[i], step_off);
      }
      const uint32_t soff = ((uint32_t)h * T + 32 * qb + l32) * 4;
      l_raw = bload_f32(rl, soff);
      d_raw = bload_f32(rd, soff);
    };

    // Prologue: K and V rows of the block (wave w copies eight rows of K for
    // w < 4, of V for w >= 4) and this wave's first step.
    float l_raw = 0.f, d_raw = 0.f;
    {
      const int r = 8 * (wave & 3) + dma_row;
      const uint32_t off = (uint32_t)(k0 + r) * kv_row + (uint32_t)kvh * kHeadDim * 2 + dma_chunk_bytes(r);
      char* dst = smem + KV_OFF + (wave >> 2) * ROWS_BYTES + 1024 * (wave & 3);
      dma16(wave < 4 ? k_src : v_src, dst, off);
    }
    if (wave < nsteps) issue_step(wave, 0, l_raw, d_raw);
    wait_loads();
    __syncthreads();

    // K^T and V^T as B operands (keys on the lanes): d = 16c + 8g + [0, 8).
    u32x4_t kf[4], vf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kf[c] = lds_load16_swz(sK, l32, 16 * c + 8 * g);
      vf[c] = lds_load16_swz(sV, l32, 16 * c + 8 * g);
    }
    f32x16_t dk_acc[2] = {zero16(), zero16()};  // dK^T: rows d = 32*db + 8*(r/4) + 4g + r%4
    f32x16_t dv_acc[2] = {zero16(), zero16()};

    int buf = 0;
    for (int s = wave; s < nsteps; s += NWAVES, buf ^= 1) {
      const int hh = s / per_head;
      const int q0 = 32 * (qb0 + (s - hh * per_head));
      char* cur = my_region + buf * BUF_BYTES;
      const uint16_t* sQ = reinterpret_cast<const uint16_t*>(cur);
      const uint16_t* sdO = reinterpret_cast<const uint16_t*>(cur + ROWS_BYTES);
      float* stat = reinterpret_cast<float*>(cur + 2 * ROWS_BYTES);  // [0,32): lse*log2e, [32,64): -delta

      wait_loads();  // this step's rows and statistics (issued one step ago)
      stat[lane] = g == 0 ? l_raw * kLog2e : -d_raw;
      if (s + NWAVES < nsteps) issue_step(s + NWAVES, buf ^ 1, l_raw, d_raw);
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
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sacc = E::mfma(lds_load16_swz(sQ, l32, 16 * c + 8 * g), kf[c], sacc);
        pacc = E::mfma(lds_load16_swz(sdO, l32, 16 * c + 8 * g), vf[c], pacc);
      }
      // pacc now holds dP - delta.
      if ((causal && q0 == k0) || q0 + 31 >= T) {
        // Diagonal block or sequence tail: zero P where the key is after the
        // query or the query row does not exist.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
          float p = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
          p = ((causal && my_key > qi) || qi >= T) ? 0.f : p;
          sacc[r] = p;
          pacc[r] *= p;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
          sacc[r] = p;
          pacc[r] *= p;
        }
      }
      const u32x4_t pb0 = pack_operand_e<E>(sacc, 0), pb1 = pack_operand_e<E>(sacc, 8);
      const u32x4_t sb0 = pack_operand_e<E>(pacc, 0), sb1 = pack_operand_e<E>(pacc, 8);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dv_acc[db] = E::mfma(lds_operand_T_swz(sdO, 0, 32 * db, lane), pb0, dv_acc[db]);
        dk_acc[db] = E::mfma(lds_operand_T_swz(sQ, 0, 32 * db, lane), sb0, dk_acc[db]);
        dv_acc[db] = E::mfma(lds_operand_T_swz(sdO, 16, 32 * db, lane), pb1, dv_acc[db]);
        dk_acc[db] = E::mfma(lds_operand_T_swz(sQ, 16, 32 * db, lane), sb1, dk_acc[db]);
      }
      wave_lds_fence();  // this buffer's reads complete before it is refilled
    }

    // Sum the eight partials in wave order and write dK (scaled) and dV once.
    // Each wave stores its partial in its own region as soon as its last step
    // is done: [float4 index f][lane], f = 0..7 dK, 8..15 dV, float4 f of a
    // tensor being accumulator registers 4f .. 4f+3 of the flat 32.
    {
      float4* mine = reinterpret_cast<float4*>(my_region);
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const f32x16_t& a = dk_acc[f >> 2];
        const f32x16_t& c = dv_acc[f >> 2];
        const int r = 4 * (f & 3);
        mine[f * 64 + lane] = make_float4(a[r], a[r + 1], a[r + 2], a[r + 3]);
        mine[(8 + f) * 64 + lane] = make_float4(c[r], c[r + 1], c[r + 2], c[r + 3]);
      }
    }
    __syncthreads();
    {
      // Thread -> (key kk, d = 4*c4 .. 4*c4+3), which is registers 16*db + r0 .. +3
      // of lane kk + 32*(c4 % 2) with db = c4 / 8, r0 = 4*((c4 % 8) / 2).  One wave
      // covers the 64 lanes of one float4 index, so its LDS reads are consecutive.
      const int src_lane = tid & 63;
      const int kk = tid & 31;
      const int c4 = 2 * wave + ((tid >> 5) & 1);
      const int f = 4 * (c4 >> 3) + ((c4 & 7) >> 1);  // = 4*(wave/4) + wave%4
      const float4* part0 = reinterpret_cast<const float4*>(smem);
      float4 sk = part0[f * 64 + src_lane], sv = part0[(8 + f) * 64 + src_lane];
#pragma unroll
      for (int w = 1; w < NWAVES; ++w) {
        const float4* part = reinterpret_cast<const float4*>(smem + w * WAVE_BYTES);
        const float4 xk = part[f * 64 + src_lane];
        const float4 xv = part[(8 + f) * 64 + src_lane];
        sk.x += xk.x; sk.y += xk.y; sk.z += xk.z; sk.w += xk.w;
        sv.x += xv.x; sv.y += xv.y; sv.z += xv.z; sv.w += xv.w;
      }
      const uint32_t out_off = (uint32_t)(k0 + kk) * kv_row + (uint32_t)kvh * kHeadDim * 2 + 8 * c4;
      u32x2_t ok, ov;
      float g0 = sk.x * scale, g1 = sk.y * scale, g2 = sk.z * scale, g3 = sk.w * scale;
      if (kRope) {  // d = 4*c4 .. +3: pairs 2*c4, 2*c4 + 1 of key k0 + kk
        const rsrc_t rtc = make_rsrc(rcos, (uint32_t)T * 128u), rts = make_rsrc(rsin, (uint32_t)T * 128u);
        const uint32_t toff = ((uint32_t)(k0 + kk) * 32 + 2 * c4) * 4;
        rope_rotate_back(g0, g1, bload_f32(rtc, toff), bload_f32(rts, toff));
        rope_rotate_back(g2, g3, bload_f32(rtc, toff + 4), bload_f32(rts, toff + 4));
      }
      ok[0] = E::pack2(g0, g1);
      ok[1] = E::pack2(g2, g3);
      ov[0] = E::pack2(sv.x, sv.y);
      ov[1] = E::pack2(sv.z, sv.w);
      bstore8(rdk, out_off, ok);  // rows past the sequence end are dropped
      bstore8(rdv, out_off, ov);
    }
    __syncthreads();  // the regions are refilled by the next block
  }
}

}  // namespace dkdv
}  // namespace rca
