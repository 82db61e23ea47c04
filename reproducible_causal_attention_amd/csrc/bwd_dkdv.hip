// bwd_dkdv.hip -- dK and dV of fused causal attention, bf16 on gfx950 MFMA.
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
//   * per step the wave copies the 32 query rows of q and dO (loaded from HBM
//     during its previous step, eight whole rows per load instruction) to a
//     wave-private LDS region, immediately
//     issues the loads of its next step, computes S = Q K^T and
//     dP = dO V^T with the keys on the lanes, then P and dS, packs them from the
//     accumulators into B operands and adds dO^T P and Q^T dS into dV^T and dK^T;
//     the transposed A operands are read from the same LDS rows with
//     ds_read_b64_tr_b16;
//   * all loads and stores are buffer instructions whose range check supplies
//     the zero rows past the sequence end, and step indexing is scalar;
//   * the eight partials are summed through LDS in wave order 0..7 and written
//     once (dK scaled by the softmax scale), in bf16 with round to nearest even.
#include "cdna4.hpp"
#include "launch.hpp"

namespace rca {
namespace {

constexpr int PITCH = 72;                     // LDS row pitch (bf16 elements)
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int REGION = 2 * 32 * PITCH + 128;  // one wave's Q rows, dO rows, 64 row stats (bf16 units)
constexpr int PART_STRIDE = 36;               // floats per lane in the partial-sum buffer
constexpr int SMEM_BYTES = NWAVES * REGION * 2;
static_assert(NWAVES * 64 * PART_STRIDE * 4 <= SMEM_BYTES, "reduction buffer must fit");

// One step's operands as loaded: register i of qa (da) holds 16 bytes of q (dO)
// row 8i + lane/8 of the step's 32 query rows, bytes 16*(lane%8) .. +15, so each
// load instruction reads eight whole 128-byte rows; lse and delta belong to
// query row lane % 32.  Nothing reads them until the next step copies them to
// LDS, so the loads stay in flight for a whole step.
struct StepRegs {
  u32x4_t qa[4], da[4];
  float lse, delta;
};

__global__ __launch_bounds__(NTHREADS) void attn_bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int T, int Hq, int Hkv,
    float scale, float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[NWAVES * REGION];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int nkb = (T + 31) / 32;  // 32-row blocks of keys (and of queries)
  int bg, pair;
  decode_unit(blockIdx.x, B * Hkv, bg, pair);  // every pair has the same work
  const int b = bg / Hkv;
  const int kvh = bg - b * Hkv;
  const int G = Hq / Hkv;

  // Per-batch-element buffers; byte offsets below are within one batch element.
  const uint32_t q_row = (uint32_t)Hq * kHeadDim * 2;   // bytes between tokens of q / dO
  const uint32_t kv_row = (uint32_t)Hkv * kHeadDim * 2;  // bytes between tokens of k / v
  const size_t qe = (size_t)T * Hq * kHeadDim, ke = (size_t)T * Hkv * kHeadDim;
  const rsrc_t rq = make_rsrc(q + b * qe, (uint32_t)T * q_row);
  const rsrc_t rdo = make_rsrc(dO + b * qe, (uint32_t)T * q_row);
  const rsrc_t rk = make_rsrc(k + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rv = make_rsrc(v + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdk = make_rsrc(dk + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rdv = make_rsrc(dv + b * ke, (uint32_t)T * kv_row);
  const rsrc_t rl = make_rsrc(lse + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);
  const rsrc_t rd = make_rsrc(delta + (size_t)b * Hq * T, (uint32_t)Hq * T * 4);

  uint16_t* myQ = smem + wave * REGION;
  uint16_t* mydO = myQ + 32 * PITCH;
  float* mystat = reinterpret_cast<float*>(mydO + 32 * PITCH);  // [0,32): lse*log2e, [32,64): delta
  // This lane's 16-byte chunk of a row in the A-operand layout (chunk c adds 32 bytes).
  const uint32_t lane_col = 16u * g;
  // Row staging: lane copies chunk lane % 8 of rows 8i + lane / 8.
  const int st_row = lane >> 3, st_col = 8 * (lane & 7);

  for (int half = 0; half < 2; ++half) {
    const int j = half == 0 ? pair : nkb - 1 - pair;
    if (half == 1 && j == pair) break;  // middle block of an odd count: once only
    const int k0 = 32 * j;
    const int my_key = k0 + l32;

    // K^T and V^T as B operands (keys on the lanes): d = 16s + 8g + [0, 8).
    u32x4_t kf[4], vf[4];
    {
      const uint32_t off = (uint32_t)my_key * kv_row + (uint32_t)kvh * kHeadDim * 2 + lane_col;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kf[s] = bload16(rk, off + 32 * s);
        vf[s] = bload16(rv, off + 32 * s);
      }
      wait_loads();
    }
    f32x16_t dk_acc[2] = {zero16(), zero16()};  // dK^T: rows d = 32*db + 8*(r/4) + 4g + r%4
    f32x16_t dv_acc[2] = {zero16(), zero16()};

    const int qb0 = causal ? j : 0;  // first query block that sees key block j
    const int per_head = nkb - qb0;
    const int nsteps = G * per_head;

    auto load_step = [&](int s, StepRegs& R) {
      const int hh = s / per_head;  // scalar
      const int qb = qb0 + (s - hh * per_head);
      const int h = kvh * G + hh;
      const uint32_t off =
          (uint32_t)(32 * qb + st_row) * q_row + (uint32_t)h * kHeadDim * 2 + 2 * st_col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        R.qa[i] = bload16s(rq, off, (uint32_t)(8 * i) * q_row);
        R.da[i] = bload16s(rdo, off, (uint32_t)(8 * i) * q_row);
      }
      const uint32_t soff = ((uint32_t)h * T + 32 * qb + l32) * 4;
      R.lse = bload_f32(rl, soff);
      R.delta = bload_f32(rd, soff);
    };

    // One step: copy its rows to the wave's LDS region, refill the registers with
    // the rows of this wave's next step (in flight for the whole step), then
    // compute from LDS.
    auto step = [&](int s, StepRegs& R) {
      const int hh = s / per_head;
      const int qb = qb0 + (s - hh * per_head);
      const int q0 = 32 * qb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds_store16(myQ + (8 * i + st_row) * PITCH + st_col, R.qa[i]);
        lds_store16(mydO + (8 * i + st_row) * PITCH + st_col, R.da[i]);
      }
      mystat[lane] = g == 0 ? R.lse * kLog2e : R.delta;  // lanes 0..31: lse in base 2
      if (s + NWAVES < nsteps) load_step(s + NWAVES, R);
      wave_lds_fence();
      f32x16_t sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sacc = mfma_32x32x16(lds_load16(myQ + l32 * PITCH + 16 * c + 8 * g), kf[c], sacc);
        pacc = mfma_32x32x16(lds_load16(mydO + l32 * PITCH + 16 * c + 8 * g), vf[c], pacc);
      }
      // Register r holds query q0 + 8*(r/4) + 4g + r%4 against key my_key.
      float Lr[16], Dr[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 l4 = *reinterpret_cast<const float4*>(mystat + 8 * jj + 4 * g);
        const float4 d4 = *reinterpret_cast<const float4*>(mystat + 32 + 8 * jj + 4 * g);
        Lr[4 * jj + 0] = l4.x; Lr[4 * jj + 1] = l4.y; Lr[4 * jj + 2] = l4.z; Lr[4 * jj + 3] = l4.w;
        Dr[4 * jj + 0] = d4.x; Dr[4 * jj + 1] = d4.y; Dr[4 * jj + 2] = d4.z; Dr[4 * jj + 3] = d4.w;
      }
      if ((causal && qb == j) || q0 + 31 >= T) {
        // Diagonal block or sequence tail: zero P where the key is after the
        // query or the query row does not exist.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
          float p = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
          p = ((causal && my_key > qi) || qi >= T) ? 0.f : p;
          sacc[r] = p;
          pacc[r] = p * (pacc[r] - Dr[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], scale_log2, -Lr[r]));
          sacc[r] = p;
          pacc[r] = p * (pacc[r] - Dr[r]);
        }
      }
      const u32x4_t pb0 = pack_operand(sacc, 0), pb1 = pack_operand(sacc, 8);
      const u32x4_t sb0 = pack_operand(pacc, 0), sb1 = pack_operand(pacc, 8);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dv_acc[db] = mfma_32x32x16(lds_operand_T(mydO, PITCH, 0, 32 * db, lane), pb0, dv_acc[db]);
        dk_acc[db] = mfma_32x32x16(lds_operand_T(myQ, PITCH, 0, 32 * db, lane), sb0, dk_acc[db]);
        dv_acc[db] = mfma_32x32x16(lds_operand_T(mydO, PITCH, 16, 32 * db, lane), pb1, dv_acc[db]);
        dk_acc[db] = mfma_32x32x16(lds_operand_T(myQ, PITCH, 16, 32 * db, lane), sb1, dk_acc[db]);
      }
      wave_lds_fence();  // this step's LDS reads complete before the next step's writes
    };

    StepRegs R;
    if (wave < nsteps) load_step(wave, R);
    for (int s = wave; s < nsteps; s += NWAVES) step(s, R);

    // Sum the eight partials in wave order and write dK (scaled) and dV once.
    float* part = reinterpret_cast<float*>(smem);
    const int kk = tid >> 4;  // key within the block, 0..31
    const int c4 = tid & 15;  // 4-wide column chunk: d = 4*c4
    const int src_lane = kk + 32 * (c4 & 1);
    const int r0 = 16 * (c4 >> 3) + 4 * ((c4 & 7) >> 1);
    const uint32_t out_off = (uint32_t)(k0 + kk) * kv_row + (uint32_t)kvh * kHeadDim * 2 + 8 * c4;
    auto reduce_store = [&](const f32x16_t (&acc)[2], rsrc_t out, float f) {
      __syncthreads();  // LDS free: every wave is past its previous use
      float* mine = part + (wave * 64 + lane) * PART_STRIDE;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *reinterpret_cast<float4*>(mine + 16 * db + r) =
              make_float4(acc[db][r], acc[db][r + 1], acc[db][r + 2], acc[db][r + 3]);
      }
      __syncthreads();
      float4 sum = *reinterpret_cast<const float4*>(part + src_lane * PART_STRIDE + r0);
#pragma unroll
      for (int w = 1; w < NWAVES; ++w) {
        const float4 x = *reinterpret_cast<const float4*>(part + (w * 64 + src_lane) * PART_STRIDE + r0);
        sum.x += x.x;
        sum.y += x.y;
        sum.z += x.z;
        sum.w += x.w;
      }
      u32x2_t o2;
      o2[0] = pack_bf16x2(sum.x * f, sum.y * f);
      o2[1] = pack_bf16x2(sum.z * f, sum.w * f);
      bstore8(out, out_off, o2);  // rows past the sequence end are dropped
    };
    reduce_store(dk_acc, rdk, scale);
    reduce_store(dv_acc, rdv, 1.0f);
    __syncthreads();  // partial buffer is reused as wave regions by the next block
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const void* dO, const float* lse, const float* delta, void* dk,
                                void* dv, hipStream_t s) {
  const int nkb = (p.T + 31) / 32;
  const int npairs = (nkb + 1) / 2;
  const dim3 grid((unsigned)(npairs * p.B * p.Hkv));
  attn_bwd_dkdv_bf16_kernel<<<grid, NTHREADS, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, delta,
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), p.B, p.T, p.Hq, p.Hkv, p.scale,
      p.scale_log2, p.causal);
  return hipGetLastError();
}

const char* bwd_dkdv_tiles() {
  return "dkdv_bf16{key_block=32,waves=8,pairs=(j,n-1-j),query_step=32,mfma=32x32x16,buffer_io}";
}

}  // namespace rca
