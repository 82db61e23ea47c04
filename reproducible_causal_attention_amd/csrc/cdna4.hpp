// cdna4.hpp -- gfx950 building blocks shared by the attention kernels:
// MFMA wrappers, bf16 packing, LDS transpose reads and cross-lane helpers.
//
// Register layouts of v_mfma_f32_32x32x16_bf16 (one 64-lane wave; g = lane / 32):
//   A (32 x 16, M x K): lane holds row m = lane % 32, k = 8g + e for e = 0..7
//   B (16 x 32, K x N): lane holds col n = lane % 32, k = 8g + e
//   C (32 x 32):        lane holds col n = lane % 32 and rows
//                       m = 8*(r/4) + 4g + (r%4) in its accumulator register r = 0..15
// (measured on MI355X with random operands).  Because A and B use the same
// (lane, e) -> k map, any permutation of the physical contraction index applied
// to both operands leaves the product unchanged; the kernels use this to feed
// an accumulator straight back as the next product's operand: accumulator
// registers 8t..8t+7 of a 32-row block hold the 16 rows 16t + {8*(e/4) + 4g + e%4},
// which is exactly an operand k-step whose element e is row 16t + 8*(e/4) + 4g + e%4.
//
// ds_read_b64_tr_b16 (measured): within each group of 16 lanes, let lane s
// supply an address of four consecutive 16-bit elements R[s][0..3]; lane i then
// receives R[4j + i/4][i % 4] as its element j.  If lane s addresses
// row (base + s/4), column (c0 + 4*(s%4)) of a row-major tile, lane i receives
// column c0 + i of rows base + 0..3: a column of the tile, i.e. a transposed read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rca {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D += A * B on the matrix cores, 8 bf16 per lane per operand, fp32 accumulate.
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Two floats -> one dword of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Eight consecutive accumulator registers r0..r0+7 -> one bf16 MFMA operand.
__device__ __forceinline__ u32x4_t pack_operand(const f32x16_t& acc, int r0) {
  u32x4_t o;
  o[0] = pack_bf16x2(acc[r0 + 0], acc[r0 + 1]);
  o[1] = pack_bf16x2(acc[r0 + 2], acc[r0 + 3]);
  o[2] = pack_bf16x2(acc[r0 + 4], acc[r0 + 5]);
  o[3] = pack_bf16x2(acc[r0 + 6], acc[r0 + 7]);
  return o;
}

// acc + lo(w) + hi(w) for the two bf16 halves of w (v_dot2c_f32_bf16 against ones).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions across the two 32-lane halves of a wave with one v_permlane32_swap.
// swap(x, x) leaves lane i < 32 with {x[i], x[i + 32]} and lane i + 32 with
// {x[i], x[i + 32]} as well, so both halves combine the same two values in the
// same order and get bitwise-equal results.
__device__ __forceinline__ float halves_max(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  const int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// 16-byte LDS load / store.
__device__ __forceinline__ u32x4_t lds_load16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void lds_store16(uint16_t* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// ds_read_b64_tr_b16 on an LDS address.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Operand of a 32x32x16 product whose contraction index runs along the rows of a
// row-major LDS tile and whose M (or N) index runs along its columns: lane l gets
// column c0 + l%32 of rows row0 + {4g + 0..3} (elements 0..3) and row0 + 8 + {4g + 0..3}
// (elements 4..7), g = l/32 -- the element order of an accumulator fed back as an
// operand (see the header comment).
__device__ __forceinline__ u32x4_t lds_operand_T(const uint16_t* tile, int pitch, int row0, int c0,
                                                 int lane) {
  const int grp = lane >> 4;   // 16-lane group 0..3
  const int s = lane & 15;     // lane within the group
  const int row = row0 + 4 * (grp >> 1) + (s >> 2);
  const int col = c0 + 16 * (grp & 1) + 4 * (s & 3);
  const u32x2_t lo = lds_read_tr16(tile + row * pitch + col);
  const u32x2_t hi = lds_read_tr16(tile + (row + 8) * pitch + col);
  u32x4_t o;
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
  return o;
}

// Swizzled row-major tiles of 128-byte rows (64 bf16, no padding), as written by
// load-to-LDS: 16-byte chunk c of row r is stored in slot c ^ swz(r) of that row,
// swz(r) = 4*((r/2) % 2) + (r/4) % 4.  With 64 four-byte banks two consecutive
// rows fill all banks, and this choice keeps both access patterns below free of
// bank conflicts within each 32-lane half: a 16-byte read of one chunk from 16
// consecutive rows, and the transposed reads of lds_operand_T_swz.
__device__ __forceinline__ int swz_slot(int row, int chunk) {
  return chunk ^ (4 * ((row >> 1) & 1) + ((row >> 2) & 3));
}
// Byte offset of element col (a multiple of 4) of row in a swizzled tile.
__device__ __forceinline__ uint32_t swz_off(int row, int col) {
  return (uint32_t)row * 128u + 16u * (uint32_t)swz_slot(row, col >> 3) + 2u * (uint32_t)(col & 7);
}
__device__ __forceinline__ u32x4_t lds_load16_swz(const uint16_t* tile, int row, int col) {
  return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(tile) + swz_off(row, col));
}
// lds_operand_T on a swizzled tile.
__device__ __forceinline__ u32x4_t lds_operand_T_swz(const uint16_t* tile, int row0, int c0, int lane) {
  const int grp = lane >> 4;
  const int s = lane & 15;
  const int row = row0 + 4 * (grp >> 1) + (s >> 2);
  const int col = c0 + 16 * (grp & 1) + 4 * (s & 3);
  const char* base = reinterpret_cast<const char*>(tile);
  const u32x2_t lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + swz_off(row, col)));
  const u32x2_t hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + swz_off(row + 8, col)));
  u32x4_t o;
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
  return o;
}

// Element types of the 16-bit kernels.  Each trait gives the matrix product,
// the fp32 -> 16-bit pair conversion (round to nearest even: v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32), the 16-bit -> fp32 unpacking of the two halves of a dword
// and the sum of a packed pair into an fp32 accumulator (v_dot2c against ones).
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
  static constexpr const char* name = "bf16";
  __device__ static __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return mfma_32x32x16(a, b, c);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  __device__ static __forceinline__ float add_pair(uint32_t w, float acc) { return add_bf16_pair(w, acc); }
};

struct F16 {
  static constexpr const char* name = "f16";
  __device__ static __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2_t v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
  __device__ static __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }
  __device__ static __forceinline__ float add_pair(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w),
                                  __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc, false);
  }
};

// Eight consecutive accumulator registers r0..r0+7 -> one 16-bit MFMA operand.
template <class E>
__device__ __forceinline__ u32x4_t pack_operand_e(const f32x16_t& acc, int r0) {
  u32x4_t o;
  o[0] = E::pack2(acc[r0 + 0], acc[r0 + 1]);
  o[1] = E::pack2(acc[r0 + 2], acc[r0 + 3]);
  o[2] = E::pack2(acc[r0 + 4], acc[r0 + 5]);
  o[3] = E::pack2(acc[r0 + 6], acc[r0 + 7]);
  return o;
}

// The float whose bits are w.  Takes w by value: __builtin_bit_cast applied
// directly to a vector element (v[e]) reads element 0 with this compiler.
__device__ __forceinline__ float bits_to_float(uint32_t w) { return __builtin_bit_cast(float, w); }

// Rotary embedding of one packed pair (x[2i], x[2i+1]) by (c, s) = (cos, sin) of
// its angle: (x0 c - x1 s, x0 s + x1 c), each an explicit fma so every kernel
// that rotates the same pair gets the same bits.
template <class E>
__device__ __forceinline__ uint32_t rope_rotate(uint32_t w, float c, float s) {
  const float x0 = E::lo(w), x1 = E::hi(w);
  return E::pack2(fmaf(x0, c, -(x1 * s)), fmaf(x0, s, x1 * c));
}
// The transpose, applied to an fp32 gradient pair (g0, g1): (g0 c + g1 s, -g0 s + g1 c).
__device__ __forceinline__ void rope_rotate_back(float& g0, float& g1, float c, float s) {
  const float a = fmaf(g0, c, g1 * s), b = fmaf(g1, c, -(g0 * s));
  g0 = a;
  g1 = b;
}

__device__ __forceinline__ u32x4_t zero4u() {
  u32x4_t z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

__device__ __forceinline__ u32x4_t gload16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Buffer descriptor over [base, base + bytes).  The hardware range check
// (measured on gfx950, and it includes the scalar offset) makes loads past the
// end return zero and drops stores past the end, so tail rows need no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Same with a wave-uniform byte offset added in the scalar offset field.
__device__ __forceinline__ u32x4_t bload16s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}

// Load-to-LDS (measured on gfx950): buffer_load_dwordx4 ... lds writes lane i's
// 16 bytes to LDS at M0 + 16*i; the scalar offset applies to the global address
// only, and the wave's vmcnt covers the LDS write.  It is issued from inline
// assembly so the compiler does not guard every later LDS read with a wait for
// it (it cannot tell the destination apart from the buffers being read); the
// kernels wait for these loads themselves with wait_loads().  The descriptor is
// the raw four-dword form of make_rsrc's, in scalar registers.
__device__ __forceinline__ u32x4_t raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xffffu;  // stride 0
  r[2] = bytes;                           // range checked in bytes
  r[3] = 0x00020000u;                     // the same flags make_rsrc uses
  return r;
}
__device__ __forceinline__ void dma16(const u32x4_t& r, const void* lds, uint32_t off) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(off), "s"(r)
      : "memory", "m0");
}
// Same with a wave-uniform byte offset soff added to the global address.
__device__ __forceinline__ void dma16s(const u32x4_t& r, const void* lds, uint32_t off, uint32_t soff) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(off), "s"(r), "s"(soff)
      : "memory", "m0");
}

// Load-to-LDS of one dword per lane: lane i's 4 bytes go to LDS at M0 + 4*i.
__device__ __forceinline__ void dma4s(const u32x4_t& r, const void* lds, uint32_t off, uint32_t soff) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(off), "s"(r), "s"(soff)
      : "memory", "m0");
}

// Index of the calling wave within its workgroup, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Wait for all of this wave's outstanding global/buffer loads.  Issued once
// after loads that precede a loop, so the loop's own prefetches are the only
// loads in flight inside it and the compiler's waits cover just those.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same wait as an instruction the compiler sees (s_waitcnt vmcnt(0); the other
// counters untouched), so its own wait-count bookkeeping knows every earlier
// vector-memory load has completed and adds no waits for them later (an inline
// asm wait is opaque to it: loads issued before one still count as pending).
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt = 0, expcnt = 7, lgkmcnt = 15 (gfx9 encoding)
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding
// (they complete in issue order), leaving the N most recent in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt field of the immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for the wave's
// outstanding global loads and load-to-LDS copies.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt = 0; vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this wave's outstanding LDS operations; also a compiler memory barrier.
// Used between a wave's writes to its private LDS region and its own reads.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroups are dispatched to the 8 XCDs round-robin (block i runs on XCD i % 8),
// and each XCD has its own L2.  Work is described as units (group gi, rank r):
// units of one group read the same K/V and rank orders a group's units from
// heaviest to lightest.  When the group count is a multiple of 8, the units of
// group gi all run on XCD gi % 8, and every XCD still receives its units heaviest
// rank first; otherwise units go out heaviest rank first across all groups.
// A bijection from [0, NG*U) onto the units.
__device__ __forceinline__ void decode_unit(int i, int NG, int& gi, int& r) {
  if ((NG & 7) == 0) {
    const int x = i & 7, slot = i >> 3, M = NG >> 3;
    r = slot / M;
    gi = x + 8 * (slot - r * M);
  } else {
    r = i / NG;
    gi = i - r * NG;
  }
}

// The forward's order for grids of 256 < n <= 512 workgroups (two per CU):
// workgroup i and i + 256 land on the same CU, so the first n - 256 CUs of the
// 256 host two workgroups and the rest one (measured from workgroup timelines
// on MI355X: 32 CUs per XCD, blocks dealt to XCDs round-robin).  Per XCD the
// heaviest units go to the CUs that host one workgroup, and the others are
// paired heaviest with lightest, so no CU holds a heavy unit and a second one.
// Units keep their XCD as in decode_unit.  Other grids use decode_unit.
__device__ __forceinline__ void decode_unit_paired(int i, int n, int NG, int& gi, int& r) {
  if ((NG & 7) != 0 || (n & 7) != 0 || n <= 256 || n > 512) {
    decode_unit(i, NG, gi, r);
    return;
  }
  const int x = i & 7, slot = i >> 3;  // XCD, and slot within it (32 per round)
  const int per = n >> 3;              // units per XCD
  const int dbl = per - 32;            // CUs of this XCD that host two workgroups
  int k;                               // 0 = heaviest unit of this XCD
  if (slot >= 32) k = per - 1 - (slot - 32);  // second workgroup of a CU: lightest first
  else if (slot >= dbl) k = slot - dbl;       // CUs with one workgroup: the heaviest
  else k = (32 - dbl) + slot;                 // first workgroup of a shared CU: next heaviest
  const int M = NG >> 3;
  r = k / M;
  gi = x + 8 * (k - r * M);
}

}  // namespace rca
