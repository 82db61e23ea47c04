// validate.hpp -- host-side argument checks shared by the C ABIs (no HIP calls,
// so every error path runs on a machine without a GPU).
#pragma once

#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/attn.h"

namespace rca {
namespace validate {

struct Span {
  uintptr_t lo, hi;
};

inline Span span_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + bytes};
}

inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t elem_size(attn_dtype_t dt) { return dt == ATTN_F32 ? 4 : 2; }

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

inline attn_status_t check_scalars(float scale, int causal) {
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Null and alignment checks over a list of pointers.
inline attn_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (p == nullptr || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

// No output may overlap an input or another output.
inline attn_status_t check_disjoint(std::initializer_list<Span> inputs,
                                    std::initializer_list<Span> outputs) {
  for (auto o = outputs.begin(); o != outputs.end(); ++o) {
    for (const Span& i : inputs)
      if (overlap(*o, i)) return ATTN_ERR_INVALID_ARG;
    for (auto o2 = o + 1; o2 != outputs.end(); ++o2)
      if (overlap(*o, *o2)) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

}  // namespace validate
}  // namespace rca
