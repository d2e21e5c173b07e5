// Host-side helpers for argument validation at the C ABI.
#pragma once

#include <stdint.h>

#include "../../include/cskv.h"

namespace cskv {

inline bool aligned16_one(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when every non-null pointer is 16-byte aligned.
template <typename... P>
inline bool aligned16(P... ps) {
  return (aligned16_one(static_cast<const void*>(ps)) && ...);
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace cskv
