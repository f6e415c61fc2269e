// Internal helpers shared by the HIP translation units of libscfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scfa.h"

#define SCFA_RETURN_IF_LAUNCH_FAILED()                 \
  do {                                                 \
    if (hipGetLastError() != hipSuccess) return SCFA_ERR_HIP; \
  } while (0)

namespace scfa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kInt32Max = 2147483647;
constexpr int kInt32Min = -2147483647 - 1;

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int pad_rows(int n) { return SCFA_PAD(n); }

inline bool dtype_ok(int dt) { return dt == SCFA_BF16 || dt == SCFA_F32; }
inline int dtype_size(int dt) { return dt == SCFA_BF16 ? 2 : 4; }
// Offset added to key positions in every causal comparison: 1 for the strict
// variant (a key strictly before its query), else 0.
inline int strict_of(int mode_or_flags) { return (mode_or_flags & SCFA_STRICT) ? 1 : 0; }

// Number of lanes below this one whose bit is set in `mask` (wave64).
__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ inline void set_dev_err(int32_t* dev_err, int bit) {
  if (dev_err) atomicOr(dev_err, bit);
}

}  // namespace scfa
