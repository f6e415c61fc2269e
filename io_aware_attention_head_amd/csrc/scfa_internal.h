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
// Position test of a call: the causal test or one of its variants, chosen by
// the flags SCFA_STRICT and SCFA_NONCAUSAL. Key position k is visible to
// query position q iff k_reach(k) <= q, equivalently iff k <= q_reach(q):
//   causal      k <= q
//   strict      k <= q - 1 (a key strictly before its query)
//   non-causal  every real key to every real query. Real positions lie
//               below 2^28; q_reach sets bit 28 of a real query position,
//               which then exceeds every real key and stays below the key
//               pad, and keeps the query pad -1; k_reach clears the low 28
//               bits of a key position, which maps every real key to 0 and
//               the key pad above every real query.
// Both maps are monotone, so the map of a tile's extremum is the extremum of
// its mapped positions: tile tests compare mapped extrema.
struct Reach {
  int st, qor, kand;
};
constexpr int kFlagMask = SCFA_STRICT | SCFA_NONCAUSAL;
constexpr int kPosLimit = 1 << 28;  // positions of a non-causal call lie below it
inline bool flags_ok(int f) { return !(f & ~kFlagMask) && f != kFlagMask; }
inline Reach reach_of(int f) {
  if (f & SCFA_NONCAUSAL) return Reach{0, kPosLimit, ~(kPosLimit - 1)};
  return Reach{(f & SCFA_STRICT) ? 1 : 0, 0, -1};
}
// Splits the flag bits off a mode argument: returns them, keeps the mode.
inline int take_flags(int& mode) {
  const int f = mode & kFlagMask;
  mode &= ~kFlagMask;
  return f;
}
__host__ __device__ inline int q_reach(const Reach& r, int q) { return (q - r.st) | r.qor; }
__host__ __device__ inline int k_reach(const Reach& r, int k) { return (k + r.st) & r.kand; }

// Number of lanes below this one whose bit is set in `mask` (wave64).
__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ inline void set_dev_err(int32_t* dev_err, int bit) {
  if (dev_err) atomicOr(dev_err, bit);
}

}  // namespace scfa
