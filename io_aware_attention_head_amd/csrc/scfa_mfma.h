// MFMA data-layout helpers shared by the attention kernels (gfx950).
//
// v_mfma_f32_16x16x32_bf16 operand layouts (lane l, g = l / 16):
//   A (16 x 32): lane l holds row l % 16, k = 8g .. 8g+7
//   B (32 x 16): lane l holds column l % 16, k = 8g .. 8g+7
//   C (16 x 16): lane l holds column l % 16, rows 4g .. 4g+3
// Only the M/N placement matters for a contraction: any mapping of k to
// (g, element) works as long as A and B use the same one.
#pragma once

#include "scfa_internal.h"

namespace scfa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));


constexpr float kLog2e = 1.44269504088896340736f;

// Key row of MFMA A-operand row r (0..15) for 16-key block kb of a 64-key
// tile: blocks 2kc and 2kc+1 interleave in groups of 4 so that accumulator
// element e of lane group g in block kb is key 32kc + 8g + 4(kb&1) + e.
__device__ inline int key_row(int kb, int r) { return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3); }
__device__ inline int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }

__device__ inline bf16x8 pack_bf16x8(const f32x4& a, const f32x4& b) {
  bf16x8 r;
  r[0] = static_cast<__bf16>(a[0]);
  r[1] = static_cast<__bf16>(a[1]);
  r[2] = static_cast<__bf16>(a[2]);
  r[3] = static_cast<__bf16>(a[3]);
  r[4] = static_cast<__bf16>(b[0]);
  r[5] = static_cast<__bf16>(b[1]);
  r[6] = static_cast<__bf16>(b[2]);
  r[7] = static_cast<__bf16>(b[3]);
  return r;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for_impl<I + 1, N>(f);
  }
}
// Calls f(IntC<0>), ..., f(IntC<N-1>): compile-time indices for register arrays.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}


}  // namespace scfa
