// Forward sparse causal flash attention on gfx950 (CDNA4).
//
// What is computed (explainer "Faster Causal Attention Over Large Sequences
// Through Sparse Flash Attention", 3.4): for each query tile, the key tiles
// of its range [start, end) from the tile table (Algorithm 1 for QK-drop,
// Algorithm 2 for hash-sparse) are processed; inside a tile a key is visible
// iff k_idx <= q_idx (and, in hash mode, equal bucket). Softmax statistics
// are accumulated online with the guards of Algorithm 3: a running max of
// -inf is replaced by 0 before exponentiating, and a zero denominator
// leaves the output at zero. Outputs are written straight to the original
// token positions (postprocessing scatter of "3.2 Big-Picture
// Architecture", item 4) together with the natural-log LSE.
//
// MI355X design:
//  * One workgroup = 4 wave64s = one 128-row query tile; each wave owns 32
//    queries as two 16-query MFMA column blocks.
//  * Scores are computed TRANSPOSED, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: the accumulator then gives every lane one
//    query column and 4 keys per 16x16 block, so the row max needs one
//    in-lane pass plus two cross-lane steps, the row sum stays per lane until
//    the epilogue, and the output rescale is lane-local.
//  * O^T = V^T P^T reuses the S^T accumulator as the B operand after a cvt
//    to bf16; K rows are permuted when loaded as the A operand so that each
//    lane's 8 probabilities cover 8 CONSECUTIVE keys, which makes the V^T
//    operand one 16-byte LDS read (V is stored transposed by the gather).
//  * K rows and V^T rows are double-buffered in LDS (16 B XOR-swizzled
//    chunks), the next tile's global loads are in flight during the MFMAs.
//  * Fully visible tiles (decided from the tile extrema) skip the mask.
//  * Work order: longest query tiles first, and when B*H is a multiple of 8
//    each XCD owns whole heads so K/V tiles are reused from its own L2.
//  * float32 inputs use v_mfma_f32_16x16x4_f32 with the same data flow
//    (single-buffered LDS).

#include <math.h>

#include "scfa_mfma.h"

namespace scfa {
namespace {

constexpr int BM = SCFA_TILE_M;  // 128 query rows per workgroup
constexpr int BN = SCFA_TILE_N;  // 64 keys per tile
constexpr int HD = 64;           // head dimension
constexpr float kLn2 = 0.69314718055994530942f;

struct FwdParams {
  const void* q;
  const void* k;
  const void* vt;
  const int32_t* q_idx;
  const int32_t* k_idx;
  const int32_t* q_bkt;
  const int32_t* k_bkt;
  const int4* qstats;
  const int4* kstats;
  const int2* fwd_tab;
  const int32_t* order;  // launch order of (head, query tile) items, or null
  void* O;
  float* lse;
  int B, H, T;
  int Tk;    // valid key rows (extrema/ragged test)
  int Tpad;  // rows of the compacted / sorted buffers
  int nQt, nKt;
  float c;  // scale * log2(e)
};

template <typename TOUT>
__device__ inline void store4(TOUT* p, const f32x4& v);

template <>
__device__ inline void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <>
__device__ inline void store4<uint16_t>(uint16_t* p, const f32x4& v) {
  uint2 u;
  __bf16 h0 = static_cast<__bf16>(v[0]), h1 = static_cast<__bf16>(v[1]);
  __bf16 h2 = static_cast<__bf16>(v[2]), h3 = static_cast<__bf16>(v[3]);
  u.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
  u.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h2)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h3)) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

// Element type traits of the input path.
template <bool F32>
struct Tr;
template <>
struct Tr<false> {  // bf16
  static constexpr int ESZ = 2;
  static constexpr int CH = HD * ESZ / 16;  // 16-byte chunks per 64-element row = 8
  static constexpr int NBUF = 2;
};
template <>
struct Tr<true> {  // fp32
  static constexpr int ESZ = 4;
  static constexpr int CH = HD * ESZ / 16;  // 16
  static constexpr int NBUF = 1;
};

// Registers holding the next key tile while the current one is computed.
template <int LOADS>
struct TileRegs {
  u32x4 k[LOADS];
  u32x4 v[LOADS];
  int idx;
};

// Global -> registers: the K tile (64 contiguous rows) and the V^T tile
// (64 d-rows of 64 keys), 16 bytes per load, plus the tile's key positions
// (threads 0..63) and buckets (threads 64..127).
template <bool HASH, int ESZ, int CH, int LOADS>
__device__ __forceinline__ void tile_load(TileRegs<LOADS>& r, const uint8_t* kg, const uint8_t* vg, const int32_t* kig,
                                          const int32_t* kbg, int Tpad, int j, int tid) {
  constexpr int TILE_BYTES = BN * HD * ESZ;
  static_for<LOADS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int u = tid + 256 * i;
    r.k[i] = reinterpret_cast<const u32x4*>(kg + static_cast<size_t>(j) * TILE_BYTES)[u];
    const int d = u / CH, ch = u - d * CH;
    r.v[i] = *reinterpret_cast<const u32x4*>(vg + (static_cast<size_t>(d) * Tpad + j * BN) * ESZ + ch * 16);
  });
  if (tid < BN) r.idx = kig[j * BN + tid];
  else if (HASH && tid < 2 * BN) r.idx = kbg[j * BN + tid - BN];
}

// Registers -> LDS with 16-byte XOR swizzles (K rows: swz_k, V^T rows: d & 7).
template <bool HASH, int ESZ, int CH, int LOADS>
__device__ __forceinline__ void tile_store(const TileRegs<LOADS>& r, uint8_t* ks, uint8_t* vs, int32_t* kp, int32_t* kb,
                                           int tid) {
  static_for<LOADS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int u = tid + 256 * i;
    const int row = u / CH, ch = u - row * CH;
    *reinterpret_cast<u32x4*>(ks + row * HD * ESZ + ((ch ^ swz_k(row)) * 16)) = r.k[i];
    *reinterpret_cast<u32x4*>(vs + row * BN * ESZ + ((ch ^ (row & 7)) * 16)) = r.v[i];
  });
  if (tid < BN) kp[tid] = r.idx;
  else if (HASH && tid < 2 * BN) kb[tid - BN] = r.idx;
}

template <bool HASH, bool F32, bool ZERO_DROPPED, typename TOUT>
__global__ __launch_bounds__(256) void k_fwd(FwdParams p) {
  using TR = Tr<F32>;
  constexpr int ESZ = TR::ESZ, CH = TR::CH, NBUF = TR::NBUF;
  constexpr int TILE_BYTES = BN * HD * ESZ;        // K tile and V^T tile, bytes each
  constexpr int LOADS = TILE_BYTES / 16 / 256;     // 16-byte loads per thread per tile
  // K and V^T tiles; after the loop the same bytes stage the output tile.
  __shared__ __align__(16) uint8_t smem[2 * NBUF * TILE_BYTES];
  uint8_t(*Ks)[TILE_BYTES] = reinterpret_cast<uint8_t(*)[TILE_BYTES]>(smem);
  uint8_t(*Vs)[TILE_BYTES] = reinterpret_cast<uint8_t(*)[TILE_BYTES]>(smem + NBUF * TILE_BYTES);
  static_assert(2 * NBUF * TILE_BYTES >= BM * HD * sizeof(TOUT), "output staging does not fit");
  __shared__ __align__(16) int32_t Kp[NBUF][BN];
  __shared__ __align__(16) int32_t Kb[NBUF][BN];
  __shared__ int32_t Qi[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int BH = p.B * p.H;

  // ---- work item: (head, query tile), longest first, XCD-aware ----------
  int qt, bh;
  if (p.order) {
    const int it = p.order[blockIdx.x];
    bh = it / p.nQt;
    qt = it - bh * p.nQt;
  } else {
    const int x = blockIdx.x;
    if ((BH & 7) == 0) {
      const int hpx = BH >> 3, xcd = x & 7, slot = x >> 3;
      qt = p.nQt - 1 - slot / hpx;
      bh = xcd * hpx + slot % hpx;
    } else {
      qt = p.nQt - 1 - x / BH;
      bh = x % BH;
    }
  }
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.Tpad;
  const int2 rng = p.fwd_tab[static_cast<size_t>(bh) * p.nQt + qt];
  const int4 qs = p.qstats[static_cast<size_t>(bh) * p.nQt + qt];
  const int4* kst = p.kstats + static_cast<size_t>(bh) * p.nKt;
  if (tid < BM) Qi[tid] = p.q_idx[rowbase + qt * BM + tid];  // visible after the first barrier

  // ---- queries of this wave: B operand, positions, buckets --------------
  const int q0 = qt * BM + w * 32;
  int qpos[2], qbkt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 16 + r16;
    qpos[qb] = p.q_idx[rowbase + row];
    qbkt[qb] = HASH ? p.q_bkt[rowbase + row] : 0;
  }
  // extrema of this wave's real query rows (pad rows: position -1, their
  // results are never stored): a key tile is skipped by the whole wave when
  // it holds no pair visible to any of them, and unmasked when every pair is
  // visible to all of them.
  int wmin = kInt32Max, wmax = -1, wbmin = kInt32Max, wbmax = kInt32Min;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qpos[qb] >= 0) {
      wmin = min(wmin, qpos[qb]);
      wmax = max(wmax, qpos[qb]);
      wbmin = min(wbmin, qbkt[qb]);
      wbmax = max(wbmax, qbkt[qb]);
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    wmin = min(wmin, __shfl_xor(wmin, o));
    wmax = max(wmax, __shfl_xor(wmax, o));
    wbmin = min(wbmin, __shfl_xor(wbmin, o));
    wbmax = max(wbmax, __shfl_xor(wbmax, o));
  }
  bf16x8 Qb[2][2];   // bf16: [qb][ds]
  float Qf[2][16];   // fp32: [qb][t], d = 16g + t
  if constexpr (!F32) {
    const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (rowbase + q0) * HD;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ds = 0; ds < 2; ++ds)
        Qb[qb][ds] = *reinterpret_cast<const bf16x8*>(qg + (qb * 16 + r16) * HD + ds * 32 + g * 8);
  } else {
    const float* qg = static_cast<const float*>(p.q) + (rowbase + q0) * HD;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const float4 v = *reinterpret_cast<const float4*>(qg + (qb * 16 + r16) * HD + 16 * g + 4 * t4);
        Qf[qb][4 * t4 + 0] = v.x;
        Qf[qb][4 * t4 + 1] = v.y;
        Qf[qb][4 * t4 + 2] = v.z;
        Qf[qb][4 * t4 + 3] = v.w;
      }
  }

  f32x4 Oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) Oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  // ---- tile pipeline ------------------------------------------------------
  const uint8_t* kg = static_cast<const uint8_t*>(p.k) + rowbase * HD * ESZ;
  const uint8_t* vg = static_cast<const uint8_t*>(p.vt) + static_cast<size_t>(bh) * HD * p.Tpad * ESZ;
  const int32_t* kig = p.k_idx + rowbase;
  const int32_t* kbg = HASH ? p.k_bkt + rowbase : nullptr;
  TileRegs<LOADS> tr;

  auto next_tile = [&](int j) {
    while (j < rng.y && kst[j].x > qs.y) ++j;  // causal extremum test (hash ranges)
    return j;
  };

  int j = next_tile(rng.x);
  if (j < rng.y) {
    tile_load<HASH, ESZ, CH, LOADS>(tr, kg, vg, kig, kbg, p.Tpad, j, tid);
    tile_store<HASH, ESZ, CH, LOADS>(tr, Ks[0], Vs[0], Kp[0], Kb[0], tid);
  }
  __syncthreads();
  int buf = 0;
  while (j < rng.y) {
    const int jn = next_tile(j + 1);
    if (jn < rng.y) tile_load<HASH, ESZ, CH, LOADS>(tr, kg, vg, kig, kbg, p.Tpad, jn, tid);
    const int4 ks = kst[j];
    const bool wave_empty = ks.x > wmax || (HASH && (ks.w < wbmin || ks.z > wbmax));
    if (!wave_empty) {

    // -- S^T = K Q^T --------------------------------------------------------
    f32x4 S[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) S[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!F32) {
#pragma unroll
      for (int ds = 0; ds < 2; ++ds)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int row = key_row(kb, r16);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[buf][row * HD * 2 + (((ds * 4 + g) ^ swz_k(row)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qb[qb][ds], S[kb][qb], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = key_row(kb, r16);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const float4 a = *reinterpret_cast<const float4*>(&Ks[buf][row * HD * 4 + (((4 * g + t4) ^ swz_k(row)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, Qf[qb][4 * t4 + 0], S[kb][qb], 0, 0, 0);
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, Qf[qb][4 * t4 + 1], S[kb][qb], 0, 0, 0);
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, Qf[qb][4 * t4 + 2], S[kb][qb], 0, 0, 0);
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, Qf[qb][4 * t4 + 3], S[kb][qb], 0, 0, 0);
          }
        }
      }
    }

    // -- mask on tiles that are not fully visible ---------------------------
    bool full = ks.y <= wmin && (j + 1) * BN <= p.Tk;
    if (HASH) full = full && ks.z == ks.w && wbmin == wbmax && ks.z == wbmin;
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int kbase = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
        const int4 kp4 = *reinterpret_cast<const int4*>(&Kp[buf][kbase]);
        int4 kb4 = make_int4(0, 0, 0, 0);
        if (HASH) kb4 = *reinterpret_cast<const int4*>(&Kb[buf][kbase]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qp = qpos[qb], qh = qbkt[qb];
          if (!(kp4.x <= qp && (!HASH || kb4.x == qh))) S[kb][qb][0] = -INFINITY;
          if (!(kp4.y <= qp && (!HASH || kb4.y == qh))) S[kb][qb][1] = -INFINITY;
          if (!(kp4.z <= qp && (!HASH || kb4.z == qh))) S[kb][qb][2] = -INFINITY;
          if (!(kp4.w <= qp && (!HASH || kb4.w == qh))) S[kb][qb][3] = -INFINITY;
        }
      }
    }

    // -- online softmax (base 2, scale folded into the exponent) -----------
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = fmaxf(S[0][qb][0], S[0][qb][1]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = (kb == 0 ? 2 : 0); e < 4; e += 2) mx = fmaxf(mx, fmaxf(S[kb][qb][e], S[kb][qb][e + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[qb], mx * p.c);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - muse);
      m[qb] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(S[kb][qb][e], p.c, -muse));
          S[kb][qb][e] = pv;
          ls += pv;
        }
      l[qb] = l[qb] * alpha + ls;
      if (__ballot(alpha != 1.f)) {  // the running max moved for some query of this wave
#pragma unroll
        for (int db = 0; db < 4; ++db) Oacc[db][qb] *= alpha;
      }
    }

    // -- O^T += V^T P^T -----------------------------------------------------
    if constexpr (!F32) {
      bf16x8 P[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) P[qb][kc] = pack_bf16x8(S[2 * kc][qb], S[2 * kc + 1][qb]);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int d = db * 16 + r16;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vs[buf][d * BN * 2 + (((kc * 4 + g) ^ (d & 7)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[qb][kc], Oacc[db][qb], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 16 + r16;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int ch = 8 * (kb >> 1) + 2 * g + (kb & 1);  // keys 32kc + 8g + 4hb + 0..3
          const float4 a = *reinterpret_cast<const float4*>(&Vs[buf][d * BN * 4 + ((ch ^ (d & 7)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, S[kb][qb][0], Oacc[db][qb], 0, 0, 0);
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, S[kb][qb][1], Oacc[db][qb], 0, 0, 0);
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, S[kb][qb][2], Oacc[db][qb], 0, 0, 0);
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, S[kb][qb][3], Oacc[db][qb], 0, 0, 0);
          }
        }
      }
    }

    }  // !wave_empty

    if constexpr (NBUF == 2) {
      if (jn < rng.y) tile_store<HASH, ESZ, CH, LOADS>(tr, Ks[buf ^ 1], Vs[buf ^ 1], Kp[buf ^ 1], Kb[buf ^ 1], tid);
      __syncthreads();
      buf ^= 1;
    } else {
      __syncthreads();
      if (jn < rng.y) tile_store<HASH, ESZ, CH, LOADS>(tr, Ks[0], Vs[0], Kp[0], Kb[0], tid);
      __syncthreads();
    }
    j = jn;
  }

  // ---- epilogue: normalise, stage the tile in LDS, write whole rows --------
  // Output units of 4 elements (16 B fp32 / 8 B bf16), 16 per row, XOR
  // swizzled by row so the column-wise staging writes are conflict-free.
  TOUT* ost = reinterpret_cast<TOUT*>(smem);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb] + __shfl_xor(l[qb], 16);
    lt = lt + __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float muse = (m[qb] == -INFINITY) ? 0.f : m[qb];
    const float lse = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
    const int row = w * 32 + qb * 16 + r16;
#pragma unroll
    for (int db = 0; db < 4; ++db) store4<TOUT>(ost + row * HD + (((4 * db + g) ^ (row & 15)) * 4), Oacc[db][qb] * inv);
    const int qp = qpos[qb];
    if (g == 0 && qp >= 0 && qp < p.T) p.lse[static_cast<size_t>(bh) * p.T + qp] = lse;
  }
  __syncthreads();
  TOUT* O = static_cast<TOUT*>(p.O);
#pragma unroll
  for (int it = 0; it < BM / 16; ++it) {
    const int row = it * 16 + (tid >> 4), u = tid & 15;
    const int qp = Qi[row];
    if (qp >= 0 && qp < p.T) {
      TOUT* orow = O + ((static_cast<size_t>(b) * p.T + qp) * p.H + h) * HD;
      const TOUT* src = ost + row * HD + ((u ^ (row & 15)) * 4);
      if constexpr (sizeof(TOUT) == 4)
        *reinterpret_cast<uint4*>(orow + u * 4) = *reinterpret_cast<const uint4*>(src);
      else
        *reinterpret_cast<uint2*>(orow + u * 4) = *reinterpret_cast<const uint2*>(src);
    }
  }

  // ---- QK-drop: zero the dropped queries this tile owns ------------------
  // Tile qt owns the original positions after the previous tile's last kept
  // query up to its own last kept query (the last tile holding kept queries
  // also owns everything after it; with no kept query at all, tile 0 owns
  // the whole sequence). Positions in that range that are not among the
  // tile's queries were dropped: O = 0, LSE = -inf.
  if constexpr (ZERO_DROPPED) {
    const int nreal = __syncthreads_count(tid < BM && Qi[tid] >= 0);
    int lo = 0, hi = -1;
    if (nreal > 0) {
      lo = qt == 0 ? 0 : max(0, p.q_idx[rowbase + qt * BM - 1] + 1);
      const bool next_real = (qt + 1) * BM < p.Tpad && p.q_idx[rowbase + (qt + 1) * BM] >= 0;
      hi = next_real ? min(Qi[nreal - 1], p.T - 1) : p.T - 1;
    } else if (qt == 0) {
      lo = 0;
      hi = p.T - 1;
    }
    constexpr int UPR = HD * sizeof(TOUT) / 16;  // 16-byte units per output row
    constexpr int RPI = 256 / UPR;               // rows per iteration
    for (int base = lo; base <= hi; base += RPI) {
      const int pos = base + tid / UPR;
      const int u = tid % UPR;
      if (pos <= hi) {
        int a = 0, z = nreal;  // binary search pos among the tile's kept positions
        while (a < z) {
          const int mid = (a + z) >> 1;
          if (Qi[mid] < pos) a = mid + 1; else z = mid;
        }
        if (!(a < nreal && Qi[a] == pos)) {
          TOUT* orow = O + ((static_cast<size_t>(b) * p.T + pos) * p.H + h) * HD;
          reinterpret_cast<uint4*>(orow)[u] = make_uint4(0, 0, 0, 0);
          if (u == 0) p.lse[static_cast<size_t>(bh) * p.T + pos] = -INFINITY;
        }
      }
    }
  }
}

template <bool HASH, bool F32, bool ZD, typename TOUT>
int launch_fwd(const FwdParams& p, hipStream_t stream) {
  const int grid = p.nQt * p.B * p.H;
  hipLaunchKernelGGL((k_fwd<HASH, F32, ZD, TOUT>), dim3(grid), dim3(256), 0, stream, p);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

template <bool HASH, bool ZD>
int dispatch_fwd(int dtype_in, int dtype_out, const FwdParams& p, hipStream_t stream) {
  if (dtype_in == SCFA_BF16) {
    if (dtype_out == SCFA_F32) return launch_fwd<HASH, false, ZD, float>(p, stream);
    return launch_fwd<HASH, false, ZD, uint16_t>(p, stream);
  }
  if (dtype_out == SCFA_F32) return launch_fwd<HASH, true, ZD, float>(p, stream);
  return launch_fwd<HASH, true, ZD, uint16_t>(p, stream);
}

int check_common(int dtype_in, int dtype_out, int B, int H, int T, int D, float scale) {
  if (!dtype_ok(dtype_in) || !dtype_ok(dtype_out)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1) return SCFA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SCFA_ERR_INVALID;
  if (D != HD) return SCFA_ERR_UNSUPPORTED;
  return SCFA_OK;
}

}  // namespace
}  // namespace scfa

using namespace scfa;

extern "C" {

int scfa_qk_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v_t,
                       const int32_t* q_idx, const int32_t* k_idx, const int32_t* qstats, const int32_t* kstats,
                       const int32_t* fwd_tab, const int32_t* order, int B, int H, int T, int Tc, int D, float scale,
                       void* O, float* lse, hipStream_t stream) {
  if (!q || !k || !v_t || !q_idx || !k_idx || !qstats || !kstats || !fwd_tab || !O || !lse) return SCFA_ERR_INVALID;
  const int st = check_common(dtype_in, dtype_out, B, H, T, D, scale);
  if (st != SCFA_OK) return st;
  if (Tc < SCFA_ROW_ALIGN || Tc % SCFA_ROW_ALIGN) return SCFA_ERR_INVALID;
  FwdParams p{};
  p.q = q;
  p.k = k;
  p.vt = v_t;
  p.q_idx = q_idx;
  p.k_idx = k_idx;
  p.q_bkt = nullptr;
  p.k_bkt = nullptr;
  p.qstats = reinterpret_cast<const int4*>(qstats);
  p.kstats = reinterpret_cast<const int4*>(kstats);
  p.fwd_tab = reinterpret_cast<const int2*>(fwd_tab);
  p.order = order;
  p.O = O;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.T = T;
  p.Tk = Tc;
  p.Tpad = Tc;
  p.nQt = Tc / BM;
  p.nKt = Tc / BN;
  p.c = scale * 1.44269504088896340736f;
  return dispatch_fwd<false, true>(dtype_in, dtype_out, p, stream);
}

int scfa_hash_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v_t,
                         const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt,
                         const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, const int32_t* order,
                         int B, int H, int T, int D, float scale, void* O, float* lse, hipStream_t stream) {
  if (!q || !k || !v_t || !q_idx || !k_idx || !q_bkt || !k_bkt || !qstats || !kstats || !fwd_tab || !O || !lse)
    return SCFA_ERR_INVALID;
  const int st = check_common(dtype_in, dtype_out, B, H, T, D, scale);
  if (st != SCFA_OK) return st;
  const int Tp = pad_rows(T);
  FwdParams p{};
  p.q = q;
  p.k = k;
  p.vt = v_t;
  p.q_idx = q_idx;
  p.k_idx = k_idx;
  p.q_bkt = q_bkt;
  p.k_bkt = k_bkt;
  p.qstats = reinterpret_cast<const int4*>(qstats);
  p.kstats = reinterpret_cast<const int4*>(kstats);
  p.fwd_tab = reinterpret_cast<const int2*>(fwd_tab);
  p.order = order;
  p.O = O;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.T = T;
  p.Tk = T;
  p.Tpad = Tp;
  p.nQt = Tp / BM;
  p.nKt = Tp / BN;
  p.c = scale * 1.44269504088896340736f;
  return dispatch_fwd<true, false>(dtype_in, dtype_out, p, stream);
}

}  // extern "C"
