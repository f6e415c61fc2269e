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
//  * The gather of the explainer's preprocessing ("Gather: Reordering Q, K,
//    V according to the sorted indices") is fused into the loads: query rows
//    and the key/value rows of each tile are read from the original
//    (B, T, H, D) tensors through q_idx / k_idx. Rows of pad entries read
//    token 0 instead (finite values; pad queries are never stored and pad
//    keys are always masked).
//  * One workgroup = 4 wave64s = one 128-row query tile; each wave owns 32
//    queries as two 16-query MFMA column blocks.
//  * Scores are computed TRANSPOSED, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: the accumulator then gives every lane one
//    query column and 4 keys per 16x16 block, so the row max needs one
//    in-lane pass plus two cross-lane steps and the output rescale is
//    lane-local.
//  * O^T = V^T P^T reuses the S^T accumulator as the B operand after a cvt
//    to bf16; K rows are permuted when loaded as the A operand so that each
//    lane's 8 probabilities cover 8 CONSECUTIVE keys. The V^T operand is
//    read from the row-major V tile with the LDS transpose read
//    (ds_read_b64_tr_b16: 16 lanes exchange a 16 x 4 block of 16-bit values).
//    K and V tiles share one layout whose 16-byte chunks are XOR-swizzled by
//    row, which keeps the K row reads free of bank conflicts.
//  * K and V tiles are staged by global-to-LDS DMA (no registers), double
//    buffered; the key positions of the tile after next are prefetched into
//    registers one tile ahead, so DMA addresses never wait on a load.
//  * Speculative reference max: a tile's weights are exponentiated against
//    the current reference without looking at the tile's max; the row max is
//    taken only for a row's first tile with a visible key, or when some weight
//    exceeds 2^64 (then the weights are recomputed), so the O rescale is rare
//    and the per-tile max reduction is gone. O and the LSE use the fp32 row
//    sum of the probabilities. (The fp32 kernel keeps an exact running max.)
//  * Per-wave tile tests from the extrema: a key tile holding no pair visible
//    to any of the wave's 32 queries is skipped by that wave, and one whose
//    pairs are all visible skips the mask. The tests of 64 key tiles at a time
//    are taken at once (one tile per lane) and kept as wave-uniform bit masks,
//    so the tile loop reads no statistics.
//  * Work order: a launch order (longest query tiles first, XCD-aware) from
//    scfa_work_order, or descending query-tile index.
//  * float32 inputs use v_mfma_f32_16x16x4_f32 in a single-buffered kernel
//    with the same data flow.

#include <math.h>

#include "scfa_stage.h"

namespace scfa {
namespace {

constexpr int BM = SCFA_TILE_M;  // 128 query rows per workgroup
constexpr int BN = SCFA_TILE_N;  // 64 keys per tile
constexpr int HD = 64;           // head dimension
constexpr float kLn2 = 0.69314718055994530942f;
// Largest lane sum of 16 weights accepted against a reference max (bf16
// kernel): weights up to 2^64 keep O, the row sums and their bf16 copies far
// from the fp32 range limits.
constexpr float kSpecCap = 18446744073709551616.0f;  // 2^64

struct FwdParams {
  const void* q;  // (B, T, H, D) original order, as are k and v
  const void* k;
  const void* v;
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
  int Tkv;   // tokens of the original k and v tensors (B, Tkv, H, D)
  int Tk;    // valid key rows (extrema/ragged test)
  int TqPad;  // rows per head of the query-side index arrays (q_idx, q_bkt)
  int TkPad;  // rows per head of the key-side index arrays (k_idx, k_bkt)
  int nQt, nKt;
  float c;     // scale * log2(e)
  Reach rc;  // position test (causal, strict or non-causal)
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

// Work item of this workgroup: (head, query tile).
__device__ inline void pick_work(const FwdParams& p, int& qt, int& bh) {
  const int BH = p.B * p.H;
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
}

// Max (log2 units) of the 16 scores a lane holds for query column qb
// (max3 chains).
__device__ inline float lane_max_scaled(const f32x4 (&S)[4][2], int qb, float c) {
  float mx = fmaxf(S[0][qb][0], fmaxf(S[0][qb][1], S[0][qb][2]));
#pragma unroll
  for (int i = 3; i < 15; i += 2)
    mx = fmaxf(mx, fmaxf(S[i >> 2][qb][i & 3], S[(i + 1) >> 2][qb][(i + 1) & 3]));
  mx = fmaxf(mx, S[3][qb][3]);
  return mx * c;
}

// Max over the 4 lane groups that hold the same query column.
__device__ inline float group_max(float mx) {
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// Row max (log2 units) of a score tile.
__device__ inline float row_max_scaled(const f32x4 (&S)[4][2], int qb, float c) {
  return group_max(lane_max_scaled(S, qb, c));
}

// Epilogue: normalise, stage the tile in LDS, write whole rows at the
// original positions, LSE; in QK-drop mode zero the dropped queries the tile
// owns. `ost` must hold BM * HD * sizeof(TOUT) bytes of LDS.
template <bool ZERO_DROPPED, typename TOUT>
__device__ inline void fwd_epilogue(const FwdParams& p, TOUT* ost, const int32_t* Qi, const f32x4 (&Oacc)[4][2],
                                    const float (&inv)[2], const float (&lse)[2], const int (&qpos)[2], int qt, int bh,
                                    size_t rowbase) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int b = bh / p.H, h = bh - b * p.H;
  // Output units of 4 elements (16 B fp32 / 8 B bf16), 16 per row, XOR
  // swizzled by row so the column-wise staging writes are conflict-free.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = w * 32 + qb * 16 + r16;
#pragma unroll
    for (int db = 0; db < 4; ++db) store4<TOUT>(ost + row * HD + (((4 * db + g) ^ (row & 15)) * 4), Oacc[db][qb] * inv[qb]);
    const int qp = qpos[qb];
    if (g == 0 && qp >= 0 && qp < p.T) p.lse[static_cast<size_t>(bh) * p.T + qp] = lse[qb];
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

  // QK-drop: tile qt owns the original positions after the previous tile's
  // last kept query up to its own last kept query (the last tile holding kept
  // queries also owns everything after it; with no kept query at all, tile 0
  // owns the whole sequence). Positions in that range that are not among the
  // tile's queries were dropped: O = 0, LSE = -inf.
  if constexpr (ZERO_DROPPED) {
    const int nreal = __syncthreads_count(tid < BM && Qi[tid] >= 0);
    int lo = 0, hi = -1;
    if (nreal > 0) {
      lo = qt == 0 ? 0 : max(0, p.q_idx[rowbase + qt * BM - 1] + 1);
      const bool next_real = (qt + 1) * BM < p.TqPad && p.q_idx[rowbase + (qt + 1) * BM] >= 0;
      hi = next_real ? min(Qi[nreal - 1], p.T - 1) : p.T - 1;
    } else if (qt == 0) {
      lo = 0;
      hi = p.T - 1;
    }
    // 256 positions per pass, one per thread: the tile's kept positions in
    // the pass's window are flagged in LDS, and each thread writes the whole
    // row of its position when that is not flagged
    constexpr int UPR = HD * sizeof(TOUT) / 16;  // 16-byte units per output row
    __shared__ uint8_t kept_w[256];
    for (int base = lo; base <= hi; base += 256) {
      kept_w[tid] = 0;
      __syncthreads();
      if (tid < nreal) {
        const int d = Qi[tid] - base;
        if (d >= 0 && d < 256) kept_w[d] = 1;
      }
      __syncthreads();
      const int pos = base + tid;
      if (pos <= hi && !kept_w[tid]) {
        uint4* orow = reinterpret_cast<uint4*>(O + ((static_cast<size_t>(b) * p.T + pos) * p.H + h) * HD);
#pragma unroll
        for (int u = 0; u < UPR; ++u) orow[u] = make_uint4(0, 0, 0, 0);
        p.lse[static_cast<size_t>(bh) * p.T + pos] = -INFINITY;
      }
      __syncthreads();  // kept_w is cleared for the next pass
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs.
// ---------------------------------------------------------------------------


// S^T += K Q^T for one staged key tile: 2 x 4 x 2 MFMAs over the two
// 32-wide halves of D. K rows are read permuted (key_row) so that each
// lane's accumulator elements are consecutive keys.
__device__ __forceinline__ void scores_bf16(f32x4 (&S)[4][2], const uint8_t* Ks, const bf16x8 (&Qb)[2][2], int r16,
                                            int g) {
#pragma unroll
  for (int ds = 0; ds < 2; ++ds)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 a = read_row_op(Ks, kb, r16, ds * 4 + g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qb[qb][ds], S[kb][qb], 0, 0, 0);
    }
}

template <bool HASH, bool ZERO_DROPPED, typename TOUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_fwd_bf16(FwdParams p) {
  constexpr int TB = BN * HD * 2;  // K tile and V tile, bytes each (8 KB)
  // Two stages of (K, V); after the loop the same bytes stage the output.
  __shared__ __align__(16) uint8_t smem[4 * TB];
  static_assert(4 * TB >= BM * HD * sizeof(TOUT), "output staging does not fit");
  __shared__ __align__(16) int32_t Kp[2][BN];
  __shared__ __align__(16) int32_t Kb[2][BN];
  __shared__ int32_t Qi[BM];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  int qt, bh;
  pick_work(p, qt, bh);
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqPad;  // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkPad;    // key side
  const int2 rng = p.fwd_tab[static_cast<size_t>(bh) * p.nQt + qt];
  const int4 qs = p.qstats[static_cast<size_t>(bh) * p.nQt + qt];
  const int qreach = q_reach(p.rc, qs.y);  // largest key position a query of the tile may see
  const int4* kst = p.kstats + static_cast<size_t>(bh) * p.nKt;
  // index entries of the tile (to LDS before the first barrier; loaded here with
  // the table so the stores wait on nothing later)
  const int qi_v = tid < BM ? p.q_idx[rowbase + qt * BM + tid] : 0;
  const uint32_t rstride = static_cast<uint32_t>(p.H) * HD * 2;  // bytes between token rows
  const size_t head0 = (static_cast<size_t>(b) * p.T * p.H + h) * HD * 2;     // token 0 of this head in q
  const size_t khead0 = (static_cast<size_t>(b) * p.Tkv * p.H + h) * HD * 2;  // and in k, v

  // ---- queries of this wave: B operand, positions, buckets --------------
  const int q0 = qt * BM + w * 32;
  int qpos[2], qbkt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 16 + r16;
    qpos[qb] = p.q_idx[rowbase + row];
    qbkt[qb] = HASH ? p.q_bkt[rowbase + row] : 0;
  }
  TileWalk<HASH> walk(kst, rng.x, rng.y, lane);  // tile tests of the range, 64 tiles per window
  const WaveRows wr = wave_rows(qpos, qbkt, p.rc);
  // positions the masks compare keys against: the largest visible key position
  const int qcmp[2] = {q_reach(p.rc, qpos[0]), q_reach(p.rc, qpos[1])};
  bf16x8 Qb[2][2];  // [qb][ds]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint8_t* qrow = static_cast<const uint8_t*>(p.q) + head0 +
                          static_cast<size_t>(src_row(qpos[qb], p.T)) * rstride;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) Qb[qb][ds] = *reinterpret_cast<const bf16x8*>(qrow + (ds * 32 + g * 8) * 2);
  }

  f32x4 Oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) Oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};  // fp32 row sums (per lane: its 16 keys of each tile)

  // ---- DMA staging of a key tile -----------------------------------------
  // Wave w stages rows 16w .. 16w+15 of the K and V tiles, 8 rows (1 KB) per
  // instruction: lane l writes chunk position l % 8 of row 16w + 8i + l / 8
  // and reads the chunk of that row's token that the swizzle puts there.
  const uint8_t* kg = static_cast<const uint8_t*>(p.k) + khead0;
  const uint8_t* vg = static_cast<const uint8_t*>(p.v) + khead0;
  const int32_t* kig = p.k_idx + kbase;
  const int32_t* kbg = HASH ? p.k_bkt + kbase : nullptr;
  uint32_t kch[2];  // K and V tiles share the swz_k layout
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * w + 8 * i + (lane >> 3), cp = lane & 7;
    kch[i] = (cp ^ swz_k(row)) * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t ldsp = lds_addr(&Kp[0][0]), ldsb = lds_addr(&Kb[0][0]);
  // positions of the rows this lane stages for key tile j
  auto tile_rows = [&](int j, int (&pos)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) pos[i] = kig[min(j, p.nKt - 1) * BN + 16 * w + 8 * i + (lane >> 3)];
  };
  auto stage_tile = [&](int j, int s, const int (&pos)[2]) {
    const uint32_t ks = lds0 + s * TB + ws * 2048, vs = lds0 + (2 + s) * TB + ws * 2048;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = static_cast<uint32_t>(src_row(pos[i], p.Tkv)) * rstride;
      dma16(kg, off + kch[i], ks + i * 1024);
      dma16(vg, off + kch[i], vs + i * 1024);
    }
    if (ws == 0) dma4(kig + j * BN, lane * 4, ldsp + s * BN * 4);
    else if (HASH && ws == 1) dma4(kbg + j * BN, lane * 4, ldsb + s * BN * 4);
  };

  auto tests = [&](const int4& st, int jj) { return key_tile_masks<HASH>(st, jj, rng.y, qreach, wr, p.Tk); };
  walk.first(tests);

  // The first tile of the range is staged at once (a tile failing the causal
  // extremum test is skipped by every wave's own test), so the table, query
  // and key loads form as short a chain as possible.
  int j = rng.x < rng.y ? rng.x : rng.y;
  int pos[2];
  if (j < rng.y) {
    tile_rows(j, pos);
    stage_tile(j, 0, pos);
  }
  if (tid < BM) Qi[tid] = qi_v;  // published by the barriers below
  int jn = j < rng.y ? walk.next(j + 1, tests) : rng.y;
  tile_rows(jn, pos);  // rows of the next tile, used by the first iteration
  dma_wait();
  __syncthreads();
  int s = 0;
  while (j < rng.y) {
    walk.enter(j, tests);
    const int jnn = jn < rng.y ? walk.next(jn + 1, tests) : rng.y;
    // the rows of the tile after next are loaded before the DMA, so that
    // waiting for them never waits for it
    int pos_nn[2];
    tile_rows(jnn, pos_nn);
    __builtin_amdgcn_sched_barrier(0);
    if (jn < rng.y) stage_tile(jn, s ^ 1, pos);

    if (!walk.has(walk.cw.empty, j)) {
      const uint8_t* Ks = smem + s * TB;
      const uint8_t* Vs = smem + (2 + s) * TB;
      // -- S^T = K Q^T ------------------------------------------------------
      // A tile that is not fully visible starts the accumulators at the
      // mask bias (0 or -inf), so masked scores come out of the MFMAs as
      // -inf; both branches define S afresh.
      f32x4 S[4][2];
      if (walk.has(walk.cw.full, j)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) S[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        scores_bf16(S, Ks, Qb, r16, g);
      } else {
        if (HASH && walk.has(walk.cw.mixed, j))
          bias_tile<true>(S, Kp[s], Kb[s], qcmp, qbkt, g);
        else
          bias_tile<false>(S, Kp[s], Kb[s], qcmp, qbkt, g);
        scores_bf16(S, Ks, Qb, r16, g);
      }
      // -- online softmax, speculative reference ------------------------------
      // The weights are exponentiated against the current reference max
      // without looking at this tile's max; the row max is taken only while a
      // row of the wave has no reference yet (its first tile with a visible
      // key) or when some weight of the tile exceeds 2^kSpec (a lane's sum of
      // its 16 weights above 2^kSpec, or not finite); then the reference
      // moves to the row max and the weights are recomputed.
      bf16x8 P[2][2];
      float ls[2];
      auto expo = [&](int qb, float muse) {
        float sum = 0.f;
        f32x4 t[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            t[kb][e] = __builtin_amdgcn_exp2f(fmaf(S[kb][qb][e], p.c, -muse));
            sum += t[kb][e];
          }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) P[qb][kc] = pack_bf16x8(t[2 * kc], t[2 * kc + 1]);
        return sum;
      };
      bool need_max = __ballot(m[0] == -INFINITY || m[1] == -INFINITY) != 0;
      if (!need_max) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) ls[qb] = expo(qb, m[qb]);
        need_max = __ballot(!(ls[0] <= kSpecCap) || !(ls[1] <= kSpecCap)) != 0;
      }
      if (need_max) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mnew = fmaxf(m[qb], row_max_scaled(S, qb, p.c));
          const float muse = (mnew == -INFINITY) ? 0.f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - muse);  // 1 when unchanged, 0 from -inf
          m[qb] = mnew;
#pragma unroll
          for (int db = 0; db < 4; ++db) Oacc[db][qb] *= alpha;
          l[qb] *= alpha;
          ls[qb] = expo(qb, muse);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) l[qb] += ls[qb];

      // -- O^T += V^T P^T ------------------------------------------------------
      // V^T operand of (db, kc): dims 16db + r16, keys 32kc + 8g + 0..7. The
      // key halves are the outer loop, so the two MFMAs that accumulate into
      // one O block are eight apart.
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a = read_tr_op(Vs, db, kc, g, r16);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[qb][kc], Oacc[db][qb], 0, 0, 0);
        }
    }

    dma_wait();
    __syncthreads();
    s ^= 1;
    j = jn;
    jn = jnn;
    pos[0] = pos_nn[0];
    pos[1] = pos_nn[1];
  }

  // ---- epilogue --------------------------------------------------------------
  float inv[2], lse[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb] + __shfl_xor(l[qb], 16);
    lt = lt + __shfl_xor(lt, 32);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const float muse = (m[qb] == -INFINITY) ? 0.f : m[qb];
    lse[qb] = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
  }
  fwd_epilogue<ZERO_DROPPED, TOUT>(p, reinterpret_cast<TOUT*>(smem), Qi, Oacc, inv, lse, qpos, qt, bh, rowbase);
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_16x16x4_f32, single-buffered LDS, same layout.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZERO_DROPPED, typename TOUT>
__global__ __launch_bounds__(256) void k_fwd_f32(FwdParams p) {
  constexpr int TB = BN * HD * 4;  // 16 KB
  __shared__ __align__(16) uint8_t smem[2 * TB];
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + TB;
  static_assert(2 * TB >= BM * HD * sizeof(TOUT), "output staging does not fit");
  __shared__ __align__(16) int32_t Kp[BN];
  __shared__ __align__(16) int32_t Kb[BN];
  __shared__ int32_t Qi[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  int qt, bh;
  pick_work(p, qt, bh);
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqPad;  // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkPad;    // key side
  const int2 rng = p.fwd_tab[static_cast<size_t>(bh) * p.nQt + qt];
  const int4 qs = p.qstats[static_cast<size_t>(bh) * p.nQt + qt];
  const int qreach = q_reach(p.rc, qs.y);  // largest key position a query of the tile may see
  const int4* kst = p.kstats + static_cast<size_t>(bh) * p.nKt;
  if (tid < BM) Qi[tid] = p.q_idx[rowbase + qt * BM + tid];
  const size_t rstride = static_cast<size_t>(p.H) * HD;                 // floats between token rows
  const size_t head0 = (static_cast<size_t>(b) * p.T * p.H + h) * HD;     // token 0 of this head in q
  const size_t khead0 = (static_cast<size_t>(b) * p.Tkv * p.H + h) * HD;  // and in k, v

  const int q0 = qt * BM + w * 32;
  int qpos[2], qbkt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 16 + r16;
    qpos[qb] = p.q_idx[rowbase + row];
    qbkt[qb] = HASH ? p.q_bkt[rowbase + row] : 0;
  }
  const WaveRows wr = wave_rows(qpos, qbkt, p.rc);
  // positions the masks compare keys against: the largest visible key position
  const int qcmp[2] = {q_reach(p.rc, qpos[0]), q_reach(p.rc, qpos[1])};
  float Qf[2][16];  // [qb][t], d = 16g + t
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float* qrow = static_cast<const float*>(p.q) + head0 + src_row(qpos[qb], p.T) * rstride;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const float4 v = *reinterpret_cast<const float4*>(qrow + 16 * g + 4 * t4);
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

  const float* kg = static_cast<const float*>(p.k) + khead0;
  const float* vg = static_cast<const float*>(p.v) + khead0;
  const int32_t* kig = p.k_idx + kbase;
  const int32_t* kbg = HASH ? p.k_bkt + kbase : nullptr;

  for (int j = rng.x; j < rng.y; ++j) {
    if (kst[j].x > qreach) continue;  // causal extremum test (uniform)
    __syncthreads();  // previous tile no longer read
    // K and V rows of the tile (16 chunks of 16 bytes per row), through k_idx
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i, row = u >> 4, ch = u & 15;
      const size_t off = src_row(kig[j * BN + row], p.Tkv) * rstride + ch * 4;
      const float4 kr = *reinterpret_cast<const float4*>(kg + off);
      const float4 vr = *reinterpret_cast<const float4*>(vg + off);
      *reinterpret_cast<float4*>(Ks + row * HD * 4 + ((ch ^ swz_k(row)) * 16)) = kr;
      *reinterpret_cast<float4*>(Vs + row * HD * 4 + ch * 16) = vr;
    }
    if (tid < BN) Kp[tid] = kig[j * BN + tid];
    else if (HASH && tid < 2 * BN) Kb[tid - BN] = kbg[j * BN + tid - BN];
    __syncthreads();
    if (tile_empty_for<HASH>(kst[j], wr)) continue;

    f32x4 S[4][2];  // starts at the mask bias (0 or -inf) unless all pairs are visible
    if (tile_full_for<HASH>(kst[j], wr, j, p.Tk)) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) S[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      mask_bias<HASH>(S, kst[j], wr, Kp, Kb, qcmp, qbkt, g);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = key_row(kb, r16);
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const float4 a = *reinterpret_cast<const float4*>(&Ks[row * HD * 4 + (((4 * g + t4) ^ swz_k(row)) * 16)]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, Qf[qb][4 * t4 + 0], S[kb][qb], 0, 0, 0);
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, Qf[qb][4 * t4 + 1], S[kb][qb], 0, 0, 0);
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, Qf[qb][4 * t4 + 2], S[kb][qb], 0, 0, 0);
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, Qf[qb][4 * t4 + 3], S[kb][qb], 0, 0, 0);
        }
      }
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mnew = fmaxf(m[qb], row_max_scaled(S, qb, p.c));
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
#pragma unroll
      for (int db = 0; db < 4; ++db) Oacc[db][qb] *= alpha;
    }

    // O^T += V^T P^T: the A operand of block kb, element e is V[key][d] for
    // key 32 (kb >> 1) + 8 g + 4 (kb & 1) + e, d = 16 db + r16.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 16 + r16;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key0 = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
        const float* vcol = reinterpret_cast<const float*>(Vs) + key0 * HD + d;
        const float a0 = vcol[0], a1 = vcol[HD], a2 = vcol[2 * HD], a3 = vcol[3 * HD];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, S[kb][qb][0], Oacc[db][qb], 0, 0, 0);
          Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, S[kb][qb][1], Oacc[db][qb], 0, 0, 0);
          Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, S[kb][qb][2], Oacc[db][qb], 0, 0, 0);
          Oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, S[kb][qb][3], Oacc[db][qb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // LDS tiles no longer read: the epilogue reuses them

  float inv[2], lse[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb] + __shfl_xor(l[qb], 16);
    lt = lt + __shfl_xor(lt, 32);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const float muse = (m[qb] == -INFINITY) ? 0.f : m[qb];
    lse[qb] = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
  }
  fwd_epilogue<ZERO_DROPPED, TOUT>(p, reinterpret_cast<TOUT*>(smem), Qi, Oacc, inv, lse, qpos, qt, bh, rowbase);
}

template <bool HASH, bool ZD>
int dispatch_fwd(int dtype_in, int dtype_out, const FwdParams& p, hipStream_t stream) {
  const dim3 grid(p.nQt * p.B * p.H), block(256);
  if (dtype_in == SCFA_BF16) {
    if (dtype_out == SCFA_F32) hipLaunchKernelGGL((k_fwd_bf16<HASH, ZD, float>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_fwd_bf16<HASH, ZD, uint16_t>), grid, block, 0, stream, p);
  } else {
    if (dtype_out == SCFA_F32) hipLaunchKernelGGL((k_fwd_f32<HASH, ZD, float>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_fwd_f32<HASH, ZD, uint16_t>), grid, block, 0, stream, p);
  }
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int check_common(int dtype_in, int dtype_out, int B, int H, int T, int T_kv, int D, float scale) {
  if (!dtype_ok(dtype_in) || !dtype_ok(dtype_out)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || T_kv < 1) return SCFA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return SCFA_ERR_INVALID;
  if (D != HD) return SCFA_ERR_UNSUPPORTED;
  // row offsets within one batch entry's (T, H, D) block are 32-bit
  if (static_cast<uint64_t>(max(T, T_kv)) * H * D * dtype_size(dtype_in) > 0xFFFFFFFFull) return SCFA_ERR_UNSUPPORTED;
  return SCFA_OK;
}

}  // namespace
}  // namespace scfa

using namespace scfa;

extern "C" {

int scfa_qk_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v,
                       const int32_t* q_idx, const int32_t* k_idx, const int32_t* qstats, const int32_t* kstats,
                       const int32_t* fwd_tab, const int32_t* order, int B, int H, int T, int T_kv, int Tc, int D,
                       float scale,
                       int flags, void* O, float* lse, hipStream_t stream) {
  if (!q || !k || !v || !q_idx || !k_idx || !qstats || !kstats || !fwd_tab || !O || !lse) return SCFA_ERR_INVALID;
  if (!flags_ok(flags)) return SCFA_ERR_INVALID;
  const int st = check_common(dtype_in, dtype_out, B, H, T, T_kv, D, scale);
  if (st != SCFA_OK) return st;
  if ((flags & SCFA_NONCAUSAL) && max(T, T_kv) > kPosLimit) return SCFA_ERR_UNSUPPORTED;
  if (Tc < SCFA_ROW_ALIGN || Tc % SCFA_ROW_ALIGN) return SCFA_ERR_INVALID;
  FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
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
  p.Tkv = T_kv;
  p.Tk = Tc;
  p.TqPad = Tc;
  p.TkPad = Tc;
  p.nQt = Tc / BM;
  p.nKt = Tc / BN;
  p.c = scale * 1.44269504088896340736f;
  p.rc = reach_of(flags);
  return dispatch_fwd<false, true>(dtype_in, dtype_out, p, stream);
}

int scfa_hash_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v,
                         const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt,
                         const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, const int32_t* order,
                         int B, int H, int T, int T_kv, int Tq, int Tk, int D, float scale, int flags, void* O,
                         float* lse,
                         hipStream_t stream) {
  if (!q || !k || !v || !q_idx || !k_idx || !q_bkt || !k_bkt || !qstats || !kstats || !fwd_tab || !O || !lse)
    return SCFA_ERR_INVALID;
  if (!flags_ok(flags)) return SCFA_ERR_INVALID;
  const int st = check_common(dtype_in, dtype_out, B, H, T, T_kv, D, scale);
  if (st != SCFA_OK) return st;
  if ((flags & SCFA_NONCAUSAL) && max(T, T_kv) > kPosLimit) return SCFA_ERR_UNSUPPORTED;
  if (Tq < 1 || Tk < 1) return SCFA_ERR_INVALID;
  FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
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
  p.Tkv = T_kv;
  p.Tk = Tk;
  p.TqPad = pad_rows(Tq);
  p.TkPad = pad_rows(Tk);
  p.nQt = p.TqPad / BM;
  p.nKt = p.TkPad / BN;
  p.c = scale * 1.44269504088896340736f;
  p.rc = reach_of(flags);
  return dispatch_fwd<true, false>(dtype_in, dtype_out, p, stream);
}

}  // extern "C"
