// Backward of sparse causal flash attention on gfx950 (CDNA4).
//
// What is computed (explainer "Faster Causal Attention Over Large Sequences
// Through Sparse Flash Attention", 3.4 "Backward Pass Design"): the score
// tiles are recomputed from the saved log-sum-exp with the same tile ranges
// and local masks as the forward, roles of queries and keys swapped for dK
// and dV (per key tile, the range of query tiles of the backward table) and
// as in the forward for dQ (per query tile, the forward table). With
// P = exp(s - LSE) on visible pairs:
//   dV = P^T dO,  dP = dO V^T,  Delta_i = dO_i . O_i,  dS = P (dP - Delta),
//   dQ = scale dS K,  dK = scale dS^T Q.
// A query whose LSE is -inf (no visible key) contributes nothing: its
// log2-LSE is stored as +inf, so exp2(s - lse) = 0 (the guard of the
// NaN-safe softmax carried to the backward).
//
// MI355X design:
//  * Two kernels, no atomics (deterministic): dQ per 128-query tile (4 waves
//    x 32 queries, key tiles of 64), which also computes Delta and log2 LSE
//    of its rows from O, dO and the LSE and leaves them in the workspace,
//    then dK/dV, which reads them. dK/dV runs per pair of 64-key
//    tiles (4 waves x 32 keys, query chunks of 32: 38 KB of LDS, 3 waves per
//    SIMD; each Q / dO operand read from LDS serves two 16-key blocks) for
//    the long ranges of QK and dense attention, and per 64-key tile (4 waves
//    x 16 keys, 4 waves per SIMD) for the short ranges of the hash layout.
//  * Operands are read from the original (B, T, H, D) tensors through the
//    index arrays (gather fused into the loads, as in the forward): each
//    lane's own rows straight into registers, the shared tiles by
//    global-to-LDS DMA, double buffered. A tile needed both as row operand
//    and transposed (Q and dO for dK/dV, K for dQ) is staged once, in the
//    layout of the row reads, which the transposed reads
//    (ds_read_b64_tr_b16) also read at full speed; no transposed copy exists
//    in memory.
//  * All six products are v_mfma_f32_16x16x32_bf16. The score-like tiles
//    (S, dP) are laid out so that each lane owns one column (a key in dK/dV,
//    a query in dQ) and 4 rows per 16x16 block; their A-operand rows are
//    permuted so a lane's 8 probabilities cover 8 consecutive rows, which
//    lets P and dS feed the next MFMA directly as B operands.
//  * Masks are accumulator biases (0 / -inf) built with VCC-only selects;
//    tiles proven fully visible by the extrema skip them, and each wave
//    skips chunks holding no pair visible to its rows. The dQ and hash dK/dV
//    kernels take these tests for 64 tiles of their range at once and keep
//    them as wave-uniform bit masks; the tile-pair dK/dV kernel stages the
//    statistics of its range in LDS once.
//  * Gradients are staged in LDS and written as whole rows at the original
//    token positions; QK-drop zeroes the rows of dropped tokens.

#include <math.h>

#include <mutex>

#include "scfa_stage.h"

namespace scfa {
namespace {

constexpr int BM = SCFA_TILE_M;  // 128: dQ workgroup rows, table granularity
constexpr int BN = SCFA_TILE_N;  // 64: dK/dV workgroup keys, table granularity
constexpr int QC = 32;          // query chunk of the dK/dV loop
constexpr int HD = 64;
constexpr int TB = 64 * HD * 2;  // bytes of one 64 x 64 bf16 tile
constexpr int kStatCap = 256;    // tile statistics of a range held in LDS (dK/dV of tile pairs)

struct BwdParams {
  const void* q;   // (B, T, H, D) bf16, original order, as are k, v, dO
  const void* k;
  const void* v;
  const void* dO;
  const float* O;      // (B, T, H, D) forward output, original order
  const float* lse;    // (B*H, T) forward natural-log LSE, original order
  float* lse2;         // (BH, TqP) sorted query rows: log2 LSE, +inf when no visible key / pad row (written by dQ)
  float* delta;        // (BH, TqP) Delta = dO . O per sorted query row (written by dQ)
  const int32_t* q_idx;
  const int32_t* k_idx;
  const int32_t* q_bkt;
  const int32_t* k_bkt;
  const int4* qstats;
  const int4* kstats;
  const int2* fwd_tab;
  const int2* bwd_tab;
  const int32_t* q_order;  // launch order of the dQ workgroups (over fwd_tab items), or null
  const int32_t* k_order;  // launch order of the dK/dV workgroups (over bwd_tab items), or null
  float* dQ;
  float* dK;
  float* dV;
  int B, H, T;
  int Tkv;       // tokens of the original k and v tensors (B, Tkv, H, D); T is that of q, dO
  int Tq, Tk;    // valid query / key rows (as passed to the range table)
  int TqP, TkP;  // rows per head of the query-side / key-side index arrays
  int nQt, nKt;
  float c;      // scale * log2(e)
  float scale;  // score scale
  Reach rc;     // position test (causal, strict or non-causal)
};

// Zero the gradient rows of the tokens a tile owns but does not hold
// (QK-drop: dropped tokens). Tile `tile` of `rows` rows of the index array
// owns the original positions after the previous tile's last real entry up
// to its own last real entry; the last tile holding real entries owns the
// rest of the sequence, and with no real entry at all tile 0 owns all of it.
// `ti` holds the tile's index entries in LDS; real entries are < T, >= 0 and
// form a sorted prefix of the array.
template <int ROWS>
__device__ void zero_unheld(const int32_t* idx_bh, const int32_t* ti, int tile, int Tpad, int T, int H, int b, int h,
                            float* out0, float* out1) {
  const int tid = threadIdx.x;
  const int nreal = __syncthreads_count(tid < ROWS && ti[tid] >= 0 && ti[tid] < T);
  int lo = 0, hi = -1;
  if (nreal > 0) {
    lo = tile == 0 ? 0 : max(0, idx_bh[tile * ROWS - 1] + 1);
    const int nx = (tile + 1) * ROWS < Tpad ? idx_bh[(tile + 1) * ROWS] : -1;
    const bool next_real = nx >= 0 && nx < T;
    hi = next_real ? min(ti[nreal - 1], T - 1) : T - 1;
  } else if (tile == 0) {
    lo = 0;
    hi = T - 1;
  }
  // 256 positions per pass, one per thread: the tile's real entries in the
  // pass's window are flagged in LDS, and each thread zeroes the whole rows of
  // its position when that is not flagged
  __shared__ uint8_t held_w[256];
  for (int base = lo; base <= hi; base += 256) {
    held_w[tid] = 0;
    __syncthreads();
    if (tid < nreal) {
      const int d = ti[tid] - base;
      if (d >= 0 && d < 256) held_w[d] = 1;
    }
    __syncthreads();
    const int pos = base + tid;
    if (pos <= hi && !held_w[tid]) {
      const size_t o = ((static_cast<size_t>(b) * T + pos) * H + h) * HD;
#pragma unroll
      for (int u = 0; u < HD / 4; ++u) {
        reinterpret_cast<f32x4*>(out0 + o)[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (out1) reinterpret_cast<f32x4*>(out1 + o)[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    __syncthreads();  // held_w is cleared for the next pass
  }
}

// Stage a 16 x 64 gradient block (lane: column key/query n = l % 16, dims
// 16db + 4g + e) into an LDS tile of fp32 rows (64 floats, 16-byte units
// XOR-swizzled by row).
__device__ inline void stage_rows(float* tile, int row, int g, const f32x4 (&acc)[4], float mul) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
    *reinterpret_cast<f32x4*>(tile + row * HD + (((4 * db + g) ^ (row & 15)) * 4)) = acc[db] * mul;
}

// Write `nrows` staged rows to their original positions (16 threads / row).
__device__ inline void write_rows(const float* tile, const int32_t* pos, int nrows, float* out, int T, int H, int b,
                                  int h) {
  for (int row = threadIdx.x >> 4; row < nrows; row += 16) {
    const int u = threadIdx.x & 15;
    const int p = pos[row];
    if (p >= 0 && p < T)
      *reinterpret_cast<f32x4*>(out + ((static_cast<size_t>(b) * T + p) * H + h) * HD + u * 4) =
          *reinterpret_cast<const f32x4*>(tile + row * HD + ((u ^ (row & 15)) * 4));
  }
}

__device__ inline void map_work(int x, int BH, int ntiles, int& tile, int& bh, bool reverse) {
  int t;
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3, xcd = x & 7, slot = x >> 3;
    t = slot / hpx;
    bh = xcd * hpx + slot % hpx;
  } else {
    t = x / BH;
    bh = x % BH;
  }
  tile = reverse ? ntiles - 1 - t : t;
}

// Work item of workgroup x: from a launch order (item = bh * ntiles + tile,
// longest range first) when one is given, else the default mapping.
__device__ inline void pick_item(const int32_t* order, int x, int BH, int ntiles, int& tile, int& bh, bool reverse) {
  if (order) {
    const int it = order[x];
    bh = it / ntiles;
    tile = it - bh * ntiles;
  } else {
    map_work(x, BH, ntiles, tile, bh, reverse);
  }
}

__device__ __forceinline__ int4 uniform4(const int4& v) {
  return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                   __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
}

// Extrema of this wave's 16 keys (lane column r16; the 4 lane groups hold the
// same keys), over the real ones (0 <= position < T); `all` = no pad key.
struct WaveKeys {
  int minpos, maxpos, minb, maxb;
  bool any, all;
};

// The extrema are of k_reach(position), the smallest query position that
// sees the key.
__device__ inline WaveKeys wave_keys(int kpos, int kbkt, int T, const Reach& rc) {
  const bool real = kpos >= 0 && kpos < T;
  int mn = real ? k_reach(rc, kpos) : kInt32Max, mx = real ? k_reach(rc, kpos) : kInt32Min;
  int mnb = real ? kbkt : kInt32Max, mxb = real ? kbkt : kInt32Min;
  int nreal = real ? 1 : 0;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
    mnb = min(mnb, __shfl_xor(mnb, o));
    mxb = max(mxb, __shfl_xor(mxb, o));
    nreal += __shfl_xor(nreal, o);
  }
  WaveKeys k;
  k.minpos = __builtin_amdgcn_readfirstlane(mn);
  k.maxpos = __builtin_amdgcn_readfirstlane(mx);
  k.minb = __builtin_amdgcn_readfirstlane(mnb);
  k.maxb = __builtin_amdgcn_readfirstlane(mxb);
  nreal = __builtin_amdgcn_readfirstlane(nreal);
  k.any = nreal > 0;
  k.all = nreal == 16;
  return k;
}

// ---------------------------------------------------------------------------
// dK, dV for short query ranges (the hash layout's): one workgroup per 64-key
// tile; wave w owns keys 16w .. 16w+15 (its K and V rows in registers, one
// key per lane column). Query chunks of 32 rows are staged by DMA: Q and dO
// once each, read as rows (A operands of S = Q K^T and dP = dO V^T) and
// transposed (A operands of dK^T += Q^T dS and dV^T += dO^T P), with their
// positions, buckets, log2 LSE and Delta.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZD>
__global__ __launch_bounds__(256) void k_bwd_dkdv64(BwdParams p) {
  constexpr int CQ = 2 * QC;     // query rows of a staged chunk, processed in two halves of QC
  constexpr int CB = CQ * 128;   // bytes of one staged chunk copy
  __shared__ __align__(16) uint8_t smem[2 * BN * HD * 4];  // 2 stages x (Q, dO) chunks; epilogue staging (32 KB)
  static_assert(2 * 2 * CB <= 2 * BN * HD * 4, "chunk staging does not fit");
  __shared__ __align__(16) int32_t qpos_s[2][CQ];
  __shared__ __align__(16) int32_t qbkt_s[2][CQ];
  __shared__ __align__(16) float lse_s[2][CQ];
  __shared__ __align__(16) float del_s[2][CQ];
  __shared__ int32_t Ki[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int BH = p.B * p.H;
  int kt, bh;
  pick_item(p.k_order, blockIdx.x, BH, p.nKt, kt, bh, false);  // longest ranges first
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqP;  // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkP;    // key side
  const int2 rng = p.bwd_tab[static_cast<size_t>(bh) * p.nKt + kt];
  // tests of the range's query tiles, 64 tiles per window
  TileWalk<true> walk(p.qstats + static_cast<size_t>(bh) * p.nQt, rng.x, rng.y, lane);
  const int ki_v = tid < BN ? p.k_idx[kbase + kt * BN + tid] : 0;  // the tile's key entries

  const uint32_t rstride = static_cast<uint32_t>(p.H) * HD * 2;  // bytes between token rows
  const size_t head0 = (static_cast<size_t>(b) * p.T * p.H + h) * HD * 2;     // token 0 of this head in q, dO
  const size_t khead0 = (static_cast<size_t>(b) * p.Tkv * p.H + h) * HD * 2;  // and in k, v
  const int krow = kt * BN + w * 16 + r16;  // this lane's key
  const int kpos = p.k_idx[kbase + krow];
  const int kbkt = HASH ? p.k_bkt[kbase + krow] : 0;
  // the smallest query position that sees this key (kpos + 1 when strict):
  // masks and tile tests compare queries against it
  const int kcmp = k_reach(p.rc, kpos);
  const WaveKeys wk = wave_keys(kpos, kbkt, p.Tkv, p.rc);
  bf16x8 Kb[2], Vb[2];
  {
    const size_t off = khead0 + static_cast<size_t>(src_row(kpos, p.Tkv)) * rstride;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      Kb[ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.k) + off + (ds * 32 + g * 8) * 2);
      Vb[ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.v) + off + (ds * 32 + g * 8) * 2);
    }
  }
  f32x4 dVa[4], dKa[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dVa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- DMA staging of a query chunk: wave w stages rows 16w .. 16w+15 ------
  const uint8_t* qg = static_cast<const uint8_t*>(p.q) + head0;
  const uint8_t* dg = static_cast<const uint8_t*>(p.dO) + head0;
  uint32_t rch[2];  // swz_k layout: serves the row and the transposed reads
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * w + 8 * i + (lane >> 3), cp = lane & 7;
    rch[i] = (cp ^ swz_k(row)) * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t lds_small = ws == 0 ? lds_addr(&qpos_s[0][0])
                             : ws == 1 ? lds_addr(&qbkt_s[0][0])
                             : ws == 2 ? lds_addr(&lse_s[0][0])
                                       : lds_addr(&del_s[0][0]);
  const void* small_src = ws == 0 ? static_cast<const void*>(p.q_idx + rowbase)
                          : ws == 1 ? static_cast<const void*>(HASH ? p.q_bkt + rowbase : p.q_idx + rowbase)
                          : ws == 2 ? static_cast<const void*>(p.lse2 + rowbase)
                                    : static_cast<const void*>(p.delta + rowbase);
  constexpr int CPT = BM / CQ;  // chunks per query tile
  const int nch = CPT * p.nQt;
  auto chunk_rows = [&](int ci, int (&pos)[2]) {  // the two rows this lane stages
#pragma unroll
    for (int i = 0; i < 2; ++i) pos[i] = p.q_idx[rowbase + min(ci, nch - 1) * CQ + 16 * w + 8 * i + (lane >> 3)];
  };
  auto stage = [&](int ci, int s, const int (&pos)[2]) {
    const uint32_t base = lds0 + s * 2 * CB + ws * 2048;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = static_cast<uint32_t>(src_row(pos[i], p.T)) * rstride;
      dma16(qg, off + rch[i], base + i * 1024);
      dma16(dg, off + rch[i], base + CB + i * 1024);
    }
    static_assert(CQ == 64, "one 4-byte entry per lane");
    dma4(static_cast<const uint8_t*>(small_src) + ci * CQ * 4, lane * 4, lds_small + s * CQ * 4);
  };
  // chunk ci = CPT * query tile + part; tiles failing the causal test are
  // skipped
  const int4 ks = p.kstats[static_cast<size_t>(bh) * p.nKt + kt];
  const int kreach = k_reach(p.rc, ks.x);  // smallest query position that sees a key of the tile
  const int cend = CPT * rng.y;
  // query tile ii (statistics qs) against this wave's keys
  auto tests = [&](const int4& qs, int ii) {
    const bool valid = ii < rng.y;
    bool full = wk.all && wk.maxpos <= qs.x && (ii + 1) * BM <= p.Tq;
    if (HASH) full = full && qs.z == qs.w && wk.minb == wk.maxb && wk.minb == qs.z;
    TileMasks m;
    m.pass = __ballot(valid && qs.y >= kreach);
    m.empty = __ballot(valid && (!wk.any || wk.minpos > qs.y || (HASH && (wk.minb > qs.w || wk.maxb < qs.z))));
    m.full = __ballot(valid && full);
    m.mixed = HASH ? static_cast<uint64_t>(__ballot(valid && !(qs.z == qs.w && wk.minb == wk.maxb))) : 0ull;
    return m;
  };
  walk.first(tests);
  // first chunk at or after c whose query tile passes the causal test
  auto next_chunk = [&](int c) {
    if (c >= cend) return cend;
    const int t = c / CPT, t2 = walk.next(t, tests);
    return t2 == t ? c : (t2 < rng.y ? CPT * t2 : cend);
  };

  // The first chunk of the range is staged at once (a chunk failing the
  // causal extremum test is skipped by every wave's own test).
  int ci = CPT * rng.x < cend ? CPT * rng.x : cend;
  int pos[2];
  if (ci < cend) {
    chunk_rows(ci, pos);
    stage(ci, 0, pos);
  }
  if (tid < BN) Ki[tid] = ki_v;  // published by the barriers below
  int cn = ci < cend ? next_chunk(ci + 1) : cend;
  chunk_rows(cn, pos);
  dma_wait();
  __syncthreads();
  int s = 0;
  while (ci < cend) {
    walk.enter(ci / CPT, tests);
    const int cnn = cn < cend ? next_chunk(cn + 1) : cend;
    int pos_nn[2];
    chunk_rows(cnn, pos_nn);  // issued before the DMA: waiting for it never waits for the DMA
    __builtin_amdgcn_sched_barrier(0);
    if (cn < cend) stage(cn, s ^ 1, pos);

    // this wave's keys against the chunk's query tile: skip / no mask
    const int qt = ci / CPT;
    if (!walk.has(walk.cw.empty, qt)) {
      const uint8_t* Qr = smem + s * 2 * CB;
      const uint8_t* Dr = Qr + CB;
      const bool full = walk.has(walk.cw.full, qt);
      const bool buckets = HASH && walk.has(walk.cw.mixed, qt);
      // the chunk's two halves of QC queries (rows 32 hq .. 32 hq + 31)
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        // S = Q K^T (from the mask bias) and dP = dO V^T: rows = queries,
        // column = this lane's key; element e of block qb is query
        // 32 hq + 8 g + 4 qb + e of the chunk. Both branches define S afresh
        // (a fully visible chunk starts the accumulators at zero).
        f32x4 S[2], dP[2];
        // log2 LSE and Delta of the half's queries, read before the products
        // so that the exponentials do not wait for LDS
        f32x4 l4[2], d4[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qo = 32 * hq + 8 * g + 4 * qb;
          l4[qb] = *reinterpret_cast<const f32x4*>(&lse_s[s][qo]);
          d4[qb] = *reinterpret_cast<const f32x4*>(&del_s[s][qo]);
        }
        auto scores = [&]() {
#pragma unroll
          for (int ds = 0; ds < 2; ++ds)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              S[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_row_op(Qr, 2 * hq + qb, r16, ds * 4 + g), Kb[ds],
                                                              S[qb], 0, 0, 0);
        };
        if (full) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) S[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          scores();
        } else {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int qo = 32 * hq + 8 * g + 4 * qb;
            const int4 qp4 = *reinterpret_cast<const int4*>(&qpos_s[s][qo]);
            f32x4 c;
            c[0] = bias_if_ge(qp4.x, kcmp);
            c[1] = bias_if_ge(qp4.y, kcmp);
            c[2] = bias_if_ge(qp4.z, kcmp);
            c[3] = bias_if_ge(qp4.w, kcmp);
            if (buckets) {
              const int4 qb4 = *reinterpret_cast<const int4*>(&qbkt_s[s][qo]);
              c[0] = keep_if_eq(c[0], qb4.x, kbkt);
              c[1] = keep_if_eq(c[1], qb4.y, kbkt);
              c[2] = keep_if_eq(c[2], qb4.z, kbkt);
              c[3] = keep_if_eq(c[3], qb4.w, kbkt);
            }
            S[qb] = c;
          }
          scores();
        }
        // dP - Delta straight from the MFMAs: the accumulators start at -Delta
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dP[qb] = -d4[qb];
#pragma unroll
        for (int ds = 0; ds < 2; ++ds)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            dP[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_row_op(Dr, 2 * hq + qb, r16, ds * 4 + g), Vb[ds],
                                                             dP[qb], 0, 0, 0);
        // P = exp2(S c - lse2), dS = P (dP - Delta)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(S[qb][e], p.c, -l4[qb][e]));
            S[qb][e] = pe;
            dP[qb][e] = pe * dP[qb][e];
          }
        }
        const bf16x8 Pp = pack_bf16x8(S[0], S[1]);
        const bf16x8 Sp = pack_bf16x8(dP[0], dP[1]);
        // dV^T += dO^T P,  dK^T += Q^T dS  (rows = dims, column = this lane's key)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dVa[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_tr_op(Dr, db, hq, g, r16), Pp, dVa[db], 0, 0, 0);
          dKa[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_tr_op(Qr, db, hq, g, r16), Sp, dKa[db], 0, 0, 0);
        }
      }
    }

    dma_wait();
    __syncthreads();
    s ^= 1;
    ci = cn;
    cn = cnn;
    pos[0] = pos_nn[0];
    pos[1] = pos_nn[1];
  }

  // ---- epilogue: stage dK (scaled) and dV in LDS, write whole rows ---------
  float* tk = reinterpret_cast<float*>(smem);
  float* tv = tk + BN * HD;
  const int row = w * 16 + r16;
  stage_rows(tk, row, g, dKa, p.scale);
  stage_rows(tv, row, g, dVa, 1.f);
  __syncthreads();
  write_rows(tk, Ki, BN, p.dK, p.Tkv, p.H, b, h);
  write_rows(tv, Ki, BN, p.dV, p.Tkv, p.H, b, h);
  if constexpr (ZD) zero_unheld<BN>(p.k_idx + kbase, Ki, kt, p.TkP, p.Tkv, p.H, b, h, p.dK, p.dV);
}

// Extrema of this wave's 32 keys (two blocks of 16; lane column r16 in each).
__device__ inline WaveKeys wave_keys2(const int (&kpos)[2], const int (&kbkt)[2], int T, const Reach& rc) {
  int mn = kInt32Max, mx = kInt32Min, mnb = kInt32Max, mxb = kInt32Min, nreal = 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bool real = kpos[kb] >= 0 && kpos[kb] < T;
    if (real) {
      mn = min(mn, k_reach(rc, kpos[kb]));
      mx = max(mx, k_reach(rc, kpos[kb]));
      mnb = min(mnb, kbkt[kb]);
      mxb = max(mxb, kbkt[kb]);
      ++nreal;
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
    mnb = min(mnb, __shfl_xor(mnb, o));
    mxb = max(mxb, __shfl_xor(mxb, o));
    nreal += __shfl_xor(nreal, o);
  }
  WaveKeys k;
  k.minpos = __builtin_amdgcn_readfirstlane(mn);
  k.maxpos = __builtin_amdgcn_readfirstlane(mx);
  k.minb = __builtin_amdgcn_readfirstlane(mnb);
  k.maxb = __builtin_amdgcn_readfirstlane(mxb);
  nreal = __builtin_amdgcn_readfirstlane(nreal);
  k.any = nreal > 0;
  k.all = nreal == 32;
  return k;
}

// ---------------------------------------------------------------------------
// dK, dV for long query ranges (QK and dense): one workgroup per pair of
// 64-key tiles (2 kt, 2 kt + 1); wave w
// owns keys 32w .. 32w+31 of the pair (waves 0-1 the first tile, 2-3 the
// second), over the union of the two tiles' query ranges from the backward
// table in chunks of 32 queries. The chunk's Q and dO operands read from LDS
// serve both 16-key blocks of a wave. Each query chunk's 32 rows are staged
// by DMA: Q and dO once each, read as rows (A operands of S = Q K^T and
// dP = dO V^T) and transposed (A operands of dK^T += Q^T dS and
// dV^T += dO^T P), with their positions, buckets, log2 LSE and Delta.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_dkdv(BwdParams p) {
  constexpr int CB = QC * 128;  // bytes of one staged chunk copy (QC rows)
  constexpr int KR = 2 * BN;    // keys of a workgroup
  __shared__ __align__(16) uint8_t smem[2 * BN * HD * 4];  // 2 stages x (Q, dO) chunks; epilogue staging (32 KB)
  __shared__ __align__(16) int32_t qpos_s[2][QC];
  __shared__ __align__(16) int32_t qbkt_s[2][QC];
  __shared__ __align__(16) float lse_s[2][QC];
  __shared__ __align__(16) float del_s[2][QC];
  __shared__ __align__(16) int4 Qst[kStatCap];
  __shared__ int32_t Ki[KR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int BH = p.B * p.H;
  const int nKp = (p.nKt + 1) / 2;
  int kp, bh;
  map_work(blockIdx.x, BH, nKp, kp, bh, false);  // early key tiles see the most queries
  const int kt0 = 2 * kp;
  const bool has1 = kt0 + 1 < p.nKt;
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqP;  // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkP;    // key side
  const int2 rng0 = p.bwd_tab[static_cast<size_t>(bh) * p.nKt + kt0];
  const int2 rng1 = has1 ? p.bwd_tab[static_cast<size_t>(bh) * p.nKt + kt0 + 1] : make_int2(0, 0);
  const int4 ks0 = p.kstats[static_cast<size_t>(bh) * p.nKt + kt0];
  const int4 ks1 = has1 ? p.kstats[static_cast<size_t>(bh) * p.nKt + kt0 + 1] : make_int4(0, 0, 0, 0);
  // smallest query position that sees a key of each tile
  const int kreach0 = k_reach(p.rc, ks0.x), kreach1 = k_reach(p.rc, ks1.x);
  const bool e0 = rng0.y <= rng0.x, e1 = rng1.y <= rng1.x;
  const int lo = e0 ? rng1.x : (e1 ? rng0.x : min(rng0.x, rng1.x));
  const int hi = e0 ? (e1 ? lo : rng1.y) : (e1 ? rng0.y : max(rng0.y, rng1.y));
  const int4* qst = p.qstats + static_cast<size_t>(bh) * p.nQt;
  const bool qst_lds = hi - lo <= kStatCap;
  if (qst_lds)
    for (int i = tid; i < hi - lo; i += 256) Qst[i] = qst[lo + i];
  if (tid < KR) Ki[tid] = (tid < BN || has1) ? p.k_idx[kbase + kt0 * BN + tid] : SCFA_K_PAD;
  __syncthreads();
  auto qstat = [&](int i) { return uniform4(stat_entry(qst_lds, Qst, i - lo, qst, i)); };

  const uint32_t rstride = static_cast<uint32_t>(p.H) * HD * 2;  // bytes between token rows
  const size_t head0 = (static_cast<size_t>(b) * p.T * p.H + h) * HD * 2;     // token 0 of this head in q, dO
  const size_t khead0 = (static_cast<size_t>(b) * p.Tkv * p.H + h) * HD * 2;  // and in k, v
  int kpos[2], kbkt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = w * 32 + kb * 16 + r16;  // this lane's key of block kb
    kpos[kb] = Ki[r];
    kbkt[kb] = HASH ? ((r < BN || has1) ? p.k_bkt[kbase + kt0 * BN + r] : 0) : 0;
  }
  const WaveKeys wk = wave_keys2(kpos, kbkt, p.Tkv, p.rc);
  // the smallest query position that sees each key (kpos + 1 when strict)
  const int kcmp[2] = {k_reach(p.rc, kpos[0]), k_reach(p.rc, kpos[1])};
  bf16x8 Kb[2][2], Vb[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const size_t off = khead0 + static_cast<size_t>(src_row(kpos[kb], p.Tkv)) * rstride;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      Kb[kb][ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.k) + off + (ds * 32 + g * 8) * 2);
      Vb[kb][ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.v) + off + (ds * 32 + g * 8) * 2);
    }
  }
  f32x4 dVa[2][4], dKa[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dVa[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dKa[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // ---- DMA staging of a query chunk: wave w stages rows 8w .. 8w+7 --------
  const uint8_t* qg = static_cast<const uint8_t*>(p.q) + head0;
  const uint8_t* dg = static_cast<const uint8_t*>(p.dO) + head0;
  uint32_t rch;  // swz_k layout: serves the row and the transposed reads
  {
    const int row = 8 * w + (lane >> 3), cp = lane & 7;
    rch = (cp ^ swz_k(row)) * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t lds_small = ws == 0 ? lds_addr(&qpos_s[0][0])
                             : ws == 1 ? lds_addr(&qbkt_s[0][0])
                             : ws == 2 ? lds_addr(&lse_s[0][0])
                                       : lds_addr(&del_s[0][0]);
  const void* small_src = ws == 0 ? static_cast<const void*>(p.q_idx + rowbase)
                          : ws == 1 ? static_cast<const void*>(HASH ? p.q_bkt + rowbase : p.q_idx + rowbase)
                          : ws == 2 ? static_cast<const void*>(p.lse2 + rowbase)
                                    : static_cast<const void*>(p.delta + rowbase);
  constexpr int CPT = BM / QC;  // chunks per query tile
  const int nch = CPT * p.nQt;
  auto chunk_rows = [&](int ci, int (&pos)[2]) {  // pos[0]: the row this lane stages
    pos[0] = p.q_idx[rowbase + min(ci, nch - 1) * QC + 8 * w + (lane >> 3)];
    pos[1] = 0;
  };
  auto stage = [&](int ci, int s, const int (&pos)[2]) {
    const uint32_t base = lds0 + s * 2 * CB + ws * 1024;
    const uint32_t off = static_cast<uint32_t>(src_row(pos[0], p.T)) * rstride;
    dma16(qg, off + rch, base);
    dma16(dg, off + rch, base + CB);
    if (lane < QC) dma4(static_cast<const uint8_t*>(small_src) + ci * QC * 4, lane * 4, lds_small + s * QC * 4);
  };
  // chunk ci = CPT * query tile + part: query tiles in either tile's range
  // that pass that tile's causal test
  const int cend = CPT * hi;
  auto needed = [&](int t) {
    const int qy = qstat(t).y;
    return (t >= rng0.x && t < rng0.y && qy >= kreach0) || (t >= rng1.x && t < rng1.y && qy >= kreach1);
  };
  auto next_chunk = [&](int ci) {
    while (ci < cend && !needed(ci / CPT)) ci = (ci / CPT + 1) * CPT;
    return ci;
  };

  int ci = next_chunk(CPT * lo);
  int cn = ci < cend ? next_chunk(ci + 1) : cend;
  int pos[2];
  if (ci < cend) {
    chunk_rows(ci, pos);
    stage(ci, 0, pos);
  }
  chunk_rows(cn, pos);
  dma_wait();
  __syncthreads();
  int s = 0;
  int4 qs_cur = ci < cend ? qstat(ci / CPT) : make_int4(0, 0, 0, 0);
  while (ci < cend) {
    const int cnn = cn < cend ? next_chunk(cn + 1) : cend;
    const int4 qs = qs_cur;
    if (cn < cend) qs_cur = qstat(cn / CPT);
    int pos_nn[2];
    chunk_rows(cnn, pos_nn);  // issued before the DMA: waiting for it never waits for the DMA
    __builtin_amdgcn_sched_barrier(0);
    if (cn < cend) stage(cn, s ^ 1, pos);

    // this wave's keys against the chunk's query tile: skip / no mask
    const bool empty = !wk.any || wk.minpos > qs.y || (HASH && (wk.minb > qs.w || wk.maxb < qs.z));
    if (!empty) {
      const uint8_t* Qr = smem + s * 2 * CB;
      const uint8_t* Qt = Qr;
      const uint8_t* Dr = Qr + CB;
      const uint8_t* Dt = Dr;
      bool full = wk.all && wk.maxpos <= qs.x && (ci / CPT + 1) * BM <= p.Tq;
      if (HASH) full = full && qs.z == qs.w && wk.minb == wk.maxb && wk.minb == qs.z;
      // S = Q K^T (from the mask bias) and dP = dO V^T: rows = queries,
      // column = this lane's key of block kb; element e of block qb is
      // query 8 g + 4 qb + e of the chunk
      f32x4 S[2][2], dP[2][2];
      if (full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) S[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const bool buckets = HASH && !(qs.z == qs.w && wk.minb == wk.maxb);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qo = 8 * g + 4 * qb;
          const int4 qp4 = *reinterpret_cast<const int4*>(&qpos_s[s][qo]);
          const int4 qb4 = *reinterpret_cast<const int4*>(&qbkt_s[s][qo]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            f32x4 c;
            c[0] = bias_if_ge(qp4.x, kcmp[kb]);
            c[1] = bias_if_ge(qp4.y, kcmp[kb]);
            c[2] = bias_if_ge(qp4.z, kcmp[kb]);
            c[3] = bias_if_ge(qp4.w, kcmp[kb]);
            if (buckets) {
              c[0] = keep_if_eq(c[0], qb4.x, kbkt[kb]);
              c[1] = keep_if_eq(c[1], qb4.y, kbkt[kb]);
              c[2] = keep_if_eq(c[2], qb4.z, kbkt[kb]);
              c[3] = keep_if_eq(c[3], qb4.w, kbkt[kb]);
            }
            S[kb][qb] = c;
          }
        }
      }
      // dP - Delta straight from the MFMAs: the accumulators start at -Delta
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&del_s[s][8 * g + 4 * qb]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dP[kb][qb] = -d4;
      }
#pragma unroll
      for (int ds = 0; ds < 2; ++ds)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 qa = read_row_op(Qr, qb, r16, ds * 4 + g);
          const bf16x8 da = read_row_op(Dr, qb, r16, ds * 4 + g);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, Kb[kb][ds], S[kb][qb], 0, 0, 0);
            dP[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, Vb[kb][ds], dP[kb][qb], 0, 0, 0);
          }
        }
      // P = exp2(S c - lse2), dS = P (dP - Delta)
      bf16x8 Pp[2], Sp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qo = 8 * g + 4 * qb;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[s][qo]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(S[kb][qb][e], p.c, -l4[e]));
            S[kb][qb][e] = pe;
            dP[kb][qb][e] = pe * dP[kb][qb][e];
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Pp[kb] = pack_bf16x8(S[kb][0], S[kb][1]);
        Sp[kb] = pack_bf16x8(dP[kb][0], dP[kb][1]);
      }
      // dV^T += dO^T P,  dK^T += Q^T dS  (rows = dims, column = this lane's key)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 dt = read_tr_op(Dt, db, 0, g, r16);
        const bf16x8 qt = read_tr_op(Qt, db, 0, g, r16);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dVa[kb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dt, Pp[kb], dVa[kb][db], 0, 0, 0);
          dKa[kb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt, Sp[kb], dKa[kb][db], 0, 0, 0);
        }
      }
    }

    dma_wait();
    __syncthreads();
    s ^= 1;
    ci = cn;
    cn = cnn;
    pos[0] = pos_nn[0];
    pos[1] = pos_nn[1];
  }

  // ---- epilogue: stage dK (scaled), then dV, in LDS; write whole rows ------
  float* tg = reinterpret_cast<float*>(smem);  // 128 rows x 64 fp32 = 32 KB
  const int nrows = has1 ? KR : BN;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) stage_rows(tg, w * 32 + kb * 16 + r16, g, dKa[kb], p.scale);
  __syncthreads();
  write_rows(tg, Ki, nrows, p.dK, p.Tkv, p.H, b, h);
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) stage_rows(tg, w * 32 + kb * 16 + r16, g, dVa[kb], 1.f);
  __syncthreads();
  write_rows(tg, Ki, nrows, p.dV, p.Tkv, p.H, b, h);
  if constexpr (ZD) {
    zero_unheld<BN>(p.k_idx + kbase, Ki, kt0, p.TkP, p.Tkv, p.H, b, h, p.dK, p.dV);
    if (has1) zero_unheld<BN>(p.k_idx + kbase, Ki + BN, kt0 + 1, p.TkP, p.Tkv, p.H, b, h, p.dK, p.dV);
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128-query tile, over the forward table's key tiles;
// wave w owns queries 32w .. 32w+31 (Q and dO rows in registers). Key tiles
// are staged by DMA: K once, read as rows (A operand of S^T = K Q^T) and
// transposed (A operand of dQ^T += K^T dS^T), and V (A operand of
// dP^T = V dO^T), with the keys' positions / buckets.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_dq(BwdParams p) {
  __shared__ __align__(16) uint8_t smem[2 * 2 * TB];  // 2 stages x (K, V); epilogue staging
  __shared__ __align__(16) int32_t Kp[2][BN];
  __shared__ __align__(16) int32_t Kb[2][BN];
  static_assert(2 * 2 * TB >= BM * HD * 4, "dQ staging does not fit");

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int BH = p.B * p.H;
  int qt, bh;
  pick_item(p.q_order, blockIdx.x, BH, p.nQt, qt, bh, true);
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqP;  // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkP;    // key side
  const int2 rng = p.fwd_tab[static_cast<size_t>(bh) * p.nQt + qt];
  const int4 qs = p.qstats[static_cast<size_t>(bh) * p.nQt + qt];
  const int qreach = q_reach(p.rc, qs.y);  // largest key position a query of the tile may see
  // tile tests of the range, 64 key tiles per window
  TileWalk<HASH> walk(p.kstats + static_cast<size_t>(bh) * p.nKt, rng.x, rng.y, lane);

  const uint32_t rstride = static_cast<uint32_t>(p.H) * HD * 2;
  const size_t head0 = (static_cast<size_t>(b) * p.T * p.H + h) * HD * 2;     // token 0 of this head in q, dO
  const size_t khead0 = (static_cast<size_t>(b) * p.Tkv * p.H + h) * HD * 2;  // and in k, v
  const int q0 = qt * BM + w * 32;
  int qpos[2], qbkt[2];
  float ql2[2], qdl[2];
  bf16x8 Qb[2][2], Db[2][2];
  // O and the LSE of the same rows, for Delta: loaded with Q and dO (all
  // loads of the rows in flight together, before any store)
  f32x4 Ov[2][2][2];  // [qb][ds][half]
  float lraw[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 16 + r16;
    qpos[qb] = p.q_idx[rowbase + row];
    qbkt[qb] = HASH ? p.q_bkt[rowbase + row] : 0;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qp = qpos[qb];
    const size_t off = head0 + static_cast<size_t>(src_row(qp, p.T)) * rstride;
    const float* orow = p.O + ((static_cast<size_t>(b) * p.T + src_row(qp, p.T)) * p.H + h) * HD;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      Qb[qb][ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.q) + off + (ds * 32 + g * 8) * 2);
      Db[qb][ds] = *reinterpret_cast<const bf16x8*>(static_cast<const uint8_t*>(p.dO) + off + (ds * 32 + g * 8) * 2);
      Ov[qb][ds][0] = *reinterpret_cast<const f32x4*>(orow + ds * 32 + g * 8);
      Ov[qb][ds][1] = *reinterpret_cast<const f32x4*>(orow + ds * 32 + g * 8 + 4);
    }
    lraw[qb] = p.lse[static_cast<size_t>(bh) * p.T + src_row(qp, p.T)];
  }
  // Delta = dO . O and log2 LSE of this wave's rows (the four lane groups
  // hold 16 dims each of a row), written to the workspace for dK/dV, which
  // runs after this kernel. Rows without a visible key (LSE = -inf) and pad
  // rows get log2 LSE = +inf, so exp2(s - lse2) = 0 there.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qp = qpos[qb];
    const bool valid = qp >= 0 && qp < p.T;
    float dot = 0.f;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf(static_cast<float>(Db[qb][ds][e]), Ov[qb][ds][0][e], dot);
        dot = fmaf(static_cast<float>(Db[qb][ds][4 + e]), Ov[qb][ds][1][e], dot);
      }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float l = valid ? lraw[qb] : -INFINITY;
    qdl[qb] = valid ? dot : 0.f;
    ql2[qb] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  if (g == 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const size_t r = rowbase + q0 + qb * 16 + r16;
      p.lse2[r] = ql2[qb];
      p.delta[r] = qdl[qb];
    }
  }
  const WaveRows wr = wave_rows(qpos, qbkt, p.rc);
  // positions the masks compare keys against: the largest visible key position
  const int qcmp[2] = {q_reach(p.rc, qpos[0]), q_reach(p.rc, qpos[1])};
  f32x4 dQa[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dQa[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- DMA staging of a key tile: wave w stages rows 16w .. 16w+15 --------
  const uint8_t* kg = static_cast<const uint8_t*>(p.k) + khead0;
  const uint8_t* vg = static_cast<const uint8_t*>(p.v) + khead0;
  const int32_t* kig = p.k_idx + kbase;
  const int32_t* kbg = HASH ? p.k_bkt + kbase : nullptr;
  uint32_t rch[2];  // swz_k layout: serves the row and the transposed reads
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * w + 8 * i + (lane >> 3), cp = lane & 7;
    rch[i] = (cp ^ swz_k(row)) * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t ldsp = lds_addr(&Kp[0][0]), ldsb = lds_addr(&Kb[0][0]);
  auto tile_rows = [&](int j, int (&pos)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) pos[i] = kig[min(j, p.nKt - 1) * BN + 16 * w + 8 * i + (lane >> 3)];
  };
  auto stage = [&](int j, int s, const int (&pos)[2]) {
    const uint32_t base = lds0 + s * 2 * TB + ws * 2048;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = static_cast<uint32_t>(src_row(pos[i], p.Tkv)) * rstride;
      dma16(kg, off + rch[i], base + i * 1024);
      dma16(vg, off + rch[i], base + TB + i * 1024);
    }
    if (ws == 0) dma4(kig + j * BN, lane * 4, ldsp + s * BN * 4);
    else if (HASH && ws == 1) dma4(kbg + j * BN, lane * 4, ldsb + s * BN * 4);
  };
  auto tests = [&](const int4& st, int jj) { return key_tile_masks<HASH>(st, jj, rng.y, qreach, wr, p.Tk); };
  walk.first(tests);

  // The first tile of the range is staged at once (a tile failing the causal
  // extremum test is skipped by every wave's own test).
  int j = rng.x < rng.y ? rng.x : rng.y;
  int pos[2];
  if (j < rng.y) {
    tile_rows(j, pos);
    stage(j, 0, pos);
  }
  int jn = j < rng.y ? walk.next(j + 1, tests) : rng.y;
  tile_rows(jn, pos);
  dma_wait();
  __syncthreads();
  int s = 0;
  while (j < rng.y) {
    walk.enter(j, tests);
    const int jnn = jn < rng.y ? walk.next(jn + 1, tests) : rng.y;
    int pos_nn[2];
    tile_rows(jnn, pos_nn);
    __builtin_amdgcn_sched_barrier(0);
    if (jn < rng.y) stage(jn, s ^ 1, pos);

    if (!walk.has(walk.cw.empty, j)) {
      const uint8_t* Kr = smem + s * 2 * TB;
      const uint8_t* Kt = Kr;
      const uint8_t* Vr = Kr + TB;
      const bool full = walk.has(walk.cw.full, j);
      const bool buckets = HASH && walk.has(walk.cw.mixed, j);
      // Two halves of 32 keys (blocks 2 kc, 2 kc + 1), so that only half of
      // the score tiles is live at a time. S^T = K Q^T (from the mask bias)
      // and dP^T = V dO^T: rows = keys, column = this lane's query.
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        // both branches define S afresh: a fully visible tile starts the
        // score accumulators at zero, others at the mask bias
        f32x4 S[2][2], dP[2][2];
        auto products = [&]() {
          // dP^T - Delta straight from the MFMAs: the accumulators start at -Delta
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) dP[h2][qb] = f32x4{-qdl[qb], -qdl[qb], -qdl[qb], -qdl[qb]};
#pragma unroll
          for (int ds = 0; ds < 2; ++ds)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const bf16x8 ak = read_row_op(Kr, 2 * kc + h2, r16, ds * 4 + g);
              const bf16x8 av = read_row_op(Vr, 2 * kc + h2, r16, ds * 4 + g);
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) {
                S[h2][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, Qb[qb][ds], S[h2][qb], 0, 0, 0);
                dP[h2][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, Db[qb][ds], dP[h2][qb], 0, 0, 0);
              }
            }
        };
        if (full) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) S[h2][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          products();
        } else {
          mask_bias_half(S, buckets, Kp[s], Kb[s], qcmp, qbkt, g, kc);
          products();
        }
        // dS^T = P^T (dP^T - Delta), P^T = exp2(S^T c - lse2)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pe = __builtin_amdgcn_exp2f(fmaf(S[h2][qb][e], p.c, -ql2[qb]));
              dP[h2][qb][e] = pe * dP[h2][qb][e];
            }
        // dQ^T += K^T dS^T (rows = dims, column = this lane's query)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 sp = pack_bf16x8(dP[0][qb], dP[1][qb]);
#pragma unroll
          for (int db = 0; db < 4; ++db)
            dQa[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_tr_op(Kt, db, kc, g, r16), sp, dQa[db][qb], 0,
                                                                 0, 0);
        }
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

  // ---- epilogue ------------------------------------------------------------
  float* tq = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const f32x4 a[4] = {dQa[0][qb], dQa[1][qb], dQa[2][qb], dQa[3][qb]};
    stage_rows(tq, w * 32 + qb * 16 + r16, g, a, p.scale);
  }
  __syncthreads();
  const int32_t* qi = p.q_idx + rowbase + qt * BM;  // this tile's index entries
  write_rows(tq, qi, BM, p.dQ, p.T, p.H, b, h);
  if constexpr (ZD) zero_unheld<BM>(p.q_idx + rowbase, qi, qt, p.TqP, p.T, p.H, b, h, p.dQ, nullptr);
}

// Workspace: log2 LSE and Delta per sorted query row.
size_t ws_layout(int B, int H, int TqP, size_t off[3]) {
  const size_t f = static_cast<size_t>(B) * H * TqP * 4;
  off[0] = 0;
  off[1] = (f + 255) & ~size_t(255);
  off[2] = off[1] + ((f + 255) & ~size_t(255));
  return off[2];
}

template <bool HASH, bool ZD>
int launch_bwd(const BwdParams& p, hipStream_t stream) {
  // dQ first: it also writes Delta and log2 LSE of every sorted query row,
  // which dK/dV reads
  hipLaunchKernelGGL((k_bwd_dq<HASH, ZD>), dim3(p.nQt * p.B * p.H), dim3(256), 0, stream, p);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  // hash ranges are short (one bucket's query tiles): more, smaller
  // workgroups keep the CUs busier than sharing each chunk between two tiles
  if constexpr (HASH)
    hipLaunchKernelGGL((k_bwd_dkdv64<HASH, ZD>), dim3(p.nKt * p.B * p.H), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_bwd_dkdv<HASH, ZD>), dim3((p.nKt + 1) / 2 * p.B * p.H), dim3(256), 0, stream, p);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

// Scratch of scfa_bwd_noalloc (log2 LSE and Delta of the sorted query
// rows), in place of a caller-supplied workspace. Each device holds its own
// copy for the life of the process; host code reaches it only through the
// address hipGetSymbolAddress returns for that device (the array's name is
// a host-side stand-in, not a device address). The dQ kernel writes every
// row of it before the dK/dV kernel reads it, so nothing has to be cleared
// between calls.
__device__ __align__(256) uint8_t scratch[SCFA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the device of `stream`, looked up once per
// device (with that device current, as it must be for the calls on it).
int scratch_of_stream(hipStream_t stream, uint8_t** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SCFA_ERR_HIP;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SCFA_ERR_HIP;
  if (dev != cur) return SCFA_ERR_INVALID;  // the stream must belong to the current device
  if (dev < 0 || dev >= kMaxDevices) return SCFA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SCFA_ERR_HIP;
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return SCFA_OK;
}

// Shared body of scfa_bwd and scfa_bwd_noalloc: argument checks, then the
// dQ kernel (which fills the workspace of log2 LSE and Delta) and the dK/dV
// kernel: `ws` (ws_bytes bytes) from the caller, or with `noalloc` the
// device's static scratch (after every argument check).
int bwd_run(int mode, int dtype_in, const void* q, const void* k, const void* v, const int32_t* q_idx,
            const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
            const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const int32_t* fwd_order,
            const int32_t* bwd_order, const float* O, const float* lse, const void* dO, int B, int H, int T, int T_kv,
            int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV, uint8_t* ws, size_t ws_bytes,
            bool noalloc, hipStream_t stream) {
  const int flags = take_flags(mode);
  if (!flags_ok(flags) || (mode != SCFA_QK && mode != SCFA_HASH)) return SCFA_ERR_INVALID;
  if (!q || !k || !v || !q_idx || !k_idx || !qstats || !kstats || !fwd_tab || !bwd_tab || !O || !lse || !dO || !dQ ||
      !dK || !dV || (!noalloc && !ws))
    return SCFA_ERR_INVALID;
  if (mode == SCFA_HASH && (!q_bkt || !k_bkt)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || T_kv < 1 || Tq < 1 || Tk < 1 || !(scale > 0.f) || !isfinite(scale))
    return SCFA_ERR_INVALID;
  if (!dtype_ok(dtype_in)) return SCFA_ERR_INVALID;
  if (D != HD || dtype_in != SCFA_BF16) return SCFA_ERR_UNSUPPORTED;
  // row offsets within one batch entry's (T, H, D) block are 32-bit
  if (static_cast<uint64_t>(max(T, T_kv)) * H * D * 2 > 0xFFFFFFFFull) return SCFA_ERR_UNSUPPORTED;
  if ((flags & SCFA_NONCAUSAL) && max(T, T_kv) > kPosLimit) return SCFA_ERR_UNSUPPORTED;
  if (mode == SCFA_QK && (Tq % SCFA_ROW_ALIGN || Tk != Tq)) return SCFA_ERR_INVALID;
  const int TqP = pad_rows(Tq), TkP = pad_rows(Tk);
  size_t off[3];
  if (noalloc) {
    if (ws_layout(B, H, TqP, off) > SCFA_NOALLOC_SCRATCH_BYTES) return SCFA_ERR_TOO_LARGE;
    const int st = scratch_of_stream(stream, &ws);
    if (st != SCFA_OK) return st;
  } else if (ws_bytes < ws_layout(B, H, TqP, off)) {
    return SCFA_ERR_INVALID;
  }
  BwdParams p{};
  p.rc = reach_of(flags);
  p.q = q;
  p.k = k;
  p.v = v;
  p.dO = dO;
  p.O = O;
  p.lse = lse;
  p.lse2 = reinterpret_cast<float*>(ws + off[0]);
  p.delta = reinterpret_cast<float*>(ws + off[1]);
  p.q_idx = q_idx;
  p.k_idx = k_idx;
  p.q_bkt = q_bkt;
  p.k_bkt = k_bkt;
  p.qstats = reinterpret_cast<const int4*>(qstats);
  p.kstats = reinterpret_cast<const int4*>(kstats);
  p.fwd_tab = reinterpret_cast<const int2*>(fwd_tab);
  p.bwd_tab = reinterpret_cast<const int2*>(bwd_tab);
  p.q_order = fwd_order;
  p.k_order = bwd_order;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = B;
  p.H = H;
  p.T = T;
  p.Tkv = T_kv;
  p.Tq = Tq;
  p.Tk = Tk;
  p.TqP = TqP;
  p.TkP = TkP;
  p.nQt = TqP / BM;
  p.nKt = TkP / BN;
  p.c = scale * kLog2e;
  p.scale = scale;
  if (mode == SCFA_HASH) return launch_bwd<true, false>(p, stream);
  return launch_bwd<false, true>(p, stream);
}


}  // namespace
}  // namespace scfa

using namespace scfa;

extern "C" {

size_t scfa_bwd_workspace_bytes(int mode, int B, int H, int Tq, int Tk, int D) {
  if (!flags_ok(take_flags(mode))) return 0;
  if ((mode != SCFA_QK && mode != SCFA_HASH) || B < 1 || H < 1 || Tq < 1 || Tk < 1 || D != HD) return 0;
  size_t off[3];
  return ws_layout(B, H, pad_rows(Tq), off);
}

int scfa_bwd(int mode, int dtype_in, const void* q, const void* k, const void* v, const int32_t* q_idx,
             const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
             const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const int32_t* fwd_order,
             const int32_t* bwd_order, const float* O, const float* lse, const void* dO, int B, int H, int T, int T_kv,
             int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  return bwd_run(mode, dtype_in, q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, bwd_tab, fwd_order,
                 bwd_order, O, lse, dO, B, H, T, T_kv, Tq, Tk, D, scale, dQ, dK, dV, static_cast<uint8_t*>(workspace),
                 workspace_bytes, false, stream);
}

int scfa_bwd_noalloc(int mode, int dtype_in, const void* q, const void* k, const void* v, const int32_t* q_idx,
                     const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
                     const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const int32_t* fwd_order,
                     const int32_t* bwd_order, const float* O, const float* lse, const void* dO, int B, int H, int T,
                     int T_kv, int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV, hipStream_t stream) {
  return bwd_run(mode, dtype_in, q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, bwd_tab, fwd_order,
                 bwd_order, O, lse, dO, B, H, T, T_kv, Tq, Tk, D, scale, dQ, dK, dV, nullptr, 0, true, stream);
}

}  // extern "C"
