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
//  * Three kernels, no atomics (deterministic): a preparation kernel (dO in
//    sorted order, Delta, log2 LSE), dK/dV per 64-key tile (4 waves x 16
//    keys, query chunks of 64 double-buffered in LDS), dQ per 128-query tile
//    (4 waves x 32 queries, key tiles of 64 double-buffered in LDS).
//  * All six products are v_mfma_f32_16x16x32_bf16. The score-like tiles
//    (S, dP) are laid out so that each lane owns one column (a key in dK/dV,
//    a query in dQ) and 4 rows per 16x16 block; their A-operand rows are
//    permuted so a lane's 8 probabilities cover 8 consecutive rows, which
//    lets P and dS feed the next MFMA directly as B operands against a
//    transposed operand read with one 16-byte LDS load.
//  * Operands needed transposed (Q^T, dO^T for dK/dV; K^T for dQ) are
//    produced once by a tiled transpose into the workspace.
//  * Gradients are staged in LDS and written as whole rows at the original
//    token positions; QK-drop zeroes the rows of dropped tokens.

#include <math.h>

#include "scfa_mfma.h"

namespace scfa {
namespace {

constexpr int BM = SCFA_TILE_M;  // 128: dQ workgroup rows, table granularity
constexpr int BN = SCFA_TILE_N;  // 64: dK/dV workgroup keys, table granularity
constexpr int QC = 64;           // query chunk of the dK/dV loop
constexpr int HD = 64;
constexpr int TB = 64 * HD * 2;  // bytes of one 64 x 64 bf16 tile

struct BwdParams {
  const uint16_t* q_s;   // (BH, Tp, D) rows
  const uint16_t* k_s;   // (BH, Tp, D) rows
  const uint16_t* v_s;   // (BH, Tp, D) rows
  const uint16_t* q_t;   // (BH, D, Tp)
  const uint16_t* k_t;   // (BH, D, Tp)
  const uint16_t* do_s;  // (BH, Tp, D) rows
  const uint16_t* do_t;  // (BH, D, Tp)
  const float* lse2;     // (BH, Tp) log2-domain LSE, +inf when no visible key / pad row
  const float* delta;    // (BH, Tp)
  const int32_t* q_idx;
  const int32_t* k_idx;
  const int32_t* q_bkt;
  const int32_t* k_bkt;
  const int4* qstats;
  const int4* kstats;
  const int2* fwd_tab;
  const int2* bwd_tab;
  float* dQ;
  float* dK;
  float* dV;
  int B, H, T;
  int Tq, Tk;    // valid query / key rows (as passed to the range table)
  int TqP, TkP;  // rows per head of the query-side / key-side buffers
  int nQt, nKt;
  float c;      // scale * log2(e)
  float scale;  // score scale
};

// ---------------------------------------------------------------------------
// Preparation: dO gathered to sorted order, Delta = dO . O, log2 LSE.
// 8 threads per row (8 dims each), 32 rows per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_prep(const uint16_t* __restrict__ dO, const float* __restrict__ O,
                                                  const float* __restrict__ lse, const int32_t* __restrict__ q_idx,
                                                  int H, int T, int Tp, uint16_t* __restrict__ do_s,
                                                  float* __restrict__ lse2, float* __restrict__ delta) {
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int r = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const int qp = q_idx[static_cast<size_t>(bh) * Tp + r];
  const bool valid = qp >= 0 && qp < T;
  u32x4 dv = {0u, 0u, 0u, 0u};
  float s = 0.f;
  if (valid) {
    const size_t row = (static_cast<size_t>(b) * T + qp) * H + h;
    dv = *reinterpret_cast<const u32x4*>(dO + row * HD + part * 8);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + row * HD + part * 8);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + row * HD + part * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(dv[i] << 16), hi = __uint_as_float(dv[i] & 0xffff0000u);
      s += lo * (i < 2 ? o0[2 * i] : o1[2 * i - 4]) + hi * (i < 2 ? o0[2 * i + 1] : o1[2 * i - 3]);
    }
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  *reinterpret_cast<u32x4*>(do_s + (static_cast<size_t>(bh) * Tp + r) * HD + part * 8) = dv;
  if (part == 0) {
    const size_t o = static_cast<size_t>(bh) * Tp + r;
    delta[o] = valid ? s : 0.f;
    const float l = valid ? lse[static_cast<size_t>(bh) * T + qp] : -INFINITY;
    lse2[o] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// (BH, Tp, 64) rows <-> (BH, 64, Tp) columns, one 64 x 64 tile per workgroup.
template <bool TO_COLS>
__global__ __launch_bounds__(256) void k_transpose(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int Tp) {
  __shared__ uint16_t t[64][66];
  const int bh = blockIdx.y;
  const int r0 = blockIdx.x * 64;
  const size_t base = static_cast<size_t>(bh) * Tp * HD;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = threadIdx.x + 256 * i;  // 512 units of 8 elements
    const int a = u >> 3, c8 = (u & 7) * 8;
    u32x4 v;
    if (TO_COLS)
      v = *reinterpret_cast<const u32x4*>(in + base + static_cast<size_t>(r0 + a) * HD + c8);  // row a
    else
      v = *reinterpret_cast<const u32x4*>(in + base + static_cast<size_t>(a) * Tp + r0 + c8);  // dim a
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[a][c8 + 2 * e] = static_cast<uint16_t>(v[e] & 0xffffu);
      t[a][c8 + 2 * e + 1] = static_cast<uint16_t>(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int a = u >> 3, c8 = (u & 7) * 8;  // output line a, 8 consecutive elements
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<uint32_t>(t[c8 + 2 * e][a]) | (static_cast<uint32_t>(t[c8 + 2 * e + 1][a]) << 16);
    if (TO_COLS)
      *reinterpret_cast<u32x4*>(out + base + static_cast<size_t>(a) * Tp + r0 + c8) = v;
    else
      *reinterpret_cast<u32x4*>(out + base + static_cast<size_t>(r0 + a) * HD + c8) = v;
  }
}

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
  for (int base = lo; base <= hi; base += 16) {
    const int pos = base + (tid >> 4);
    const int u = tid & 15;
    if (pos <= hi) {
      int a = 0, z = nreal;
      while (a < z) {
        const int mid = (a + z) >> 1;
        if (ti[mid] < pos) a = mid + 1; else z = mid;
      }
      if (!(a < nreal && ti[a] == pos)) {
        const size_t o = ((static_cast<size_t>(b) * T + pos) * H + h) * HD;
        reinterpret_cast<f32x4*>(out0 + o)[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (out1) reinterpret_cast<f32x4*>(out1 + o)[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
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

// 64 x 64 bf16 tile loads: rows (64 rows x 128 B contiguous) and transposed
// (64 lines of 128 B at a stride of Tpad elements), 2 x 16 B per thread.
struct Tile2 {
  u32x4 a, b;
};
__device__ __forceinline__ Tile2 load_rows_tile(const uint16_t* base, int tid) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base);
  return Tile2{p[tid], p[tid + 256]};
}
__device__ __forceinline__ Tile2 load_cols_tile(const uint16_t* base, int Tpad, int tid) {
  const int u0 = tid, u1 = tid + 256;
  return Tile2{*reinterpret_cast<const u32x4*>(base + static_cast<size_t>(u0 >> 3) * Tpad + (u0 & 7) * 8),
               *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(u1 >> 3) * Tpad + (u1 & 7) * 8)};
}
// Rows are read as A operands with permuted rows (swz_k); transposed tiles
// are read line by line (swizzle line & 7).
__device__ __forceinline__ void store_rows_tile(uint8_t* lds, const Tile2& t, int tid) {
  const int u0 = tid, u1 = tid + 256;
  *reinterpret_cast<u32x4*>(lds + (u0 >> 3) * 128 + (((u0 & 7) ^ swz_k(u0 >> 3)) * 16)) = t.a;
  *reinterpret_cast<u32x4*>(lds + (u1 >> 3) * 128 + (((u1 & 7) ^ swz_k(u1 >> 3)) * 16)) = t.b;
}
__device__ __forceinline__ void store_cols_tile(uint8_t* lds, const Tile2& t, int tid) {
  const int u0 = tid, u1 = tid + 256;
  *reinterpret_cast<u32x4*>(lds + (u0 >> 3) * 128 + (((u0 & 7) ^ ((u0 >> 3) & 7)) * 16)) = t.a;
  *reinterpret_cast<u32x4*>(lds + (u1 >> 3) * 128 + (((u1 & 7) ^ ((u1 >> 3) & 7)) * 16)) = t.b;
}
// A operand of a permuted-row tile: block blk, lane row r16, k-chunk ch.
__device__ __forceinline__ bf16x8 read_rows_op(const uint8_t* lds, int blk, int r16, int ch) {
  const int row = key_row(blk, r16);
  return *reinterpret_cast<const bf16x8*>(lds + row * 128 + ((ch ^ swz_k(row)) * 16));
}
// A operand of a transposed tile: line d, 8 consecutive entries at chunk ch.
__device__ __forceinline__ bf16x8 read_cols_op(const uint8_t* lds, int d, int ch) {
  return *reinterpret_cast<const bf16x8*>(lds + d * 128 + ((ch ^ (d & 7)) * 16));
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

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 64-key tile.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZD>
__global__ __launch_bounds__(256) void k_bwd_dkdv(BwdParams p) {
  __shared__ __align__(16) uint8_t stage[2][4 * TB];  // Q rows, Q^T, dO rows, dO^T
  __shared__ __align__(16) int32_t qpos_s[2][QC];
  __shared__ __align__(16) int32_t qbkt_s[2][QC];
  __shared__ __align__(16) float lse_s[2][QC];
  __shared__ __align__(16) float del_s[2][QC];
  __shared__ int32_t Ki[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int BH = p.B * p.H;
  int kt, bh;
  map_work(blockIdx.x, BH, p.nKt, kt, bh, false);  // early key tiles see the most queries
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqP;        // query side
  const size_t colbase = static_cast<size_t>(bh) * HD * p.TqP;
  const size_t kbase = static_cast<size_t>(bh) * p.TkP;          // key side

  if (tid < BN) Ki[tid] = p.k_idx[kbase + kt * BN + tid];
  const int krow = kt * BN + w * 16 + r16;  // this lane's key
  const int kpos = p.k_idx[kbase + krow];
  const int kbkt = HASH ? p.k_bkt[kbase + krow] : 0;
  bf16x8 Kb[2], Vb[2];
#pragma unroll
  for (int ds = 0; ds < 2; ++ds) {
    Kb[ds] = *reinterpret_cast<const bf16x8*>(p.k_s + (kbase + krow) * HD + ds * 32 + g * 8);
    Vb[ds] = *reinterpret_cast<const bf16x8*>(p.v_s + (kbase + krow) * HD + ds * 32 + g * 8);
  }
  f32x4 dVa[4], dKa[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dVa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int2 rng = p.bwd_tab[static_cast<size_t>(bh) * p.nKt + kt];
  const int4 ks = p.kstats[static_cast<size_t>(bh) * p.nKt + kt];
  const int4* qst = p.qstats + static_cast<size_t>(bh) * p.nQt;
  const bool kfull = (kt + 1) * BN <= p.Tk;

  // chunk ci = 2 * query tile + half; skip tiles failing the causal test
  auto next_chunk = [&](int ci) {
    while (ci < 2 * rng.y && qst[ci >> 1].y < ks.x) ci = (ci | 1) + 1;
    return ci;
  };
  Tile2 rq, rqt, rdo, rdot;
  float rsc = 0.f;
  int rsi = 0;
  auto load = [&](int ci) {
    const int q0 = ci * QC;
    rq = load_rows_tile(p.q_s + (rowbase + q0) * HD, tid);
    rqt = load_cols_tile(p.q_t + colbase + q0, p.TqP, tid);
    rdo = load_rows_tile(p.do_s + (rowbase + q0) * HD, tid);
    rdot = load_cols_tile(p.do_t + colbase + q0, p.TqP, tid);
    const int which = tid >> 6, r = tid & 63;
    if (which == 0) rsi = p.q_idx[rowbase + q0 + r];
    else if (which == 1) rsi = HASH ? p.q_bkt[rowbase + q0 + r] : 0;
    else if (which == 2) rsc = p.lse2[rowbase + q0 + r];
    else rsc = p.delta[rowbase + q0 + r];
  };
  auto store = [&](int s) {
    store_rows_tile(stage[s], rq, tid);
    store_cols_tile(stage[s] + TB, rqt, tid);
    store_rows_tile(stage[s] + 2 * TB, rdo, tid);
    store_cols_tile(stage[s] + 3 * TB, rdot, tid);
    const int which = tid >> 6, r = tid & 63;
    if (which == 0) qpos_s[s][r] = rsi;
    else if (which == 1) qbkt_s[s][r] = rsi;
    else if (which == 2) lse_s[s][r] = rsc;
    else del_s[s][r] = rsc;
  };

  int ci = next_chunk(2 * rng.x);
  if (ci < 2 * rng.y) {
    load(ci);
    store(0);
  }
  __syncthreads();
  int s = 0;
  while (ci < 2 * rng.y) {
    const int cn = next_chunk(ci + 1);
    if (cn < 2 * rng.y) load(cn);
    const uint8_t* Qr = stage[s];
    const uint8_t* Qt = stage[s] + TB;
    const uint8_t* Dr = stage[s] + 2 * TB;
    const uint8_t* Dt = stage[s] + 3 * TB;

    // S = Q K^T and dP = dO V^T: lane column = this lane's key, rows = queries
    f32x4 S[4], dP[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      S[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dP[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        S[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_rows_op(Qr, qb, r16, ds * 4 + g), Kb[ds], S[qb], 0, 0, 0);
        dP[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_rows_op(Dr, qb, r16, ds * 4 + g), Vb[ds], dP[qb], 0, 0, 0);
      }

    const int4 qs = qst[ci >> 1];
    bool full = kfull && ks.y <= qs.x && ((ci >> 1) + 1) * BM <= p.Tq;
    if (HASH) full = full && ks.z == ks.w && qs.z == qs.w && ks.z == qs.z;
    bf16x8 Pp[2], Sp[2];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int qo = 32 * (qb >> 1) + 8 * g + 4 * (qb & 1);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[s][qo]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&del_s[s][qo]);
      int4 qp4 = make_int4(0, 0, 0, 0), qb4 = make_int4(0, 0, 0, 0);
      if (!full) {
        qp4 = *reinterpret_cast<const int4*>(&qpos_s[s][qo]);
        if (HASH) qb4 = *reinterpret_cast<const int4*>(&qbkt_s[s][qo]);
      }
      f32x4 P, dS;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qpe = e == 0 ? qp4.x : e == 1 ? qp4.y : e == 2 ? qp4.z : qp4.w;
        const int qbe = e == 0 ? qb4.x : e == 1 ? qb4.y : e == 2 ? qb4.z : qb4.w;
        const bool vis = full || (qpe >= kpos && (!HASH || qbe == kbkt));
        const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(S[qb][e], p.c, -l4[e])) : 0.f;
        P[e] = pe;
        dS[e] = pe * (dP[qb][e] - d4[e]);
      }
      S[qb] = P;
      dP[qb] = dS;
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      Pp[kc] = pack_bf16x8(S[2 * kc], S[2 * kc + 1]);
      Sp[kc] = pack_bf16x8(dP[2 * kc], dP[2 * kc + 1]);
    }
    // dV^T += dO^T P,  dK^T += Q^T dS  (rows = dims, column = this lane's key)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int d = db * 16 + r16;
        dVa[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_cols_op(Dt, d, kc * 4 + g), Pp[kc], dVa[db], 0, 0, 0);
        dKa[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_cols_op(Qt, d, kc * 4 + g), Sp[kc], dKa[db], 0, 0, 0);
      }

    if (cn < 2 * rng.y) store(s ^ 1);
    __syncthreads();
    s ^= 1;
    ci = cn;
  }

  // ---- epilogue: stage dK (scaled) and dV in LDS, write whole rows ---------
  float* tk = reinterpret_cast<float*>(&stage[0][0]);
  float* tv = tk + BN * HD;
  const int row = w * 16 + r16;
  stage_rows(tk, row, g, dKa, p.scale);
  stage_rows(tv, row, g, dVa, 1.f);
  __syncthreads();
  write_rows(tk, Ki, BN, p.dK, p.T, p.H, b, h);
  write_rows(tv, Ki, BN, p.dV, p.T, p.H, b, h);
  if constexpr (ZD) zero_unheld<BN>(p.k_idx + kbase, Ki, kt, p.TkP, p.T, p.H, b, h, p.dK, p.dV);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128-query tile, over the forward table's key tiles.
// ---------------------------------------------------------------------------
template <bool HASH, bool ZD>
__global__ __launch_bounds__(256) void k_bwd_dq(BwdParams p) {
  __shared__ __align__(16) uint8_t stage[2][3 * TB];  // K rows, V rows, K^T
  __shared__ __align__(16) int32_t kpos_s[2][BN];
  __shared__ __align__(16) int32_t kbkt_s[2][BN];
  __shared__ int32_t Qi[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int BH = p.B * p.H;
  int qt, bh;
  map_work(blockIdx.x, BH, p.nQt, qt, bh, true);
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t rowbase = static_cast<size_t>(bh) * p.TqP;        // query side
  const size_t kbase = static_cast<size_t>(bh) * p.TkP;          // key side
  const size_t kcolbase = static_cast<size_t>(bh) * HD * p.TkP;
  if (tid < BM) Qi[tid] = p.q_idx[rowbase + qt * BM + tid];

  const int q0 = qt * BM + w * 32;
  int qpos[2], qbkt[2];
  float ql2[2], qdl[2];
  bf16x8 Qb[2][2], Db[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 16 + r16;
    qpos[qb] = p.q_idx[rowbase + row];
    qbkt[qb] = HASH ? p.q_bkt[rowbase + row] : 0;
    ql2[qb] = p.lse2[rowbase + row];
    qdl[qb] = p.delta[rowbase + row];
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      Qb[qb][ds] = *reinterpret_cast<const bf16x8*>(p.q_s + (rowbase + row) * HD + ds * 32 + g * 8);
      Db[qb][ds] = *reinterpret_cast<const bf16x8*>(p.do_s + (rowbase + row) * HD + ds * 32 + g * 8);
    }
  }
  f32x4 dQa[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dQa[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int2 rng = p.fwd_tab[static_cast<size_t>(bh) * p.nQt + qt];
  const int4 qs = p.qstats[static_cast<size_t>(bh) * p.nQt + qt];
  const int4* kst = p.kstats + static_cast<size_t>(bh) * p.nKt;
  const bool qfull = (qt + 1) * BM <= p.Tq;
  auto next_tile = [&](int j) {
    while (j < rng.y && kst[j].x > qs.y) ++j;
    return j;
  };
  Tile2 rk, rv, rkt;
  int ri = 0;
  auto load = [&](int j) {
    rk = load_rows_tile(p.k_s + (kbase + j * BN) * HD, tid);
    rv = load_rows_tile(p.v_s + (kbase + j * BN) * HD, tid);
    rkt = load_cols_tile(p.k_t + kcolbase + j * BN, p.TkP, tid);
    if (tid < BN) ri = p.k_idx[kbase + j * BN + tid];
    else if (HASH && tid < 2 * BN) ri = p.k_bkt[kbase + j * BN + tid - BN];
  };
  auto store = [&](int s) {
    store_rows_tile(stage[s], rk, tid);
    store_rows_tile(stage[s] + TB, rv, tid);
    store_cols_tile(stage[s] + 2 * TB, rkt, tid);
    if (tid < BN) kpos_s[s][tid] = ri;
    else if (HASH && tid < 2 * BN) kbkt_s[s][tid - BN] = ri;
  };

  int j = next_tile(rng.x);
  if (j < rng.y) {
    load(j);
    store(0);
  }
  __syncthreads();
  int s = 0;
  while (j < rng.y) {
    const int jn = next_tile(j + 1);
    if (jn < rng.y) load(jn);
    const uint8_t* Kr = stage[s];
    const uint8_t* Vr = stage[s] + TB;
    const uint8_t* Kt = stage[s] + 2 * TB;

    // S^T = K Q^T and dP^T = V dO^T: lane column = query, rows = keys
    f32x4 S[4][2], dP[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        S[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dP[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 ak = read_rows_op(Kr, kb, r16, ds * 4 + g);
        const bf16x8 av = read_rows_op(Vr, kb, r16, ds * 4 + g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, Qb[qb][ds], S[kb][qb], 0, 0, 0);
          dP[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, Db[qb][ds], dP[kb][qb], 0, 0, 0);
        }
      }
    const int4 ks = kst[j];
    bool full = qfull && ks.y <= qs.x && (j + 1) * BN <= p.Tk;
    if (HASH) full = full && ks.z == ks.w && qs.z == qs.w && ks.z == qs.z;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int kbase = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
      int4 kp4 = make_int4(0, 0, 0, 0), kb4 = make_int4(0, 0, 0, 0);
      if (!full) {
        kp4 = *reinterpret_cast<const int4*>(&kpos_s[s][kbase]);
        if (HASH) kb4 = *reinterpret_cast<const int4*>(&kbkt_s[s][kbase]);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kpe = e == 0 ? kp4.x : e == 1 ? kp4.y : e == 2 ? kp4.z : kp4.w;
          const int kbe = e == 0 ? kb4.x : e == 1 ? kb4.y : e == 2 ? kb4.z : kb4.w;
          const bool vis = full || (kpe <= qpos[qb] && (!HASH || kbe == qbkt[qb]));
          const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(S[kb][qb][e], p.c, -ql2[qb])) : 0.f;
          dP[kb][qb][e] = pe * (dP[kb][qb][e] - qdl[qb]);
        }
    }
    // dQ^T += K^T dS^T (rows = dims, column = this lane's query)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const bf16x8 sp = pack_bf16x8(dP[2 * kc][qb], dP[2 * kc + 1][qb]);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dQa[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_cols_op(Kt, db * 16 + r16, kc * 4 + g), sp,
                                                               dQa[db][qb], 0, 0, 0);
      }

    if (jn < rng.y) store(s ^ 1);
    __syncthreads();
    s ^= 1;
    j = jn;
  }

  // ---- epilogue ------------------------------------------------------------
  float* tq = reinterpret_cast<float*>(&stage[0][0]);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const f32x4 a[4] = {dQa[0][qb], dQa[1][qb], dQa[2][qb], dQa[3][qb]};
    stage_rows(tq, w * 32 + qb * 16 + r16, g, a, p.scale);
  }
  __syncthreads();
  write_rows(tq, Qi, BM, p.dQ, p.T, p.H, b, h);
  if constexpr (ZD) zero_unheld<BM>(p.q_idx + rowbase, Qi, qt, p.TqP, p.T, p.H, b, h, p.dQ, nullptr);
}

// Workspace: v_s and k_t on the key side, q_t, do_s, do_t, lse2 and delta on
// the query side.
size_t ws_layout(int B, int H, int TqP, int TkP, size_t off[8]) {
  const size_t bfq = static_cast<size_t>(B) * H * TqP * HD * 2;  // one bf16 (BH, TqP, D) tensor
  const size_t bfk = static_cast<size_t>(B) * H * TkP * HD * 2;
  const size_t f = static_cast<size_t>(B) * H * TqP * 4;
  size_t o = 0;
  for (int i = 0; i < 5; ++i) {  // v_s, q_t, k_t, do_s, do_t
    off[i] = o;
    const size_t bf = (i == 0 || i == 2) ? bfk : bfq;
    o += (bf + 255) & ~size_t(255);
  }
  off[5] = o;  // lse2
  o += (f + 255) & ~size_t(255);
  off[6] = o;  // delta
  o += (f + 255) & ~size_t(255);
  off[7] = o;
  return o;
}

template <bool HASH, bool ZD>
int launch_bwd(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((k_bwd_dkdv<HASH, ZD>), dim3(p.nKt * p.B * p.H), dim3(256), 0, stream, p);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL((k_bwd_dq<HASH, ZD>), dim3(p.nQt * p.B * p.H), dim3(256), 0, stream, p);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

}  // namespace
}  // namespace scfa

using namespace scfa;

extern "C" {

size_t scfa_bwd_workspace_bytes(int mode, int B, int H, int Tq, int Tk, int D) {
  if ((mode != SCFA_QK && mode != SCFA_HASH) || B < 1 || H < 1 || Tq < 1 || Tk < 1 || D != HD) return 0;
  size_t off[8];
  return ws_layout(B, H, pad_rows(Tq), pad_rows(Tk), off);
}

int scfa_bwd(int mode, int dtype_in, const void* q, const void* k, const void* v_t, const int32_t* q_idx,
             const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
             const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const float* O, const float* lse,
             const void* dO, int B, int H, int T, int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (mode != SCFA_QK && mode != SCFA_HASH) return SCFA_ERR_INVALID;
  if (!q || !k || !v_t || !q_idx || !k_idx || !qstats || !kstats || !fwd_tab || !bwd_tab || !O || !lse || !dO ||
      !dQ || !dK || !dV || !workspace)
    return SCFA_ERR_INVALID;
  if (mode == SCFA_HASH && (!q_bkt || !k_bkt)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || Tq < 1 || Tk < 1 || !(scale > 0.f) || !isfinite(scale)) return SCFA_ERR_INVALID;
  if (!dtype_ok(dtype_in)) return SCFA_ERR_INVALID;
  if (D != HD || dtype_in != SCFA_BF16) return SCFA_ERR_UNSUPPORTED;
  if (mode == SCFA_QK && (Tq % SCFA_ROW_ALIGN || Tk != Tq)) return SCFA_ERR_INVALID;
  const int TqP = pad_rows(Tq), TkP = pad_rows(Tk);
  size_t off[8];
  if (workspace_bytes < ws_layout(B, H, TqP, TkP, off)) return SCFA_ERR_INVALID;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  BwdParams p{};
  p.q_s = static_cast<const uint16_t*>(q);
  p.k_s = static_cast<const uint16_t*>(k);
  p.v_s = reinterpret_cast<uint16_t*>(ws + off[0]);
  p.q_t = reinterpret_cast<uint16_t*>(ws + off[1]);
  p.k_t = reinterpret_cast<uint16_t*>(ws + off[2]);
  p.do_s = reinterpret_cast<uint16_t*>(ws + off[3]);
  p.do_t = reinterpret_cast<uint16_t*>(ws + off[4]);
  p.lse2 = reinterpret_cast<float*>(ws + off[5]);
  p.delta = reinterpret_cast<float*>(ws + off[6]);
  p.q_idx = q_idx;
  p.k_idx = k_idx;
  p.q_bkt = q_bkt;
  p.k_bkt = k_bkt;
  p.qstats = reinterpret_cast<const int4*>(qstats);
  p.kstats = reinterpret_cast<const int4*>(kstats);
  p.fwd_tab = reinterpret_cast<const int2*>(fwd_tab);
  p.bwd_tab = reinterpret_cast<const int2*>(bwd_tab);
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = B;
  p.H = H;
  p.T = T;
  p.Tq = Tq;
  p.Tk = Tk;
  p.TqP = TqP;
  p.TkP = TkP;
  p.nQt = TqP / BM;
  p.nKt = TkP / BN;
  p.c = scale * kLog2e;
  p.scale = scale;
  const int BH = B * H;
  // preparation: transposes / row copies of the sorted operands, dO, Delta, LSE
  hipLaunchKernelGGL(k_transpose<false>, dim3(TkP / 64, BH), dim3(256), 0, stream, static_cast<const uint16_t*>(v_t),
                     const_cast<uint16_t*>(p.v_s), TkP);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_transpose<true>, dim3(TqP / 64, BH), dim3(256), 0, stream, p.q_s, const_cast<uint16_t*>(p.q_t),
                     TqP);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_transpose<true>, dim3(TkP / 64, BH), dim3(256), 0, stream, p.k_s, const_cast<uint16_t*>(p.k_t),
                     TkP);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_bwd_prep, dim3(TqP / 32, BH), dim3(256), 0, stream, static_cast<const uint16_t*>(dO), O, lse,
                     q_idx, H, T, TqP, const_cast<uint16_t*>(p.do_s), const_cast<float*>(p.lse2),
                     const_cast<float*>(p.delta));
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_transpose<true>, dim3(TqP / 64, BH), dim3(256), 0, stream, p.do_s, const_cast<uint16_t*>(p.do_t),
                     TqP);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  if (mode == SCFA_HASH) return launch_bwd<true, false>(p, stream);
  return launch_bwd<false, true>(p, stream);
}

}  // extern "C"
