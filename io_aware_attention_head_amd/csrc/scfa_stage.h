// Staging helpers shared by the attention kernels (gfx950): global -> LDS
// DMA of index-gathered rows, the XOR layout for transposed LDS reads, and
// the VCC-only selects that build mask biases.
#pragma once

#include "scfa_mfma.h"

namespace scfa {

// Global -> LDS DMA without registers: each lane's 16 (or 4) bytes land at
// consecutive LDS addresses from the wave-uniform byte address `lds`; the
// source is a wave-uniform base plus a per-lane 32-bit offset. Issued as
// inline assembly so that the compiler does not order the LDS reads of the
// other stage behind it; completion is awaited with dma_wait() before the
// barrier that publishes the stage.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt not waited on), as a builtin so that
// the compiler knows every earlier vector-memory load has completed.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0xF70); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  const __attribute__((address_space(3))) void* lp = (const __attribute__((address_space(3))) void*)p;
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lp);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Tile statistics entry of a range: from its LDS copy when the range fits
// the copy, else from global memory. The two reads stay two loads in two
// branches (pointers of their own address spaces, and a scheduling barrier
// that makes the branches differ): folded into one load of a selected
// pointer they become a flat load, which waits on every outstanding memory
// operation (the K/V DMA included) instead of the LDS alone.
__device__ __forceinline__ int4 stat_entry(bool in_lds, const int4* lds_copy, int li, const int4* glob, int gi) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(3))) i32x4 lds_i32x4;
  typedef const __attribute__((address_space(1))) i32x4 glb_i32x4;
  i32x4 v;
  if (in_lds) {
    v = *(lds_i32x4*)(lds_copy + li);
  } else {
    v = *(glb_i32x4*)(glob + gi);
    __builtin_amdgcn_sched_barrier(0);  // the branches differ: no common load to sink
  }
  return make_int4(v[0], v[1], v[2], v[3]);
}

// Row of the original (B, T, H, D) tensors for an index entry: pads (and any
// entry outside [0, T)) read token 0, whose values are finite.
__device__ inline int src_row(int pos, int T) { return (pos >= 0 && pos < T) ? pos : 0; }

// Transposed A operand (16 x 32, bf16) from a row-major 64 x 64 tile stored
// with the swz_k layout (the layout of the row operand reads, so that one
// staged copy of a tile serves both kinds of read): operand row = column
// 16 db + r16 of the tile, k = tile rows 32 kc + 8 g .. 32 kc + 8 g + 7, as
// two ds_read_b64_tr_b16 of 4 rows each (within a 16-lane group, source lane
// r16 reads 4 columns of tile row 32 kc + 8 g + 4 hh + r16 / 4). Measured on
// gfx950, these reads run as fast from the swz_k layout as from any other
// XOR layout of the 16-byte chunks, while the row reads need swz_k.
__device__ __forceinline__ bf16x8 read_tr_op(const uint8_t* tile, int db, int kc, int g, int r16) {
  v4i16 t[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 32 * kc + 8 * g + 4 * hh + (r16 >> 2);
    const int col = 16 * db + 4 * (r16 & 3);  // first of the 4 columns
    const uint8_t* src = tile + r * 128 + (((col >> 3) ^ swz_k(r)) * 16) + (col & 7) * 2;
    t[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(__attribute__((address_space(3))) void*)src);
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row A operand of a tile stored with the swz_k layout: block blk (16 rows,
// permuted by key_row), k chunk ch (8 elements).
__device__ __forceinline__ bf16x8 read_row_op(const uint8_t* tile, int blk, int r16, int ch) {
  const int row = key_row(blk, r16);
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((ch ^ swz_k(row)) * 16));
}

// The compares below go to VCC and are consumed at once, so a masked tile
// holds no per-element lane masks in scalar registers (-inf comes from a
// VGPR: VCC already takes the one scalar operand slot).
// 0 if a >= b, else -inf.
__device__ __forceinline__ float bias_if_ge(int a, int b) {
  float r;
  asm("v_cmp_ge_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e64 %0, %3, 0, vcc"
      : "=v"(r)
      : "v"(a), "v"(b), "v"(0xff800000u)
      : "vcc");
  return r;
}
// x if a == b, else -inf.
__device__ __forceinline__ float keep_if_eq(float x, int a, int b) {
  asm("v_cmp_eq_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %3, %0, vcc"
      : "+v"(x)
      : "v"(a), "v"(b), "v"(0xff800000u)
      : "vcc");
  return x;
}

// ---------------------------------------------------------------------------
// Per-wave tile tests and mask biases of a wave that owns 32 query columns
// (two 16-query MFMA column blocks) against a 64-key tile.
// ---------------------------------------------------------------------------
constexpr int kKeyTile = SCFA_TILE_N;

// Extrema of this wave's real query rows (pad rows: position -1, their
// results are never stored): a key tile is skipped by the whole wave when it
// holds no pair visible to any of them, and unmasked when every pair is
// visible to all of them. All 4 lane groups hold the same 2 x 16 rows.
struct WaveRows {
  int minpos, maxpos, minb, maxb;
};

// The extrema are of q_reach(position), the largest key position each query
// may see, so that every tile test compares keys against them unchanged.
__device__ inline WaveRows wave_rows(const int (&qpos)[2], const int (&qbkt)[2], const Reach& rc) {
  WaveRows s{kInt32Max, q_reach(rc, -1), kInt32Max, kInt32Min};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qpos[qb] >= 0) {
      s.minpos = min(s.minpos, q_reach(rc, qpos[qb]));
      s.maxpos = max(s.maxpos, q_reach(rc, qpos[qb]));
      s.minb = min(s.minb, qbkt[qb]);
      s.maxb = max(s.maxb, qbkt[qb]);
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    s.minpos = min(s.minpos, __shfl_xor(s.minpos, o));
    s.maxpos = max(s.maxpos, __shfl_xor(s.maxpos, o));
    s.minb = min(s.minb, __shfl_xor(s.minb, o));
    s.maxb = max(s.maxb, __shfl_xor(s.maxb, o));
  }
  // wave-uniform from here on: tile tests become scalar branches
  s.minpos = __builtin_amdgcn_readfirstlane(s.minpos);
  s.maxpos = __builtin_amdgcn_readfirstlane(s.maxpos);
  s.minb = __builtin_amdgcn_readfirstlane(s.minb);
  s.maxb = __builtin_amdgcn_readfirstlane(s.maxb);
  return s;
}

template <bool HASH>
__device__ inline bool tile_empty_for(const int4& ks, const WaveRows& wr) {
  return ks.x > wr.maxpos || (HASH && (ks.w < wr.minb || ks.z > wr.maxb));
}

template <bool HASH>
__device__ inline bool tile_full_for(const int4& ks, const WaveRows& wr, int j, int Tk) {
  bool full = ks.y <= wr.minpos && (j + 1) * kKeyTile <= Tk;
  if (HASH) full = full && ks.z == ks.w && wr.minb == wr.maxb && ks.z == wr.minb;
  return full;
}


// Mask bias of a tile: element e of block kb in lane group g (key
// 32 (kb >> 1) + 8 g + 4 (kb & 1) + e of the tile) is 0 if that key is
// visible to the lane's query, else -inf. BUCKETS: also compare buckets (not
// needed when the tile and the wave's queries are all in one bucket: a tile
// that is not skipped then has the queries' bucket).
template <bool BUCKETS>
__device__ inline void bias_tile(f32x4 (&C)[4][2], const int32_t* kp, const int32_t* kbk, const int (&qpos)[2],
                                 const int (&qbkt)[2], int g) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int kbase = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
    const int4 kp4 = *reinterpret_cast<const int4*>(&kp[kbase]);
    int4 kb4 = make_int4(0, 0, 0, 0);
    if (BUCKETS) kb4 = *reinterpret_cast<const int4*>(&kbk[kbase]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qp = qpos[qb];
      f32x4 c;
      c[0] = bias_if_ge(qp, kp4.x);
      c[1] = bias_if_ge(qp, kp4.y);
      c[2] = bias_if_ge(qp, kp4.z);
      c[3] = bias_if_ge(qp, kp4.w);
      if (BUCKETS) {
        const int qh = qbkt[qb];
        c[0] = keep_if_eq(c[0], qh, kb4.x);
        c[1] = keep_if_eq(c[1], qh, kb4.y);
        c[2] = keep_if_eq(c[2], qh, kb4.z);
        c[3] = keep_if_eq(c[3], qh, kb4.w);
      }
      C[kb][qb] = c;
    }
  }
}

// The same bias for the 32 keys 32 kc .. 32 kc + 31 of the tile (blocks
// 2 kc and 2 kc + 1 as C[0], C[1]).
// buckets: also compare buckets (the tile's keys or the wave's queries span
// more than one bucket).
__device__ inline void mask_bias_half(f32x4 (&C)[2][2], bool buckets, const int32_t* kp, const int32_t* kbk,
                                      const int (&qpos)[2], const int (&qbkt)[2], int g, int kc) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int kbase = 32 * kc + 8 * g + 4 * h2;
    const int4 kp4 = *reinterpret_cast<const int4*>(&kp[kbase]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qp = qpos[qb];
      f32x4 c;
      c[0] = bias_if_ge(qp, kp4.x);
      c[1] = bias_if_ge(qp, kp4.y);
      c[2] = bias_if_ge(qp, kp4.z);
      c[3] = bias_if_ge(qp, kp4.w);
      if (buckets) {
        const int4 kb4 = *reinterpret_cast<const int4*>(&kbk[kbase]);
        const int qh = qbkt[qb];
        c[0] = keep_if_eq(c[0], qh, kb4.x);
        c[1] = keep_if_eq(c[1], qh, kb4.y);
        c[2] = keep_if_eq(c[2], qh, kb4.z);
        c[3] = keep_if_eq(c[3], qh, kb4.w);
      }
      C[h2][qb] = c;
    }
  }
}

// Tests of up to 64 consecutive tiles of a range, as wave-uniform bit masks
// (bit i: tile i of the window).
struct TileMasks {
  uint64_t pass;   // passes the workgroup's causal extremum test (hash ranges)
  uint64_t empty;  // holds no pair visible to the wave's rows
  uint64_t full;   // every pair visible to them: no mask
  uint64_t mixed;  // tile or wave rows span buckets: the mask compares buckets
};

// Walk over a range [beg, end) of tiles whose tests are kept as bit masks, 64
// tiles per window (window k: tiles beg + 64 k, ...). Lane i loads the
// statistics of tile i of a window, and `tests(stats, tile)` turns them into
// the window's masks (ballots; tiles at or past `end` must test false); `cw`
// holds the masks of the window of the current tile.
// SKIP: tiles failing `pass` are not visited, and a window is loaded when the
// walk reaches it (hash ranges are short). Otherwise every tile is visited
// and the statistics of the window after the current one are prefetched.
template <bool SKIP>
struct TileWalk {
  const int4* stats;
  int beg, end, lane;
  int cw_wb;
  int4 st0, nx_st;
  TileMasks cw;

  // Issues the loads of the first window (and of the second one).
  __device__ TileWalk(const int4* st, int b, int e, int l) : stats(st), beg(b), end(e), lane(l), cw_wb(b) {
    st0 = load(beg);
    if (!SKIP) nx_st = end - beg > 64 ? load(beg + 64) : make_int4(0, 0, 0, 0);
  }
  __device__ int4 load(int wb) const {
    int4 v = make_int4(0, 0, 0, 0);
    if (wb + lane < end) v = stats[wb + lane];
    return v;
  }
  // Masks of the first window (waits for its statistics).
  template <class Tests>
  __device__ void first(Tests&& tests) {
    cw = tests(st0, beg + lane);
  }
  // First tile at or after `from` (>= the current tile) to visit, or end.
  template <class Tests>
  __device__ int next(int from, Tests&& tests) {
    if (!SKIP) return min(from, end);
    if (from >= end) return end;
    const int o = from - cw_wb;
    if (o < 64) {
      const uint64_t m = cw.pass & (~0ull << o);
      if (m) return cw_wb + static_cast<int>(__builtin_ctzll(m));
      from = cw_wb + 64;
    }
    while (from < end) {  // later windows
      const int wb = beg + ((from - beg) & ~63);
      const uint64_t m = tests(load(wb), wb + lane).pass & (~0ull << (from - wb));
      if (m) return wb + static_cast<int>(__builtin_ctzll(m));
      from = wb + 64;
    }
    return end;
  }
  // Makes the window of tile j current.
  template <class Tests>
  __device__ void enter(int j, Tests&& tests) {
    if (j - cw_wb < 64) return;
    const int wb = beg + ((j - beg) & ~63);
    if (SKIP) {
      cw = tests(load(wb), wb + lane);
    } else {  // tiles are visited in turn: wb is the window after cw
      cw = tests(nx_st, wb + lane);
      if (wb + 64 < end) nx_st = load(wb + 64);
    }
    cw_wb = wb;
  }
  __device__ bool has(uint64_t m, int j) const { return (m >> (j - cw_wb)) & 1; }
};

// Tests of key tiles (statistics st of tile jj, range end jend) against a
// wave's query rows.
template <bool HASH>
__device__ inline TileMasks key_tile_masks(const int4& st, int jj, int jend, int qreach, const WaveRows& wr, int Tk) {
  const bool valid = jj < jend;
  TileMasks m;
  m.pass = __ballot(valid && (!HASH || st.x <= qreach));
  m.empty = __ballot(valid && tile_empty_for<HASH>(st, wr));
  m.full = __ballot(valid && tile_full_for<HASH>(st, wr, jj, Tk));
  m.mixed = HASH ? static_cast<uint64_t>(__ballot(valid && !(st.z == st.w && wr.minb == wr.maxb))) : 0ull;
  return m;
}

// Mask bias of a tile that is not fully visible: positions only when the
// tile's keys and the wave's real queries share one bucket (always so in QK
// mode and in the bucket-aligned layout), positions and buckets otherwise.
template <bool HASH>
__device__ inline void mask_bias(f32x4 (&C)[4][2], const int4& ks, const WaveRows& wr, const int32_t* kp,
                                 const int32_t* kbk, const int (&qpos)[2], const int (&qbkt)[2], int g) {
  if (!HASH || (ks.z == ks.w && wr.minb == wr.maxb))
    bias_tile<false>(C, kp, kbk, qpos, qbkt, g);
  else
    bias_tile<true>(C, kp, kbk, qpos, qbkt, g);
}

}  // namespace scfa
