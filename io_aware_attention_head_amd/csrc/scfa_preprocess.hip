// Index / bucket preprocessing and tile tables for sparse causal flash
// attention on gfx950.
//
// Operations (see the explainer "Faster Causal Attention Over Large Sequences
// Through Sparse Flash Attention", section 3.4):
//   * QK-drop compaction: per-head keep counts, exclusive prefix sums,
//     stable scatter of the kept rows to the front, sentinel padding.
//   * Hash-sparse: angular LSH bucket (argmax over [xR ; -xR]), stable
//     counting sort by bucket, gather into the sorted order.
//   * Tile extrema and the per-query-tile / per-key-tile range tables of
//     Algorithms 1 and 2 and of the backward pass.
// The LSH projection is bound by its float64 FMAs; the rest is HBM-bandwidth
// or latency bound: 16-byte coalesced accesses, wave64 ballots for the
// prefix sums, and no MFMA.

#include <limits.h>

#include <utility>

#include "scfa_internal.h"

namespace scfa {
namespace {

// ---------------------------------------------------------------------------
// QK-drop: counts per 64-position chunk, then an exclusive scan per head.
// ---------------------------------------------------------------------------

__device__ inline void qk_chunk_counts(const uint8_t* __restrict__ keep, int T, int H, int nC, int c, int b,
                                       int32_t* __restrict__ chunk, int32_t* __restrict__ max_count) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (c == 0 && b == 0 && threadIdx.x == 0) *max_count = 0;
  const int t = c * SCFA_COUNT_CHUNK + lane;
  for (int h = w; h < H; h += 4) {
    const bool f = t < T && keep[(static_cast<size_t>(b) * T + t) * H + h] != 0;
    const uint64_t m = __ballot(f);
    if (lane == 0) chunk[(static_cast<size_t>(b) * H + h) * nC + c] = __popcll(m);
  }
}

__global__ __launch_bounds__(256) void k_qk_chunk_counts(const uint8_t* __restrict__ keep, int T, int H, int nC,
                                                         int32_t* __restrict__ chunk, int32_t* __restrict__ max_count) {
  qk_chunk_counts(keep, T, H, nC, blockIdx.x, blockIdx.y, chunk, max_count);
}

__device__ inline void qk_scan(int32_t* __restrict__ chunk, int nC, int bh, int32_t* __restrict__ count,
                               int32_t* __restrict__ max_count) {
  __shared__ int32_t wsum[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t* p = chunk + static_cast<size_t>(bh) * nC;
  int carry = 0;
  for (int base = 0; base < nC; base += 256) {
    const int i = base + threadIdx.x;
    const int v = i < nC ? p[i] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int pre = 0;
    for (int k = 0; k < w; ++k) pre += wsum[k];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (i < nC) p[i] = carry + pre + x - v;
    carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    count[bh] = carry;
    atomicMax(max_count, carry);
  }
}

__global__ __launch_bounds__(256) void k_qk_scan(int32_t* __restrict__ chunk, int nC, int32_t* __restrict__ count,
                                                 int32_t* __restrict__ max_count) {
  qk_scan(chunk, nC, blockIdx.x, count, max_count);
}

// One workgroup per (64-position chunk, batch), all heads: the keep bytes and
// the input rows of the chunk are one contiguous block of memory.
template <int ESZ>
__device__ inline void qk_compact(const uint8_t* __restrict__ x, const uint8_t* __restrict__ keep,
                                  const int32_t* __restrict__ count, const int32_t* __restrict__ chunk_off, int T,
                                  int H, int D, int Tc, int nC, int c, int b, int32_t pad, uint8_t* __restrict__ xc,
                                  int32_t* __restrict__ idx, int32_t* dev_err) {
  extern __shared__ int32_t rank[];  // [H][64]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int h = w; h < H; h += 4) {
    const int bh = b * H + h;
    int r = -1;
    if (c < nC) {
      const int t = c * SCFA_COUNT_CHUNK + lane;
      const bool f = t < T && keep[(static_cast<size_t>(b) * T + t) * H + h] != 0;
      const uint64_t m = __ballot(f);
      if (f) {
        r = chunk_off[static_cast<size_t>(bh) * nC + c] + lanes_below(m);
        if (r < Tc) {
          idx[static_cast<size_t>(bh) * Tc + r] = t;
        } else {
          set_dev_err(dev_err, SCFA_DEVERR_COUNT_EXCEEDS_TC);
          r = -1;
        }
      }
    }
    rank[h * 64 + lane] = r;
    const int pr = count[bh] + c * SCFA_COUNT_CHUNK + lane;
    if (pr >= 0 && pr < Tc) idx[static_cast<size_t>(bh) * Tc + pr] = pad;
  }
  __syncthreads();
  if (xc == nullptr) return;
  const int U = D * ESZ / 16;  // 16-byte units per row
  if (c < nC) {
    const int npos = min(SCFA_COUNT_CHUNK, T - c * SCFA_COUNT_CHUNK);
    const int nunits = npos * H * U;
    const uint8_t* src0 = x + (static_cast<size_t>(b) * T + static_cast<size_t>(c) * SCFA_COUNT_CHUNK) * H * D * ESZ;
    for (int u = threadIdx.x; u < nunits; u += 256) {
      const int l = u / (H * U);
      const int rem = u - l * H * U;
      const int h = rem / U;
      const int kk = rem - h * U;
      const int r = rank[h * 64 + l];
      if (r >= 0) {
        const uint4 val = reinterpret_cast<const uint4*>(src0)[u];
        uint8_t* dst = xc + ((static_cast<size_t>(b) * H + h) * Tc + r) * D * ESZ;
        reinterpret_cast<uint4*>(dst)[kk] = val;
      }
    }
  }
  // zero the pad rows [count + 64c, count + 64c + 64) of every head
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int u = threadIdx.x; u < SCFA_COUNT_CHUNK * H * U; u += 256) {
    const int l = u / (H * U);
    const int rem = u - l * H * U;
    const int h = rem / U;
    const int kk = rem - h * U;
    const int bh = b * H + h;
    const int pr = count[bh] + c * SCFA_COUNT_CHUNK + l;
    if (pr >= 0 && pr < Tc) {
      uint8_t* dst = xc + (static_cast<size_t>(bh) * Tc + pr) * D * ESZ;
      reinterpret_cast<uint4*>(dst)[kk] = z;
    }
  }
}

template <int ESZ>
__global__ __launch_bounds__(256) void k_qk_compact(const uint8_t* __restrict__ x, const uint8_t* __restrict__ keep,
                                                    const int32_t* __restrict__ count,
                                                    const int32_t* __restrict__ chunk_off, int T, int H, int D, int Tc,
                                                    int nC, int32_t pad, uint8_t* __restrict__ xc,
                                                    int32_t* __restrict__ idx, int32_t* dev_err) {
  qk_compact<ESZ>(x, keep, count, chunk_off, T, H, D, Tc, nC, blockIdx.x, blockIdx.y, pad, xc, idx, dev_err);
}

// Queries and keys in two launches (grid dimension z selects the side; the
// grid covers the longer side, and the other side's extra workgroups return
// at once): the chunk counts, then the index arrays, whose workgroups sum
// the chunk counts before their own chunk themselves (no scan launch). The
// index arrays, counts and max counts equal those of the one-side calls.
struct QkSide {
  const uint8_t* keep;
  int T, nC, nCx, Tc;  // tokens, count chunks, compaction chunks (covering max(T, Tc)), compacted length
  int32_t pad;
  int32_t* chunk;  // per-chunk kept counts
  int32_t* count;
  int32_t* max_count;
  int32_t* idx;
  int32_t* stats;  // optional (B, H, Tc / bs, 4) tile statistics over all Tc rows
  int bs;          // rows per tile of stats
};

__global__ __launch_bounds__(256) void k_qk_chunk_counts_qk(QkSide s0, QkSide s1, int H) {
  const QkSide& s = blockIdx.z == 0 ? s0 : s1;
  if (static_cast<int>(blockIdx.x) >= s.nC) return;
  qk_chunk_counts(s.keep, s.T, H, s.nC, blockIdx.x, blockIdx.y, s.chunk, s.max_count);
}

__global__ __launch_bounds__(256) void k_qk_index_qk(QkSide s0, QkSide s1, int H, int32_t* dev_err,
                                                     int32_t* tiles) {
  const QkSide& s = blockIdx.z == 0 ? s0 : s1;
  const int c = blockIdx.x, b = blockIdx.y;
  if (c >= s.nCx) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int h = w; h < H; h += 4) {
    const int bh = b * H + h;
    // kept tokens before this chunk, and in the whole head
    const int32_t* cc = s.chunk + static_cast<size_t>(bh) * s.nC;
    int pre = 0, tot = 0;
    for (int i = lane; i < s.nC; i += 64) {
      const int v = cc[i];
      tot += v;
      pre += i < c ? v : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      pre += __shfl_xor(pre, o);
      tot += __shfl_xor(tot, o);
    }
    // Tile statistics of the compacted rows (min and max position over all
    // Tc rows of a tile, pads included; buckets 0), as k_tile_stats gives
    // them: real rows come first in ascending position, then the pads, so
    // the first row of a tile gives its minimum (the query pad -1 where the
    // tile holds a pad) and its last real row, or a pad, its maximum. Each
    // field has exactly one writer.
    int32_t* st = s.stats ? s.stats + static_cast<size_t>(bh) * (s.Tc / s.bs) * 4 : nullptr;
    const bool qside = s.pad == SCFA_Q_PAD;
    if (c < s.nC) {
      const int t = c * SCFA_COUNT_CHUNK + lane;
      const bool f = t < s.T && s.keep[(static_cast<size_t>(b) * s.T + t) * H + h] != 0;
      const uint64_t m = __ballot(f);
      if (f) {
        const int r = pre + lanes_below(m);
        if (r < s.Tc) {
          s.idx[static_cast<size_t>(bh) * s.Tc + r] = t;
          if (st) {
            const int i = r / s.bs;
            const bool has_pad = tot < (i + 1) * s.bs;
            if (r == i * s.bs) {  // first row: the minimum
              st[4 * i + 0] = (qside && has_pad) ? SCFA_Q_PAD : t;
              st[4 * i + 2] = 0;
              st[4 * i + 3] = 0;
            }
            if (r == min((i + 1) * s.bs, tot) - 1)  // last real row: the maximum
              st[4 * i + 1] = (!qside && has_pad) ? SCFA_K_PAD : t;
          }
        } else {
          set_dev_err(dev_err, SCFA_DEVERR_COUNT_EXCEEDS_TC);
        }
      }
    }
    const int pr = tot + c * SCFA_COUNT_CHUNK + lane;
    if (pr < s.Tc) {
      s.idx[static_cast<size_t>(bh) * s.Tc + pr] = s.pad;
      if (st && pr % s.bs == 0) {  // a tile of pads only
        const int i = pr / s.bs;
        st[4 * i + 0] = s.pad;
        st[4 * i + 1] = s.pad;
        st[4 * i + 2] = 0;
        st[4 * i + 3] = 0;
      }
    }
    if (c == 0 && lane == 0) {
      s.count[bh] = tot;
      atomicMax(s.max_count, tot);
      if (tiles && blockIdx.z == 0) tiles[bh] = 0;  // the processed-tile count the range table adds to
    }
  }
}

// ---------------------------------------------------------------------------
// LSH bucket. One workgroup per (256 tokens, head), one wave per 64 tokens.
// A wave first copies its 64 rows into LDS with coalesced 16-byte loads
// (consecutive lanes read consecutive 16 bytes of a row), then each lane
// accumulates its own token's projections. R of the head reaches the
// float64 FMA either from LDS as a wave-wide broadcast (k_hash_bucket) or,
// up to nb = 32, from registers by a DPP row broadcast (k_hash_bucket_dpp,
// which frees the kernel of the LDS reads that otherwise bound it). A
// product of a bf16/fp32 input and an fp32 rotation is exact in float64, so
// a fused multiply-add rounds exactly where a separate multiply and add
// would (only at the sum): the accumulation matches the sequential
// definition c_j = ((0 + x_0 R_0j) + x_1 R_1j) + ... bit for bit.
// ---------------------------------------------------------------------------

template <typename TIN>
__device__ inline float unit_elem(const u32x4& u, int e);

template <>
__device__ inline float unit_elem<float>(const u32x4& u, int e) {
  return __uint_as_float(u[e]);
}

template <>
__device__ inline float unit_elem<uint16_t>(const u32x4& u, int e) {
  const uint32_t w = u[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <typename TIN, int HALF>
__global__ __launch_bounds__(256) void k_hash_bucket(const TIN* x, const TIN* x2, const float* __restrict__ R,
                                                     int T, int H, int32_t* bucket, int32_t* bucket2, int32_t* counts,
                                                     int32_t* counts2, const uint8_t* keep, const uint8_t* keep2, int nbo,
                                                     int side0) {
  if (blockIdx.z) {  // second side of a two-input launch
    x = x2;
    bucket = bucket2;
    counts = counts2;
    keep = keep2;
  }
  constexpr int D = 64;
  constexpr int EPU = 16 / sizeof(TIN);  // elements per 16-byte unit
  constexpr int NU = D / EPU;            // units per row (8 bf16, 16 fp32)
  constexpr int RPI = 64 / NU;           // rows per wave-wide load
  constexpr int LDW = NU * 4 + 4;        // LDS row stride in 32-bit words (+16 bytes)
  __shared__ double Rs[D * HALF];
  __shared__ __align__(16) uint32_t xs[4][64 * LDW];
  __shared__ int32_t hs[2 * HALF + 2];  // nbo <= 2 HALF + 2 counted buckets  // bucket counts of this workgroup's 256 tokens
  const int bh = blockIdx.y;
  if (counts && threadIdx.x < nbo) hs[threadIdx.x] = 0;
  const int b = bh / H, h = bh - b * H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < D * HALF; i += 256) Rs[i] = static_cast<double>(R[static_cast<size_t>(h) * D * HALF + i]);
  const int tw = blockIdx.x * 256 + w * 64;  // first token of this wave
#pragma unroll
  for (int k = 0; k < 64 / RPI; ++k) {
    const int row = k * RPI + lane / NU, unit = lane % NU;
    const int t = min(tw + row, T - 1);
    const u32x4 v = reinterpret_cast<const u32x4*>(x + ((static_cast<size_t>(b) * T + t) * H + h) * D)[unit];
    *reinterpret_cast<u32x4*>(&xs[w][row * LDW + unit * 4]) = v;
  }
  __syncthreads();
  double c[HALF];
#pragma unroll
  for (int j = 0; j < HALF; ++j) c[j] = 0.0;
#pragma unroll 2
  for (int i = 0; i < NU; ++i) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(&xs[w][lane * LDW + i * 4]);
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      const int d = i * EPU + e;
      const double xd = static_cast<double>(unit_elem<TIN>(u, e));
#pragma unroll
      for (int j = 0; j < HALF; ++j) c[j] = fma(xd, Rs[d * HALF + j], c[j]);
    }
  }
  const int t = tw + lane;
  // argmax over [c ; -c], first index on ties: the positive half comes first.
  int bp = 0, bn = 0;
  double vp = c[0], vn = -c[0];
#pragma unroll
  for (int j = 1; j < HALF; ++j) {
    if (c[j] > vp) { vp = c[j]; bp = j; }
    if (-c[j] > vn) { vn = -c[j]; bn = j; }
  }
  int v = (vn > vp) ? HALF + bn : bp;
  // a dropped token (hashing with within-bucket dropping) takes a bucket of
  // its own side (side0 + blockIdx.z: 0 queries, 1 keys) that matches
  // nothing: nb for queries, nb + 1 for keys
  if (keep && t < T && keep[(static_cast<size_t>(b) * T + t) * H + h] == 0) v = 2 * HALF + side0 + blockIdx.z;
  if (t < T) bucket[static_cast<size_t>(bh) * T + t] = v;
  if (counts) {  // the chunk histogram of the stable sort (chunk = this workgroup)
    if (t < T) atomicAdd(&hs[v], 1);
    __syncthreads();
    if (threadIdx.x < nbo)
      counts[(static_cast<size_t>(bh) * gridDim.x + blockIdx.x) * nbo + threadIdx.x] = hs[threadIdx.x];
  }
}

// acc += (lane K of this lane's 16-lane row of r) * x, in float64, with the
// operand broadcast by DPP inside the FMA (row_newbcast).
template <int K>
__device__ __forceinline__ void fma_row_bcast(double& acc, double r, double x) {
  asm("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(r), "v"(x), "n"(K));
}

template <int HALF, int Q>
__device__ __forceinline__ void fma_rq(double& acc, const double* Rv, double x) {
  fma_row_bcast<Q % 16>(acc, Rv[Q / 16], x);
}

template <int HALF, int D0, int... J>
__device__ __forceinline__ void fma_row_d(double* c, const double* Rv, double x, std::integer_sequence<int, J...>) {
  (fma_rq<HALF, D0 * HALF + J>(c[J], Rv, x), ...);
}

template <typename TIN, int HALF, int I, int... E>
__device__ __forceinline__ void fma_unit(double* c, const double* Rv, const u32x4 u, std::integer_sequence<int, E...>) {
  constexpr int EPU = 16 / sizeof(TIN);
  (fma_row_d<HALF, I * EPU + E>(c, Rv, static_cast<double>(unit_elem<TIN>(u, E)),
                                std::make_integer_sequence<int, HALF>{}),
   ...);
}

template <typename TIN, int HALF, int... I>
__device__ __forceinline__ void fma_units(double* c, const double* Rv, const uint32_t* xr,
                                          std::integer_sequence<int, I...>) {
  constexpr int EPU = 16 / sizeof(TIN);
  (fma_unit<TIN, HALF, I>(c, Rv, *reinterpret_cast<const u32x4*>(xr + I * 4), std::make_integer_sequence<int, EPU>{}),
   ...);
}

// Same projection and argmax as k_hash_bucket, with the rotation held in
// registers: flat entry q = d * HALF + j of the head's R sits in register
// pair q / 16 of lane q % 16 of every 16-lane row, and reaches the FMA by a
// row broadcast, so the inner loop is FMAs only. The accumulation order
// (d = 0, 1, ..., 63 for each j, one rounding per FMA) is the same.
template <typename TIN, int HALF>
__global__ __launch_bounds__(256) void k_hash_bucket_dpp(const TIN* x, const TIN* x2, const float* __restrict__ R,
                                                         int T, int H, int32_t* bucket, int32_t* bucket2, int32_t* counts,
                                                         int32_t* counts2, const uint8_t* keep, const uint8_t* keep2, int nbo,
                                                     int side0) {
  if (blockIdx.z) {  // second side of a two-input launch
    x = x2;
    bucket = bucket2;
    counts = counts2;
    keep = keep2;
  }
  constexpr int D = 64;
  constexpr int EPU = 16 / sizeof(TIN);
  constexpr int NU = D / EPU;
  constexpr int RPI = 64 / NU;
  constexpr int LDW = NU * 4 + 4;
  constexpr int NR = D * HALF / 16;  // register pairs holding R
  __shared__ __align__(16) uint32_t xs[4][64 * LDW];
  __shared__ int32_t hs[2 * HALF + 2];  // nbo <= 2 HALF + 2 counted buckets
  const int bh = blockIdx.y;
  if (counts && threadIdx.x < nbo) hs[threadIdx.x] = 0;
  const int b = bh / H, h = bh - b * H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* Rh = R + static_cast<size_t>(h) * D * HALF;
  double Rv[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) Rv[q] = static_cast<double>(Rh[16 * q + (lane & 15)]);
  const int tw = blockIdx.x * 256 + w * 64;
#pragma unroll
  for (int k = 0; k < 64 / RPI; ++k) {
    const int row = k * RPI + lane / NU, unit = lane % NU;
    const int t = min(tw + row, T - 1);
    const u32x4 v = reinterpret_cast<const u32x4*>(x + ((static_cast<size_t>(b) * T + t) * H + h) * D)[unit];
    *reinterpret_cast<u32x4*>(&xs[w][row * LDW + unit * 4]) = v;
  }
  // A DPP source must be written at least two wait states before it is
  // read; the asm (one per register pair) keeps the writes above the barrier.
#pragma unroll
  for (int q = 0; q < NR; ++q) asm volatile("s_nop 1" : "+v"(Rv[q]));
  __syncthreads();
  double c[HALF];
#pragma unroll
  for (int j = 0; j < HALF; ++j) c[j] = 0.0;
  const uint32_t* xr = &xs[w][lane * LDW];
  fma_units<TIN, HALF>(c, Rv, xr, std::make_integer_sequence<int, NU>{});
  const int t = tw + lane;
  int bp = 0, bn = 0;
  double vp = c[0], vn = -c[0];
#pragma unroll
  for (int j = 1; j < HALF; ++j) {
    if (c[j] > vp) { vp = c[j]; bp = j; }
    if (-c[j] > vn) { vn = -c[j]; bn = j; }
  }
  int v = (vn > vp) ? HALF + bn : bp;
  // a dropped token (hashing with within-bucket dropping) takes a bucket of
  // its own side (side0 + blockIdx.z: 0 queries, 1 keys) that matches
  // nothing: nb for queries, nb + 1 for keys
  if (keep && t < T && keep[(static_cast<size_t>(b) * T + t) * H + h] == 0) v = 2 * HALF + side0 + blockIdx.z;
  if (t < T) bucket[static_cast<size_t>(bh) * T + t] = v;
  if (counts) {
    if (t < T) atomicAdd(&hs[v], 1);
    __syncthreads();
    if (threadIdx.x < nbo)
      counts[(static_cast<size_t>(bh) * gridDim.x + blockIdx.x) * nbo + threadIdx.x] = hs[threadIdx.x];
  }
}

// Register-held rotation up to nb = 32 (at most 128 VGPRs of R); the LDS
// broadcast kernel above it.
template <typename TIN, int HALF>
void bucket_launch(dim3 grid, hipStream_t stream, const void* x, const void* x2, const float* R, int T, int H,
                   int32_t* bucket, int32_t* bucket2, int32_t* counts, int32_t* counts2, const uint8_t* keep,
                   const uint8_t* keep2, int side0) {
  const TIN* a = static_cast<const TIN*>(x);
  const TIN* a2 = static_cast<const TIN*>(x2);
  const int nbo = 2 * HALF + (keep ? 2 : 0);
  if constexpr (HALF <= 16)
    hipLaunchKernelGGL((k_hash_bucket_dpp<TIN, HALF>), grid, dim3(256), 0, stream, a, a2, R, T, H, bucket, bucket2,
                       counts, counts2, keep, keep2, nbo, side0);
  else
    hipLaunchKernelGGL((k_hash_bucket<TIN, HALF>), grid, dim3(256), 0, stream, a, a2, R, T, H, bucket, bucket2,
                       counts, counts2, keep, keep2, nbo, side0);
}

// ---------------------------------------------------------------------------
// Stable counting sort by bucket: per-chunk histograms, then a scatter whose
// workgroups each derive their own base from all chunk histograms of the
// head (4 KB of L2 reads at nb = 16, 64 chunks, all loads in flight at once
// and summed by LDS atomics) and whose in-chunk ranks come from wave64
// ballots.
// ---------------------------------------------------------------------------

constexpr int kSortChunk = 256;
constexpr int kMaxOrderSpan = 16383;  // length bins of k_work_order fit in 64 KB of LDS
constexpr size_t kTableOrderLds = 60 * 1024;  // dynamic LDS of k_fwd_table_order (within the default 64 KB)

__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ bucket, int T, int nb, int nC,
                                                   int32_t* __restrict__ hist, int32_t* dev_err) {
  __shared__ int32_t hs[64];
  const int c = blockIdx.x, bh = blockIdx.y;
  if (threadIdx.x < 64) hs[threadIdx.x] = 0;
  __syncthreads();
  const int t = c * kSortChunk + threadIdx.x;
  if (t < T) {
    const int v = bucket[static_cast<size_t>(bh) * T + t];
    if (v >= 0 && v < nb) {
      atomicAdd(&hs[v], 1);
    } else {
      set_dev_err(dev_err, SCFA_DEVERR_BUCKET_RANGE);
    }
  }
  __syncthreads();
  if (threadIdx.x < nb) hist[(static_cast<size_t>(bh) * nC + c) * nb + threadIdx.x] = hs[threadIdx.x];
}

// One side (queries or keys) of a sort / layout launch.
struct SortSide {
  const int32_t* bucket;  // (B, H, T)
  const int32_t* hist;    // (B, H, nC, nb) chunk counts
  int32_t pad;            // index of pad entries
  int align;              // 0: sort only; else rows per bucket run multiple
  int Tseg;               // rows per head of the aligned layout
  int32_t* perm;
  int32_t* bsorted;
  int32_t* offsets;
  int32_t* idx_seg;
  int32_t* bkt_seg;
  int32_t* seg_off;
  int32_t* stats;  // optional: (B, H, Tseg / align, 4) statistics of the aligned layout's tiles
  int32_t* tiles;  // optional: (B*H) processed-tile counters, zeroed here
};

// Workgroup (chunk c, head bh, side z: s0 or s1). base[v] = (tokens of the
// head with bucket < v) + (tokens of bucket v in chunks before c); the
// chunk-0 workgroup also writes offsets. With align > 0 the same workgroup
// also places its tokens in the bucket-aligned layout (bucket v's rows start
// at A_v) and writes the pad rows of that layout that fall in rows
// [256 c, 256 c + 256). Chunks at or beyond nC only write pad entries.
__global__ __launch_bounds__(256) void k_sort_scatter(const SortSide s0, const SortSide s1, int T, int Tp, int nb,
                                                      int nC, int32_t* dev_err) {
  const SortSide& sd = blockIdx.z ? s1 : s0;
  const int32_t* __restrict__ bucket = sd.bucket;
  const int32_t* __restrict__ hist = sd.hist;
  const int32_t pad = sd.pad;
  const int align = sd.align, Tseg = sd.Tseg;
  int32_t* __restrict__ perm = sd.perm;
  int32_t* __restrict__ bsorted = sd.bsorted;
  int32_t* __restrict__ offsets = sd.offsets;
  int32_t* __restrict__ idx_seg = sd.idx_seg;
  int32_t* __restrict__ bkt_seg = sd.bkt_seg;
  int32_t* __restrict__ seg_off = sd.seg_off;
  int32_t* __restrict__ stats = align > 0 ? sd.stats : nullptr;
  __shared__ int32_t tot_a[64], bef_a[64];
  __shared__ int32_t base_s[64];
  __shared__ int32_t wcnt[4][64];
  __shared__ int32_t tot_s[64], off_s[65], aoff_s[65];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t* pp = perm + static_cast<size_t>(bh) * Tp;
  int32_t* bp = bsorted + static_cast<size_t>(bh) * Tp;
  const int t = c * kSortChunk + threadIdx.x;
  int v = -1;
  if (c < nC && t < T) v = bucket[static_cast<size_t>(bh) * T + t];
  if (w == 0) {
    tot_a[lane] = 0;
    bef_a[lane] = 0;
  }
  wcnt[w][lane] = 0;
  __syncthreads();
  // per-bucket totals and counts before this chunk: entry e = cc nb + v of the
  // head's chunk histograms, 4 independent loads per thread in flight
  {
    const int nE = nC * nb, eb = c * nb;
    const int32_t* hp = hist + static_cast<size_t>(bh) * nE;
    for (int e0 = 0; e0 < nE; e0 += 1024) {
      int n[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = e0 + k * 256 + threadIdx.x;
        n[k] = e < nE ? hp[e] : 0;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = e0 + k * 256 + threadIdx.x;
        if (n[k] != 0) {
          const int bv = e % nb;
          atomicAdd(&tot_a[bv], n[k]);
          if (e < eb) atomicAdd(&bef_a[bv], n[k]);
        }
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    const int tot = lane < nb ? tot_a[lane] : 0;
    const int bef = lane < nb ? bef_a[lane] : 0;
    int x = tot;  // inclusive scan over buckets
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    const int off = x - tot;
    base_s[lane] = off + bef;
    tot_s[lane] = tot;
    off_s[lane] = off;
    if (lane == 63) off_s[64] = x;
    if (c == 0) {
      if (lane < nb) offsets[static_cast<size_t>(bh) * (nb + 1) + lane] = off;
      if (lane == 63) offsets[static_cast<size_t>(bh) * (nb + 1) + nb] = x;  // all tokens
      if (lane == 0 && sd.tiles) sd.tiles[bh] = 0;
    }
    if (align > 0) {
      const int a = ((tot + align - 1) / align) * align;  // aligned rows of bucket `lane`
      int y = a;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int z = __shfl_up(y, o);
        if (lane >= o) y += z;
      }
      aoff_s[lane] = y - a;
      if (lane == 63) aoff_s[64] = y;
      if (c == 0) {
        int32_t* so = seg_off + static_cast<size_t>(bh) * (nb + 1);
        if (lane < nb) so[lane] = y - a;
        if (lane == nb - 1) {
          so[nb] = y;
          if (y > Tseg) set_dev_err(dev_err, SCFA_DEVERR_SEGMENT_OVERFLOW);
        }
      }
    }
  }
  int32_t* ip = align > 0 ? idx_seg + static_cast<size_t>(bh) * Tseg : nullptr;
  int32_t* kp = align > 0 ? bkt_seg + static_cast<size_t>(bh) * Tseg : nullptr;
  const bool valid = c < nC && t < T && v >= 0 && v < nb;
  if (c < nC && t < T && !valid) set_dev_err(dev_err, SCFA_DEVERR_BUCKET_RANGE);
  int my_rank = 0;
  uint64_t remaining = __ballot(valid);
  while (remaining) {
    const int leader = __ffsll(static_cast<long long>(remaining)) - 1;
    const int lv = __shfl(v, leader);
    const bool mine = valid && v == lv;
    const uint64_t m = __ballot(mine);
    if (mine) my_rank = lanes_below(m);
    if (lane == 0) wcnt[w][lv] = __popcll(m);
    remaining &= ~m;
  }
  __syncthreads();
  if (valid) {
    int pos = base_s[v] + my_rank;
    for (int k = 0; k < w; ++k) pos += wcnt[k][v];
    pp[pos] = t;
    bp[pos] = v;
    if (align > 0) {
      const int r = aoff_s[v] + (pos - off_s[v]);
      if (r < Tseg) {
        ip[r] = t;
        kp[r] = v;
        if (stats) {
          // Tile statistics [min pos, max pos, min bucket, max bucket]: the
          // tile's rows are one bucket's tokens in ascending position, then
          // pad rows (pad sorts below every position for queries, above for
          // keys). The tile's first row writes the minimum and the bucket,
          // its last real row the maximum.
          const int r0 = r - r % align;
          const int run_end = aoff_s[v] + tot_s[v];  // first row after bucket v's tokens
          const bool has_pad = r0 + align > run_end;
          int32_t* st = stats + (static_cast<size_t>(bh) * (Tseg / align) + r / align) * 4;
          if (r == r0) {
            st[0] = has_pad ? min(t, pad) : t;
            st[2] = v;
            st[3] = v;
          }
          if (r == min(r0 + align, run_end) - 1) st[1] = has_pad ? max(t, pad) : t;
        }
      }
    }
  }
  if (t >= T && t < Tp) {
    pp[t] = pad;
    bp[t] = -1;
  }
  if (align > 0 && t < Tseg) {  // pad rows of the aligned layout among rows [256 c, 256 c + 256)
    int a = 0, z = nb;          // the last bucket v in [0, nb] with A_v <= t
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (aoff_s[mid] <= t) a = mid; else z = mid - 1;
    }
    if (a == nb || t - aoff_s[a] >= tot_s[a]) {
      ip[t] = pad;
      kp[t] = a;
      if (stats && a == nb && t % align == 0)  // a tile after the last bucket: pad rows only
        *reinterpret_cast<int4*>(stats + (static_cast<size_t>(bh) * (Tseg / align) + t / align) * 4) =
            make_int4(pad, pad, nb, nb);
    }
  }
}

// ---------------------------------------------------------------------------
// Bucket-aligned layout of a sorted head: bucket v starts at row
// A_v = sum_{u<v} ceil(n_u / align) * align; its rows keep the sorted order,
// the rest of its segment holds pad rows (bucket v), rows from A_nb on hold
// pads with bucket nb. One thread per output row; wave 0 of each workgroup
// derives A from the bucket offsets.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hash_segments(const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offsets, int Tp, int nb, int align,
                                                       int32_t pad, int Tseg, int32_t* __restrict__ idx_seg,
                                                       int32_t* __restrict__ bkt_seg, int32_t* __restrict__ seg_off,
                                                       int32_t* dev_err) {
  __shared__ int32_t off_s[65], aoff_s[65];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {  // lane v < nb: bucket v (nb <= 64)
    const int32_t* op = offsets + static_cast<size_t>(bh) * (nb + 1);
    const int lo = lane < nb ? op[lane] : 0;
    const int hi = lane < nb ? op[lane + 1] : lo;
    const int m = ((hi - lo + align - 1) / align) * align;  // aligned rows of bucket `lane`
    int x = m;  // inclusive scan over buckets
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int32_t* so = seg_off + static_cast<size_t>(bh) * (nb + 1);
    if (lane < nb) {
      off_s[lane] = lo;
      aoff_s[lane] = x - m;
      if (blockIdx.x == 0) so[lane] = x - m;
    }
    if (lane == nb - 1) {  // end of the last bucket
      off_s[nb] = hi;
      aoff_s[nb] = x;
      if (blockIdx.x == 0) so[nb] = x;
      if (x > Tseg) set_dev_err(dev_err, SCFA_DEVERR_SEGMENT_OVERFLOW);
    }
  }
  __syncthreads();
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= Tseg) return;
  // bucket of row r: the last v with A_v <= r (empty buckets share a start)
  int a = 0, z = nb;  // search v in [0, nb]
  while (a < z) {
    const int mid = (a + z + 1) >> 1;
    if (aoff_s[mid] <= r) a = mid; else z = mid - 1;
  }
  int idx = pad, bkt = a;
  if (a < nb) {
    const int k = r - aoff_s[a];
    if (k < off_s[a + 1] - off_s[a]) idx = perm[static_cast<size_t>(bh) * Tp + off_s[a] + k];
  }
  idx_seg[static_cast<size_t>(bh) * Tseg + r] = idx;
  bkt_seg[static_cast<size_t>(bh) * Tseg + r] = bkt;
}

// ---------------------------------------------------------------------------
// Gather into head-major order (rows or transposed columns).
// ---------------------------------------------------------------------------

template <int ESZ>
__global__ __launch_bounds__(256) void k_gather_rows(const uint8_t* __restrict__ x, const int32_t* __restrict__ idx,
                                                     int T, int H, int D, int Tp, uint8_t* __restrict__ out) {
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int U = D * ESZ / 16;
  const long long u = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (u >= static_cast<long long>(Tp) * U) return;
  const int r = static_cast<int>(u / U);
  const int kk = static_cast<int>(u - static_cast<long long>(r) * U);
  const int src = idx[static_cast<size_t>(bh) * Tp + r];
  uint4 val = make_uint4(0, 0, 0, 0);
  if (src >= 0 && src < T)
    val = reinterpret_cast<const uint4*>(x + ((static_cast<size_t>(b) * T + src) * H + h) * D * ESZ)[kk];
  reinterpret_cast<uint4*>(out + (static_cast<size_t>(bh) * Tp + r) * D * ESZ)[kk] = val;
}

// 64 rows per workgroup: read with 16-byte loads into an LDS tile, then
// written as D rows of 64 consecutive columns (16-byte stores).
template <typename E>
__global__ __launch_bounds__(256) void k_gather_cols(const E* __restrict__ x, const int32_t* __restrict__ idx, int T,
                                                     int H, int Tp, E* __restrict__ out) {
  constexpr int D = 64;
  constexpr int EPU = 16 / sizeof(E);  // elements per 16-byte unit
  constexpr int UPR = D / EPU;         // units per input row
  constexpr int LD = D + EPU;          // LDS row stride: 16-byte aligned, rows shifted by 4 banks
  __shared__ __align__(16) E tile[64 * LD];
  __shared__ int32_t src_s[64];
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int r0 = blockIdx.x * 64;
  if (threadIdx.x < 64) src_s[threadIdx.x] = idx[static_cast<size_t>(bh) * Tp + r0 + threadIdx.x];
  __syncthreads();
  for (int u = threadIdx.x; u < 64 * UPR; u += 256) {
    const int rr = u / UPR, k = u - rr * UPR;
    const int src = src_s[rr];
    u32x4 val = {0u, 0u, 0u, 0u};
    if (src >= 0 && src < T)
      val = *reinterpret_cast<const u32x4*>(x + ((static_cast<size_t>(b) * T + src) * H + h) * D + k * EPU);
    *reinterpret_cast<u32x4*>(&tile[rr * LD + k * EPU]) = val;
  }
  __syncthreads();
  constexpr int UPO = 64 / EPU;  // units per output row (64 columns)
  for (int u = threadIdx.x; u < D * UPO; u += 256) {
    const int d = u / UPO, k = u - d * UPO;
    u32x4 val;
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = tile[(k * 8 + 2 * e) * LD + d], hi = tile[(k * 8 + 2 * e + 1) * LD + d];
        val[e] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = __float_as_uint(tile[(k * 4 + e) * LD + d]);
    }
    *reinterpret_cast<u32x4*>(out + (static_cast<size_t>(bh) * D + d) * Tp + r0 + k * EPU) = val;
  }
}

// ---------------------------------------------------------------------------
// Tile extrema and range tables.
// ---------------------------------------------------------------------------

// [min pos, max pos, min bucket, max bucket] of rows [r0, r1) (one wave; all
// lanes return it). An empty row range gives the sentinel statistics.
__device__ inline int4 tile_stats_wave(int mode, const int32_t* ip, const int32_t* bp, int r0, int r1, bool isq,
                                       int lane) {
  int mn = kInt32Max, mx = kInt32Min, mnb = kInt32Max, mxb = kInt32Min;
  for (int r = r0 + lane; r < r1; r += 64) {
    const int p = (mode == SCFA_DENSE) ? r : ip[r];
    mn = min(mn, p);
    mx = max(mx, p);
    if (bp) {
      const int v = bp[r];
      mnb = min(mnb, v);
      mxb = max(mxb, v);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
    mnb = min(mnb, __shfl_xor(mnb, o));
    mxb = max(mxb, __shfl_xor(mxb, o));
  }
  if (r1 <= r0)
    return isq ? make_int4(SCFA_Q_PAD, SCFA_Q_PAD, kInt32Max, kInt32Min)
               : make_int4(SCFA_K_PAD, SCFA_K_PAD, kInt32Max, kInt32Max);
  return bp ? make_int4(mn, mx, mnb, mxb) : make_int4(mn, mx, 0, 0);
}

__global__ __launch_bounds__(64) void k_tile_stats(int mode, const int32_t* __restrict__ q_idx,
                                                   const int32_t* __restrict__ k_idx, const int32_t* __restrict__ q_bkt,
                                                   const int32_t* __restrict__ k_bkt, int Tq, int Tk, int TqP, int TkP,
                                                   int Bm, int Bn, int nQt, int nKt, int32_t* __restrict__ qstats,
                                                   int32_t* __restrict__ kstats, int32_t* __restrict__ tiles) {
  const int bh = blockIdx.y;
  const int x = blockIdx.x;
  const int lane = threadIdx.x;
  const bool isq = x < nQt;
  const int tile = isq ? x : x - nQt;
  const int bs = isq ? Bm : Bn;
  const int Tv = isq ? Tq : Tk;
  const int32_t* ip = isq ? q_idx + static_cast<size_t>(bh) * TqP : k_idx + static_cast<size_t>(bh) * TkP;
  const int32_t* bp = nullptr;
  if (mode == SCFA_HASH) bp = isq ? q_bkt + static_cast<size_t>(bh) * TqP : k_bkt + static_cast<size_t>(bh) * TkP;
  const int4 s = tile_stats_wave(mode, ip, bp, tile * bs, min(tile * bs + bs, Tv), isq, lane);
  if (lane == 0) {
    int32_t* out = isq ? qstats + (static_cast<size_t>(bh) * nQt + tile) * 4 : kstats + (static_cast<size_t>(bh) * nKt + tile) * 4;
    *reinterpret_cast<int4*>(out) = s;
    if (x == 0) tiles[bh] = 0;
  }
}

// One wave per query tile; lane l holds key tiles l, l+64, ... in registers
// (all loads issued up front), the scans are wave ballots.
// QK / dense (Algorithm 1): end = number of key tiles whose smallest
// position is <= the query tile's largest position (a prefix, since key
// positions ascend). Hash (Algorithm 2): start = key tiles whose largest
// bucket is below the query tile's smallest bucket; provisional stop = first
// tile at/after start whose smallest bucket exceeds the query tile's largest;
// end = one past the last tile in [start, stop) passing the causal test.
constexpr int kTabRegChunks = 8;  // register path for up to 512 tiles

// One query tile's range [start, end) and processed-tile count (one wave).
// ks: the head's key-tile statistics (global memory or LDS).
__device__ void fwd_table_row(int mode, const int4 qs, const int4* ks, int nKt, int2* __restrict__ fwd_row, int lane,
                              int32_t& cnt_out, const Reach rc) {
  const int nch = (nKt + 63) / 64;
  const int qreach = q_reach(rc, qs.y);  // largest key position a query of the tile may see
  // per chunk: a = tile below the query buckets, e = tile above them, c = causal test passes
  uint64_t A[kTabRegChunks], E[kTabRegChunks], C[kTabRegChunks];
  auto chunk_masks = [&](int ch, uint64_t& a, uint64_t& e, uint64_t& c) {
    const int j = ch * 64 + lane;
    int4 k = make_int4(kInt32Max, kInt32Max, kInt32Max, kInt32Max);
    if (j < nKt) k = ks[j];
    a = __ballot(j < nKt && k.w < qs.z);
    e = __ballot(j < nKt && k.z > qs.w);
    c = __ballot(j < nKt && k.x <= qreach);
  };
  int start = 0, end = 0, cnt = 0;
  if (nch <= kTabRegChunks) {
#pragma unroll
    for (int ch = 0; ch < kTabRegChunks; ++ch)
      if (ch < nch) chunk_masks(ch, A[ch], E[ch], C[ch]);
    if (mode != SCFA_HASH) {
#pragma unroll
      for (int ch = 0; ch < kTabRegChunks; ++ch)
        if (ch < nch) cnt += __popcll(C[ch]);
      end = cnt;
    } else {
#pragma unroll
      for (int ch = 0; ch < kTabRegChunks; ++ch)
        if (ch < nch) start += __popcll(A[ch]);
      // bits of the tiles j >= start / j < stop within chunk ch
      auto from = [](int s, int j0) {
        return s <= j0 ? ~0ull : (s >= j0 + 64 ? 0ull : (~0ull << (s - j0)));
      };
      int eh = nKt;
#pragma unroll
      for (int ch = 0; ch < kTabRegChunks; ++ch) {
        const uint64_t m = E[ch] & from(start, ch * 64);
        if (ch < nch && eh == nKt && m) eh = ch * 64 + __ffsll(static_cast<long long>(m)) - 1;
      }
      end = start;
#pragma unroll
      for (int ch = 0; ch < kTabRegChunks; ++ch) {
        if (ch < nch) {
          const int j0 = ch * 64;
          // tiles j in [start, eh) of this chunk
          const uint64_t m = C[ch] & from(start, j0) & ~from(eh, j0);
          if (m) {
            end = j0 + 64 - __clzll(static_cast<long long>(m));
            cnt += __popcll(m);
          }
        }
      }
    }
  } else {
    // long sequences: the same scans, one chunk of 64 tiles at a time
    for (int ch = 0; ch < nch; ++ch) {
      uint64_t a, e, c;
      chunk_masks(ch, a, e, c);
      start += __popcll(a);
      if (mode != SCFA_HASH) cnt += __popcll(c);
    }
    if (mode != SCFA_HASH) {
      start = 0;
      end = cnt;
    } else {
      int eh = nKt;
      for (int j0 = start & ~63; j0 < nKt; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t m = __ballot(j >= start && j < nKt && ks[j].z > qs.w);
        if (m) {
          eh = j0 + __ffsll(static_cast<long long>(m)) - 1;
          break;
        }
      }
      end = start;
      for (int j0 = start & ~63; j0 < eh; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t m = __ballot(j >= start && j < eh && ks[j].x <= qreach);
        if (m) {
          end = j0 + 64 - __clzll(static_cast<long long>(m));
          cnt += __popcll(m);
        }
      }
    }
  }
  if (lane == 0) {
    *fwd_row = make_int2(start, end);
    cnt_out = cnt;
  }
}

// 16 waves per workgroup; their processed-tile counts are summed in LDS and
// added to the head's total with one atomic per workgroup.
constexpr int kTabWaves = 16;

__global__ __launch_bounds__(64 * kTabWaves) void k_fwd_table(int mode, const int32_t* __restrict__ qstats,
                                                              const int32_t* __restrict__ kstats, int nQt, int nKt,
                                                              int32_t* __restrict__ fwd, int32_t* __restrict__ tiles,
                                                              const Reach rc) {
  __shared__ int32_t wcnt[kTabWaves];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * kTabWaves + w;
  if (lane == 0) wcnt[w] = 0;
  if (i < nQt)
    fwd_table_row(mode, reinterpret_cast<const int4*>(qstats)[static_cast<size_t>(bh) * nQt + i],
                  reinterpret_cast<const int4*>(kstats) + static_cast<size_t>(bh) * nKt, nKt,
                  reinterpret_cast<int2*>(fwd) + static_cast<size_t>(bh) * nQt + i, lane, wcnt[w], rc);
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kTabWaves; ++k) sum += wcnt[k];
    if (sum) atomicAdd(&tiles[bh], sum);
  }
}

// One wave per key tile: first and last query tile that processes it. Lane l
// holds query tiles l, l+64, ... (loads issued up front).
__global__ __launch_bounds__(256) void k_bwd_table(const int32_t* __restrict__ qstats, const int32_t* __restrict__ kstats,
                                                   const int32_t* __restrict__ fwd, int nQt, int nKt,
                                                   int32_t* __restrict__ bwd, const Reach rc) {
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= nKt) return;
  // smallest query position that sees a key of the tile
  const int kreach = k_reach(rc, reinterpret_cast<const int4*>(kstats)[static_cast<size_t>(bh) * nKt + j].x);
  const int4* qs = reinterpret_cast<const int4*>(qstats) + static_cast<size_t>(bh) * nQt;
  const int2* ft = reinterpret_cast<const int2*>(fwd) + static_cast<size_t>(bh) * nQt;
  const int nch = (nQt + 63) / 64;
  auto hit_mask = [&](int ch) {
    const int i = ch * 64 + lane;
    bool hit = false;
    if (i < nQt) {
      const int2 r = ft[i];
      hit = j >= r.x && j < r.y && kreach <= qs[i].y;
    }
    return __ballot(hit);
  };
  int first = -1, last = -1;
  auto take = [&](int ch, uint64_t m) {
    if (m) {
      if (first < 0) first = ch * 64 + __ffsll(static_cast<long long>(m)) - 1;
      last = ch * 64 + 63 - __clzll(static_cast<long long>(m));
    }
  };
  if (nch <= kTabRegChunks) {
    uint64_t M[kTabRegChunks];
#pragma unroll
    for (int ch = 0; ch < kTabRegChunks; ++ch)
      if (ch < nch) M[ch] = hit_mask(ch);
#pragma unroll
    for (int ch = 0; ch < kTabRegChunks; ++ch)
      if (ch < nch) take(ch, M[ch]);
  } else {
    for (int ch = 0; ch < nch; ++ch) take(ch, hit_mask(ch));
  }
  if (lane == 0)
    reinterpret_cast<int2*>(bwd)[static_cast<size_t>(bh) * nKt + j] =
        first < 0 ? make_int2(0, 0) : make_int2(first, last + 1);
}

// ---------------------------------------------------------------------------
// Launch order of the attention workgroups: tiles sorted by range length,
// longest first (a longest-processing-time-first schedule), within G groups
// of heads (head bh in group bh % G; G = 8 when B*H is a multiple of 8, else
// the largest divisor of B*H not above 8). Workgroup x of an attention
// launch takes order[x]; the hardware hands workgroup x to XCD x % 8, so with
// G = 8 each XCD works on its own heads (their K/V stay in that XCD's L2).
// One workgroup per group:
// counting sort over the length bins in LDS. Items of equal length may come
// in any order; every order gives the same attention results.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_work_order(const int2* __restrict__ tab, int BH, int nT, int span, int G,
                                                     int32_t* __restrict__ order) {
  extern __shared__ int32_t bins[];  // span + 1 bins: bin span - len
  __shared__ int32_t wsum[16];
  const int g = blockIdx.x;
  const int hpg = BH / G;
  const int n = hpg * nT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nbins = span + 1;
  for (int i = tid; i < nbins; i += 1024) bins[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int bh = g + (i / nT) * G, t = i % nT;
    const int2 r = tab[static_cast<size_t>(bh) * nT + t];
    const int len = min(max(r.y - r.x, 0), span);
    atomicAdd(&bins[span - len], 1);
  }
  __syncthreads();
  // exclusive scan of the bins: each thread owns a contiguous run of bins
  const int per = (nbins + 1023) / 1024;
  const int b0 = min(tid * per, nbins), b1 = min(b0 + per, nbins);
  int s = 0;
  for (int k = b0; k < b1; ++k) s += bins[k];
  int x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = x - s;
  for (int k = 0; k < w; ++k) pre += wsum[k];
  for (int k = b0; k < b1; ++k) {
    const int c = bins[k];
    bins[k] = pre;
    pre += c;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int bh = g + (i / nT) * G, t = i % nT;
    const int2 r = tab[static_cast<size_t>(bh) * nT + t];
    const int len = min(max(r.y - r.x, 0), span);
    const int slot = atomicAdd(&bins[span - len], 1);
    order[static_cast<size_t>(slot) * G + g] = bh * nT + t;
  }
}

// ---------------------------------------------------------------------------
// Work of one workgroup of the one-launch table and order kernels, and where
// its items go in the order. Groups: workgroup g takes the heads g, g + G,
// g + 2G, ... (all their tiles) and its slot s goes to order[s * G + g].
// Runs: the B*H*nT items (head-major) are cut into 8 runs of consecutive
// items of equal count (the first N % 8 one item longer); workgroup k takes
// run k, which may start or end inside a head, and its slot s goes to
// order[s * 8 + k], so that every XCD (workgroup x runs on XCD x % 8) works
// on about B*H / 8 heads, also when B*H is not a multiple of 8.
// ---------------------------------------------------------------------------
struct OrderSplit {
  bool runs;
  int k, G, nT;
  int lo, n;  // runs: first item and item count of this workgroup; groups: n = items of the group
  int bh0;    // runs: first head of the run
  __device__ OrderSplit(bool runs_, int k_, int G_, int BH, int nT_) : runs(runs_), k(k_), G(G_), nT(nT_) {
    if (runs) {
      const int N = BH * nT, c = N / 8, r = N % 8;
      lo = k * c + min(k, r);
      n = c + (k < r ? 1 : 0);
      bh0 = lo / nT;
    } else {
      lo = 0;
      n = (BH / G) * nT;
      bh0 = 0;
    }
  }
  // heads whose tiles the workgroup reads (slot hl = 0 .. heads() - 1)
  __device__ int heads() const { return runs ? (n ? (lo + n - 1) / nT - bh0 + 1 : 0) : n / nT; }
  __device__ int head(int hl) const { return runs ? bh0 + hl : k + hl * G; }
  // local item li: head slot and tile
  __device__ int slot_of(int li) const { return runs ? (lo + li) / nT - bh0 : li / nT; }
  __device__ int tile_of(int li) const { return runs ? (lo + li) % nT : li % nT; }
  __device__ size_t pos(int s) const { return static_cast<size_t>(s) * G + k; }  // G = 8 for runs
};

// ---------------------------------------------------------------------------
// Forward ranges and launch order in one launch. One workgroup per group of
// heads (the groups of k_work_order). The group's key-tile statistics go to
// LDS. Where a head's key tiles are in layout order (each tile one bucket,
// buckets non-decreasing, and within a bucket non-decreasing smallest
// positions: every layout scfa_hash_layout_qk writes, and the compacted or
// dense rows of the QK and dense modes, whose buckets are all 0), the rules
// reduce to binary searches. Hash (Algorithm 2): start = first key tile
// whose bucket reaches the query tile's, stop = first tile past its bucket,
// and the tiles passing the causal test are a prefix of [start, stop). QK and
// dense (Algorithm 1): end = the prefix of key tiles the query tile reaches.
// Otherwise (or for a hash query tile spanning buckets) the thread scans the
// head's tiles one by one with the same rules. The ranges are then
// counting-sorted by length as in k_work_order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_fwd_table_order(int mode, const int4* __restrict__ qstats,
                                                          const int4* __restrict__ kstats, int BH, int nQt, int nKt,
                                                          int G, bool runs, int2* __restrict__ fwd,
                                                          int32_t* __restrict__ tiles, int32_t* __restrict__ order,
                                                          const Reach rc) {
  extern __shared__ int4 lds4[];
  const OrderSplit sp(runs, blockIdx.x, G, BH, nQt);
  const int nh = sp.heads();
  const int n = sp.n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nbins = nKt + 1;  // bin nKt - len
  int4* ks = lds4;                                               // nh * nKt key-tile statistics
  int32_t* bins = reinterpret_cast<int32_t*>(ks + nh * nKt);     // nbins
  int32_t* lens = bins + nbins;                                  // n range lengths
  __shared__ int32_t ordered[64];                                // per head: tiles in layout order
  __shared__ int32_t cnt_s[64];                                  // per head: processed tiles
  __shared__ int32_t wsum[16];
  for (int i = tid; i < nh * nKt; i += 1024) {
    const int hl = i / nKt, j = i - hl * nKt;
    ks[i] = kstats[static_cast<size_t>(sp.head(hl)) * nKt + j];
  }
  for (int i = tid; i < nbins; i += 1024) bins[i] = 0;
  if (tid < nh) {
    ordered[tid] = 1;
    cnt_s[tid] = 0;
  }
  __syncthreads();
  for (int i = tid; i < nh * nKt; i += 1024) {
    const int hl = i / nKt, j = i - hl * nKt;
    const int4 a = ks[i];
    bool ok = a.z == a.w;
    if (j + 1 < nKt) {
      const int4 c = ks[i + 1];
      ok = ok && (a.w < c.z || (a.w == c.z && a.x <= c.x));
    }
    if (!ok) ordered[hl] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int hl = sp.slot_of(i), t = sp.tile_of(i);
    const int bh = sp.head(hl);
    const int4 qs = qstats[static_cast<size_t>(bh) * nQt + t];
    const int qreach = q_reach(rc, qs.y);
    const int4* k = ks + hl * nKt;
    int start, end, cnt;
    if (mode != SCFA_HASH) {
      // Algorithm 1: key tiles [0, end), end = the tiles whose smallest
      // position the query tile reaches (a prefix where smallest positions
      // are in order, else counted one by one)
      start = 0;
      cnt = 0;
      if (ordered[hl]) {
        int lo = 0, hi = nKt;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (k[mid].x <= qreach) lo = mid + 1; else hi = mid;
        }
        cnt = lo;
      } else {
        for (int j = 0; j < nKt; ++j) cnt += k[j].x <= qreach;
      }
      end = cnt;
    } else if (ordered[hl] && qs.z == qs.w) {
      // first tile whose bucket is >= the query bucket, first tile past it
      int lo = 0, hi = nKt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (k[mid].w < qs.z) lo = mid + 1; else hi = mid;
      }
      start = lo;
      hi = nKt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (k[mid].z <= qs.w) lo = mid + 1; else hi = mid;
      }
      const int stop = lo;
      // tiles of [start, stop) passing the causal test: a prefix
      lo = start;
      hi = stop;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (k[mid].x <= qreach) lo = mid + 1; else hi = mid;
      }
      cnt = lo - start;
      end = lo;
    } else {
      start = 0;
      for (int j = 0; j < nKt; ++j) start += k[j].w < qs.z;
      int stop = nKt;
      for (int j = start; j < nKt; ++j)
        if (k[j].z > qs.w) {
          stop = j;
          break;
        }
      end = start;
      cnt = 0;
      for (int j = start; j < stop; ++j)
        if (k[j].x <= qreach) {
          end = j + 1;
          ++cnt;
        }
    }
    fwd[static_cast<size_t>(bh) * nQt + t] = make_int2(start, end);
    const int len = min(max(end - start, 0), nKt);
    lens[i] = len;
    atomicAdd(&bins[nKt - len], 1);
    if (cnt) atomicAdd(&cnt_s[hl], cnt);
  }
  __syncthreads();
  if (tid < nh && cnt_s[tid]) atomicAdd(&tiles[sp.head(tid)], cnt_s[tid]);
  // exclusive scan of the bins (as k_work_order)
  const int per = (nbins + 1023) / 1024;
  const int b0 = min(tid * per, nbins), b1 = min(b0 + per, nbins);
  int sacc = 0;
  for (int q = b0; q < b1; ++q) sacc += bins[q];
  int x = sacc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = x - sacc;
  for (int q = 0; q < w; ++q) pre += wsum[q];
  for (int q = b0; q < b1; ++q) {
    const int c = bins[q];
    bins[q] = pre;
    pre += c;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int slot = atomicAdd(&bins[nKt - lens[i]], 1);
    order[sp.pos(slot)] = sp.head(sp.slot_of(i)) * nQt + sp.tile_of(i);
  }
}

// ---------------------------------------------------------------------------
// Backward ranges and their launch order in one launch (the results of
// k_bwd_table and k_work_order over the backward table, span = nQt). One
// workgroup per group of heads holds the group's forward ranges and query
// extrema in LDS. Key tile j of a head is processed by the query tiles whose
// forward range holds j and whose largest position reaches the tile's
// smallest; the backward range runs from the first to one past the last of
// them. Where a head's forward starts and ends are both non-decreasing over
// its query tiles (every table of the aligned hash layout, the QK and the
// dense modes), the tiles whose range holds j form one run, found by two
// binary searches, and the reach test is taken from its two ends inward;
// otherwise every query tile is tested. The ranges are then counting-sorted
// by length as in k_work_order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_bwd_table_order(const int4* __restrict__ qstats,
                                                          const int4* __restrict__ kstats,
                                                          const int2* __restrict__ fwd, int BH, int nQt, int nKt,
                                                          int G, bool runs, int2* __restrict__ bwd,
                                                          int32_t* __restrict__ order, const Reach rc) {
  extern __shared__ int2 lds2[];
  const OrderSplit sp(runs, blockIdx.x, G, BH, nKt);
  const int nh = sp.heads();
  const int n = sp.n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nbins = nQt + 1;  // bin nQt - len
  int2* ft = lds2;                                           // nh * nQt forward ranges
  int32_t* qy = reinterpret_cast<int32_t*>(ft + nh * nQt);  // nh * nQt largest query positions
  int32_t* bins = qy + nh * nQt;                             // nbins
  int32_t* lens = bins + nbins;                              // n range lengths
  __shared__ int32_t mono[64];                               // per head: starts and ends in order
  __shared__ int32_t wsum[16];
  for (int i = tid; i < nh * nQt; i += 1024) {
    const int hl = i / nQt, t = i - hl * nQt;
    const size_t gi = static_cast<size_t>(sp.head(hl)) * nQt + t;
    ft[i] = fwd[gi];
    qy[i] = qstats[gi].y;
  }
  for (int i = tid; i < nbins; i += 1024) bins[i] = 0;
  if (tid < nh) mono[tid] = 1;
  __syncthreads();
  for (int i = tid; i < nh * nQt; i += 1024) {
    const int t = i % nQt;
    if (t + 1 < nQt && (ft[i + 1].x < ft[i].x || ft[i + 1].y < ft[i].y)) mono[i / nQt] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int hl = sp.slot_of(i), j = sp.tile_of(i);
    const int bh = sp.head(hl);
    // smallest query position that sees a key of the tile
    const int kreach = k_reach(rc, kstats[static_cast<size_t>(bh) * nKt + j].x);
    const int2* f = ft + hl * nQt;
    const int32_t* y = qy + hl * nQt;
    int first = -1, last = -1;
    if (mono[hl]) {
      // tiles [lo, hi] are those with start <= j < end
      int lo = 0, hi = nQt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (f[mid].y <= j) lo = mid + 1; else hi = mid;
      }
      const int a = lo;
      hi = nQt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (f[mid].x <= j) lo = mid + 1; else hi = mid;
      }
      const int b = lo - 1;
      for (int t = a; t <= b; ++t)
        if (kreach <= y[t]) {
          first = t;
          break;
        }
      if (first >= 0)
        for (int t = b; t >= first; --t)
          if (kreach <= y[t]) {
            last = t;
            break;
          }
    } else {
      for (int t = 0; t < nQt; ++t)
        if (j >= f[t].x && j < f[t].y && kreach <= y[t]) {
          if (first < 0) first = t;
          last = t;
        }
    }
    const int2 r = first < 0 ? make_int2(0, 0) : make_int2(first, last + 1);
    bwd[static_cast<size_t>(bh) * nKt + j] = r;
    const int len = min(r.y - r.x, nQt);
    lens[i] = len;
    atomicAdd(&bins[nQt - len], 1);
  }
  __syncthreads();
  // exclusive scan of the bins (as k_work_order)
  const int per = (nbins + 1023) / 1024;
  const int b0 = min(tid * per, nbins), b1 = min(b0 + per, nbins);
  int sacc = 0;
  for (int q = b0; q < b1; ++q) sacc += bins[q];
  int x = sacc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yv = __shfl_up(x, o);
    if (lane >= o) x += yv;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = x - sacc;
  for (int q = 0; q < w; ++q) pre += wsum[q];
  for (int q = b0; q < b1; ++q) {
    const int c = bins[q];
    bins[q] = pre;
    pre += c;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int slot = atomicAdd(&bins[nQt - lens[i]], 1);
    order[sp.pos(slot)] = sp.head(sp.slot_of(i)) * nKt + sp.tile_of(i);
  }
}

// ---------------------------------------------------------------------------
// Exact visible-pair count (binary searches in the sorted key arrays).
// ---------------------------------------------------------------------------

__global__ void k_zero_i64(int64_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void k_count_visible(int mode, const int32_t* __restrict__ q_idx,
                                                       const int32_t* __restrict__ k_idx,
                                                       const int32_t* __restrict__ q_bkt,
                                                       const int32_t* __restrict__ k_bkt, int Tq, int Tk, int TqP,
                                                       int TkP, int64_t* __restrict__ pairs, const Reach rc) {
  __shared__ long long part[4];
  const int bh = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  long long n = 0;
  if (r < Tq) {
    if (mode == SCFA_DENSE) {
      n = min(static_cast<long long>(q_reach(rc, r)) + 1, static_cast<long long>(Tk));
    } else {
      const int p0 = q_idx[static_cast<size_t>(bh) * TqP + r];
      const int p = q_reach(rc, p0);  // keys at positions <= p are visible
      const int32_t* kp = k_idx + static_cast<size_t>(bh) * TkP;
      if (p0 >= 0) {
        if (mode == SCFA_QK) {
          int lo = 0, hi = Tk;  // first s with kp[s] > p
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kp[mid] <= p) lo = mid + 1; else hi = mid;
          }
          n = lo;
        } else {
          const int qb = q_bkt[static_cast<size_t>(bh) * TqP + r];
          const int32_t* kb = k_bkt + static_cast<size_t>(bh) * TkP;
          int lo = 0, hi = Tk;  // first s with (kb, kp) > (qb, p)
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kb[mid] < qb || (kb[mid] == qb && kp[mid] <= p)) lo = mid + 1; else hi = mid;
          }
          const int up = lo;
          lo = 0;
          hi = Tk;  // first s with kb >= qb
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kb[mid] < qb) lo = mid + 1; else hi = mid;
          }
          n = up - lo;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long s = part[0] + part[1] + part[2] + part[3];
    if (s) atomicAdd(reinterpret_cast<unsigned long long*>(pairs + bh), static_cast<unsigned long long>(s));
  }
}

}  // namespace
}  // namespace scfa

using namespace scfa;

extern "C" {

const char* scfa_status_string(int status) {
  switch (status) {
    case SCFA_OK: return "SCFA_OK";
    case SCFA_ERR_INVALID: return "SCFA_ERR_INVALID: invalid argument";
    case SCFA_ERR_UNSUPPORTED: return "SCFA_ERR_UNSUPPORTED: configuration not built";
    case SCFA_ERR_HIP: return "SCFA_ERR_HIP: HIP launch or runtime error";
    case SCFA_ERR_TOO_LARGE: return "SCFA_ERR_TOO_LARGE: problem exceeds the static scratch of a no-allocation entry point";
    default: return "SCFA: unknown status";
  }
}

int scfa_version(void) { return 100; }

int scfa_qk_count(const uint8_t* keep, int B, int T, int H, int32_t* count, int32_t* max_count,
                  int32_t* chunk_offsets, hipStream_t stream) {
  if (!keep || !count || !max_count || !chunk_offsets) return SCFA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1) return SCFA_ERR_INVALID;
  const int nC = ceil_div(T, SCFA_COUNT_CHUNK);
  hipLaunchKernelGGL(k_qk_chunk_counts, dim3(nC, B), dim3(256), 0, stream, keep, T, H, nC, chunk_offsets, max_count);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_qk_scan, dim3(B * H), dim3(256), 0, stream, chunk_offsets, nC, count, max_count);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_qk_index_qk(const uint8_t* keep_q, const uint8_t* keep_k, int B, int T, int T_kv, int H, int Tq, int Tk,
                     int32_t* count_q, int32_t* count_k, int32_t* max_count, int32_t* chunk_counts_q,
                     int32_t* chunk_counts_k, int32_t* q_idx, int32_t* k_idx, int32_t* qstats, int32_t* kstats,
                     int32_t* tiles, int32_t* dev_err, hipStream_t stream) {
  if (!keep_q || !keep_k || !count_q || !count_k || !max_count || !chunk_counts_q || !chunk_counts_k || !q_idx ||
      !k_idx)
    return SCFA_ERR_INVALID;
  if ((qstats == nullptr) != (kstats == nullptr) || (qstats == nullptr) != (tiles == nullptr)) return SCFA_ERR_INVALID;
  if (B < 1 || T < 1 || T_kv < 1 || H < 1 || H > 128) return SCFA_ERR_INVALID;
  for (int tc : {Tq, Tk})
    if (tc < SCFA_ROW_ALIGN || tc % SCFA_ROW_ALIGN) return SCFA_ERR_INVALID;
  auto side = [&](const uint8_t* keep, int t, int tc, int32_t pad, int32_t* chunk, int32_t* count, int32_t* mx,
                  int32_t* idx, int32_t* stats, int bs) {
    QkSide sd;
    sd.keep = keep;
    sd.T = t;
    sd.nC = ceil_div(t, SCFA_COUNT_CHUNK);
    sd.nCx = ceil_div(t > tc ? t : tc, SCFA_COUNT_CHUNK);
    sd.Tc = tc;
    sd.pad = pad;
    sd.chunk = chunk;
    sd.count = count;
    sd.max_count = mx;
    sd.idx = idx;
    sd.stats = stats;
    sd.bs = bs;
    return sd;
  };
  const QkSide sq = side(keep_q, T, Tq, SCFA_Q_PAD, chunk_counts_q, count_q, max_count, q_idx, qstats, SCFA_TILE_M);
  const QkSide sk = side(keep_k, T_kv, Tk, SCFA_K_PAD, chunk_counts_k, count_k, max_count + 1, k_idx, kstats,
                         SCFA_TILE_N);
  hipLaunchKernelGGL(k_qk_chunk_counts_qk, dim3(max(sq.nC, sk.nC), B, 2), dim3(256), 0, stream, sq, sk, H);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_qk_index_qk, dim3(max(sq.nCx, sk.nCx), B, 2), dim3(256), 0, stream, sq, sk, H, dev_err,
                     tiles);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_qk_compact(int dtype, const void* x, const uint8_t* keep, const int32_t* count, const int32_t* chunk_offsets,
                    int B, int T, int H, int D, int Tc, int32_t pad_idx, void* x_c, int32_t* idx_c, int32_t* dev_err,
                    hipStream_t stream) {
  if (!keep || !count || !chunk_offsets || !idx_c) return SCFA_ERR_INVALID;
  if (x_c && !x) return SCFA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1 || H > 128 || Tc < SCFA_ROW_ALIGN || Tc % SCFA_ROW_ALIGN) return SCFA_ERR_INVALID;
  if (!dtype_ok(dtype)) return SCFA_ERR_INVALID;
  if (x_c && D != 64) return SCFA_ERR_UNSUPPORTED;
  const int nC = ceil_div(T, SCFA_COUNT_CHUNK);
  const int nCx = ceil_div(T > Tc ? T : Tc, SCFA_COUNT_CHUNK);
  const size_t lds = static_cast<size_t>(H) * 64 * sizeof(int32_t);
  if (dtype == SCFA_BF16)
    hipLaunchKernelGGL(k_qk_compact<2>, dim3(nCx, B), dim3(256), lds, stream, static_cast<const uint8_t*>(x), keep,
                       count, chunk_offsets, T, H, D, Tc, nC, pad_idx, static_cast<uint8_t*>(x_c), idx_c, dev_err);
  else
    hipLaunchKernelGGL(k_qk_compact<4>, dim3(nCx, B), dim3(256), lds, stream, static_cast<const uint8_t*>(x), keep,
                       count, chunk_offsets, T, H, D, Tc, nC, pad_idx, static_cast<uint8_t*>(x_c), idx_c, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

// nx = 1: side x only; nx = 2: sides x and x2 in one launch (grid z);
// keep / keep2: optional keep masks of the two sides (both or neither).
static int launch_hash_bucket(int dtype, int nx, const void* x, const void* x2, const float* R, int B, int T, int H,
                              int D, int nb, int32_t* bucket, int32_t* bucket2, int32_t* counts, int32_t* counts2,
                              const uint8_t* keep, const uint8_t* keep2, int side0, hipStream_t stream) {
  if (!x || !R || !bucket || (nx == 2 && (!x2 || !bucket2))) return SCFA_ERR_INVALID;
  // keep masks: both sides or neither in a two-side launch; one side's mask
  // (keep2 unused) in a one-side launch
  if (nx == 2 ? (keep != nullptr) != (keep2 != nullptr) : keep2 != nullptr) return SCFA_ERR_INVALID;
  if (side0 != 0 && (nx != 1 || !keep)) return SCFA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1 || nb < 2 || nb % 2) return SCFA_ERR_INVALID;
  if (!dtype_ok(dtype)) return SCFA_ERR_INVALID;
  if (D != 64 || nb > (keep ? 62 : 64)) return SCFA_ERR_UNSUPPORTED;
  const dim3 grid(ceil_div(T, 256), B * H, nx);
  const int half = nb / 2;
#define SCFA_BUCKET_CASE(HALF)                                                                         \
  case HALF:                                                                                           \
    if (dtype == SCFA_BF16)                                                                            \
      bucket_launch<uint16_t, HALF>(grid, stream, x, x2, R, T, H, bucket, bucket2, counts, counts2, keep, \
                                    keep2, side0);                                                     \
    else                                                                                               \
      bucket_launch<float, HALF>(grid, stream, x, x2, R, T, H, bucket, bucket2, counts, counts2, keep,    \
                                 keep2, side0);                                                        \
    break;
  switch (half) {
    SCFA_BUCKET_CASE(1)
    SCFA_BUCKET_CASE(2)
    SCFA_BUCKET_CASE(3)
    SCFA_BUCKET_CASE(4)
    SCFA_BUCKET_CASE(5)
    SCFA_BUCKET_CASE(6)
    SCFA_BUCKET_CASE(7)
    SCFA_BUCKET_CASE(8)
    SCFA_BUCKET_CASE(12)
    SCFA_BUCKET_CASE(16)
    SCFA_BUCKET_CASE(24)
    SCFA_BUCKET_CASE(32)
    default:
      return SCFA_ERR_UNSUPPORTED;
  }
#undef SCFA_BUCKET_CASE
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_hash_bucket(int dtype, const void* x, const float* R, int B, int T, int H, int D, int nb, int32_t* bucket,
                     hipStream_t stream) {
  return launch_hash_bucket(dtype, 1, x, nullptr, R, B, T, H, D, nb, bucket, nullptr, nullptr, nullptr, nullptr,
                            nullptr, 0, stream);
}

int scfa_hash_bucket_counts(int dtype, const void* x, const float* R, int B, int T, int H, int D, int nb,
                            int32_t* bucket, int32_t* chunk_counts, hipStream_t stream) {
  if (!chunk_counts) return SCFA_ERR_INVALID;
  return launch_hash_bucket(dtype, 1, x, nullptr, R, B, T, H, D, nb, bucket, nullptr, chunk_counts, nullptr, nullptr,
                            nullptr, 0, stream);
}

int scfa_hash_bucket_counts_drop(int dtype, const void* x, const float* R, const uint8_t* keep, int side, int B, int T,
                                 int H, int D, int nb, int32_t* bucket, int32_t* chunk_counts, hipStream_t stream) {
  if (!chunk_counts || !keep || (side != 0 && side != 1)) return SCFA_ERR_INVALID;
  return launch_hash_bucket(dtype, 1, x, nullptr, R, B, T, H, D, nb, bucket, nullptr, chunk_counts, nullptr, keep,
                            nullptr, side, stream);
}

int scfa_hash_bucket_qk(int dtype, const void* q, const void* k, const float* R, const uint8_t* keep_q,
                        const uint8_t* keep_k, int B, int T, int H, int D, int nb, int32_t* bucket_q, int32_t* bucket_k,
                        int32_t* counts_q, int32_t* counts_k, hipStream_t stream) {
  if (!counts_q || !counts_k) return SCFA_ERR_INVALID;
  return launch_hash_bucket(dtype, 2, q, k, R, B, T, H, D, nb, bucket_q, bucket_k, counts_q, counts_k, keep_q, keep_k,
                            0, stream);
}

size_t scfa_hash_sort_workspace_bytes(int B, int H, int T, int nb) {
  if (B < 1 || H < 1 || T < 1 || nb < 1) return 0;
  return static_cast<size_t>(B) * H * ceil_div(T, kSortChunk) * nb * sizeof(int32_t);
}

int scfa_hash_sort(const int32_t* bucket, int B, int H, int T, int nb, int32_t pad_idx, int32_t* perm,
                   int32_t* bucket_sorted, int32_t* offsets, void* workspace, size_t workspace_bytes,
                   int32_t* dev_err, hipStream_t stream) {
  if (!bucket || !perm || !bucket_sorted || !offsets || !workspace) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || nb < 1) return SCFA_ERR_INVALID;
  if (nb > 64) return SCFA_ERR_UNSUPPORTED;
  if (workspace_bytes < scfa_hash_sort_workspace_bytes(B, H, T, nb)) return SCFA_ERR_INVALID;
  const int nC = ceil_div(T, kSortChunk);
  const int Tp = pad_rows(T);
  const int nCx = ceil_div(Tp, kSortChunk);
  int32_t* hist = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(k_sort_hist, dim3(nC, B * H), dim3(256), 0, stream, bucket, T, nb, nC, hist, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  const SortSide sd{bucket, hist, pad_idx, 0, 0, perm, bucket_sorted, offsets, nullptr, nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(k_sort_scatter, dim3(nCx, B * H), dim3(256), 0, stream, sd, sd, T, Tp, nb, nC, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_hash_segment_rows(int T, int nb, int align) {
  if (T < 1 || nb < 1 || nb > 64 || !(align == 16 || align == 32 || align == 64 || align == 128)) return 0;
  const long long n = static_cast<long long>(T) + static_cast<long long>(nb) * (align - 1);
  if (n > (1ll << 30)) return 0;
  return pad_rows(static_cast<int>(n));
}

int scfa_hash_segments(const int32_t* perm, const int32_t* offsets, int B, int H, int T, int nb, int align,
                       int32_t pad_idx, int Tseg, int32_t* idx_seg, int32_t* bkt_seg, int32_t* seg_offsets,
                       int32_t* dev_err, hipStream_t stream) {
  if (!perm || !offsets || !idx_seg || !bkt_seg || !seg_offsets) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || nb < 1) return SCFA_ERR_INVALID;
  if (nb > 64) return SCFA_ERR_UNSUPPORTED;
  if (!(align == 16 || align == 32 || align == 64 || align == 128)) return SCFA_ERR_INVALID;
  if (Tseg < SCFA_ROW_ALIGN || Tseg % SCFA_ROW_ALIGN || Tseg < T) return SCFA_ERR_INVALID;
  hipLaunchKernelGGL(k_hash_segments, dim3(ceil_div(Tseg, 256), B * H), dim3(256), 0, stream, perm, offsets,
                     pad_rows(T), nb, align, pad_idx, Tseg, idx_seg, bkt_seg, seg_offsets, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_hash_layout(const int32_t* bucket, const int32_t* chunk_counts, int B, int H, int T, int nb, int align,
                     int32_t pad_idx, int Tseg, int32_t* perm, int32_t* bucket_sorted, int32_t* offsets,
                     int32_t* idx_seg, int32_t* bkt_seg, int32_t* seg_offsets, int32_t* dev_err, hipStream_t stream) {
  if (!bucket || !chunk_counts || !perm || !bucket_sorted || !offsets) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || nb < 1) return SCFA_ERR_INVALID;
  if (nb > 64) return SCFA_ERR_UNSUPPORTED;
  if (align != 0) {
    if (!(align == 16 || align == 32 || align == 64 || align == 128)) return SCFA_ERR_INVALID;
    if (!idx_seg || !bkt_seg || !seg_offsets) return SCFA_ERR_INVALID;
    if (Tseg < SCFA_ROW_ALIGN || Tseg % SCFA_ROW_ALIGN || Tseg < T) return SCFA_ERR_INVALID;
  }
  const int nC = ceil_div(T, kSortChunk);
  const int Tp = pad_rows(T);
  const int nW = ceil_div(align != 0 ? max(Tp, Tseg) : Tp, kSortChunk);
  const SortSide sd{bucket, chunk_counts, pad_idx, align,       Tseg,    perm,    bucket_sorted,
                    offsets, idx_seg,      bkt_seg, seg_offsets, nullptr, nullptr};
  hipLaunchKernelGGL(k_sort_scatter, dim3(nW, B * H), dim3(256), 0, stream, sd, sd, T, Tp, nb, nC, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_hash_layout_qk(const int32_t* bucket_q, const int32_t* bucket_k, const int32_t* counts_q,
                        const int32_t* counts_k, int B, int H, int T, int nb, int Tseg_q, int Tseg_k, int32_t* perm_q,
                        int32_t* perm_k, int32_t* bsorted_q, int32_t* bsorted_k, int32_t* offsets_q,
                        int32_t* offsets_k, int32_t* idx_q, int32_t* idx_k, int32_t* bkt_q, int32_t* bkt_k,
                        int32_t* seg_q, int32_t* seg_k, int32_t* qstats, int32_t* kstats, int32_t* tiles,
                        int32_t* dev_err, hipStream_t stream) {
  if (!bucket_q || !bucket_k || !counts_q || !counts_k || !perm_q || !perm_k || !bsorted_q || !bsorted_k ||
      !offsets_q || !offsets_k || !idx_q || !idx_k || !bkt_q || !bkt_k || !seg_q || !seg_k)
    return SCFA_ERR_INVALID;
  if (!((qstats && kstats && tiles) || (!qstats && !kstats && !tiles))) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1 || nb < 1) return SCFA_ERR_INVALID;
  if (nb > 64) return SCFA_ERR_UNSUPPORTED;
  for (const int Tseg : {Tseg_q, Tseg_k})
    if (Tseg < SCFA_ROW_ALIGN || Tseg % SCFA_ROW_ALIGN || Tseg < T) return SCFA_ERR_INVALID;
  const int nC = ceil_div(T, kSortChunk);
  const int Tp = pad_rows(T);
  const int nW = ceil_div(max(Tp, max(Tseg_q, Tseg_k)), kSortChunk);
  const SortSide sq{bucket_q, counts_q, SCFA_Q_PAD, SCFA_TILE_M, Tseg_q, perm_q, bsorted_q, offsets_q, idx_q, bkt_q,
                    seg_q,    qstats,   tiles};
  const SortSide sk{bucket_k, counts_k, SCFA_K_PAD, SCFA_TILE_N, Tseg_k, perm_k, bsorted_k, offsets_k, idx_k, bkt_k,
                    seg_k,    kstats,   nullptr};
  hipLaunchKernelGGL(k_sort_scatter, dim3(nW, B * H, 2), dim3(256), 0, stream, sq, sk, T, Tp, nb, nC, dev_err);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_gather(int dtype, int layout, const void* x, const int32_t* idx, int B, int T, int H, int D, int Tp,
                void* x_p, hipStream_t stream) {
  if (!x || !idx || !x_p) return SCFA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1 || Tp < SCFA_ROW_ALIGN || Tp % SCFA_ROW_ALIGN) return SCFA_ERR_INVALID;
  if (!dtype_ok(dtype) || (layout != SCFA_ROWS && layout != SCFA_COLS)) return SCFA_ERR_INVALID;
  if (D != 64) return SCFA_ERR_UNSUPPORTED;
  if (layout == SCFA_ROWS) {
    const int U = D * dtype_size(dtype) / 16;
    const dim3 grid(ceil_div(Tp * U, 256), B * H);
    if (dtype == SCFA_BF16)
      hipLaunchKernelGGL(k_gather_rows<2>, grid, dim3(256), 0, stream, static_cast<const uint8_t*>(x), idx, T, H, D,
                         Tp, static_cast<uint8_t*>(x_p));
    else
      hipLaunchKernelGGL(k_gather_rows<4>, grid, dim3(256), 0, stream, static_cast<const uint8_t*>(x), idx, T, H, D,
                         Tp, static_cast<uint8_t*>(x_p));
  } else {
    const dim3 grid(Tp / 64, B * H);
    if (dtype == SCFA_BF16)
      hipLaunchKernelGGL(k_gather_cols<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x), idx, T,
                         H, Tp, static_cast<uint16_t*>(x_p));
    else
      hipLaunchKernelGGL(k_gather_cols<float>, grid, dim3(256), 0, stream, static_cast<const float*>(x), idx, T, H,
                         Tp, static_cast<float*>(x_p));
  }
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_range_table(int mode, const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt,
                     int B, int H, int Tq, int Tk, int Bm, int Bn, int32_t* qstats, int32_t* kstats, int32_t* fwd_tab,
                     int32_t* bwd_tab, int32_t* tiles, hipStream_t stream) {
  const int flags = take_flags(mode);
  if (!flags_ok(flags) || (mode != SCFA_DENSE && mode != SCFA_QK && mode != SCFA_HASH)) return SCFA_ERR_INVALID;
  const Reach rc = reach_of(flags);
  if (!qstats || !kstats || !tiles || (!fwd_tab && bwd_tab)) return SCFA_ERR_INVALID;
  if (mode != SCFA_DENSE && (!q_idx || !k_idx)) return SCFA_ERR_INVALID;
  if (mode == SCFA_HASH && (!q_bkt || !k_bkt)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || Tq < 1 || Tk < 1) return SCFA_ERR_INVALID;
  auto tile_ok = [](int t) { return t == 16 || t == 32 || t == 64 || t == 128; };
  if (!tile_ok(Bm) || !tile_ok(Bn)) return SCFA_ERR_INVALID;
  const int TqP = pad_rows(Tq), TkP = pad_rows(Tk);
  const int nQt = TqP / Bm, nKt = TkP / Bn;
  hipLaunchKernelGGL(k_tile_stats, dim3(nQt + nKt, B * H), dim3(64), 0, stream, mode, q_idx, k_idx, q_bkt, k_bkt, Tq,
                     Tk, TqP, TkP, Bm, Bn, nQt, nKt, qstats, kstats, tiles);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  if (!fwd_tab) return SCFA_OK;  // statistics only (scfa_fwd_table_order builds the ranges)
  hipLaunchKernelGGL(k_fwd_table, dim3(ceil_div(nQt, kTabWaves), B * H), dim3(64 * kTabWaves), 0, stream, mode, qstats,
                     kstats, nQt, nKt, fwd_tab, tiles, rc);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  if (bwd_tab) {
    hipLaunchKernelGGL(k_bwd_table, dim3(ceil_div(nKt, 4), B * H), dim3(256), 0, stream, qstats, kstats, fwd_tab, nQt,
                       nKt, bwd_tab, rc);
    SCFA_RETURN_IF_LAUNCH_FAILED();
  }
  return SCFA_OK;
}

int scfa_fwd_table(int mode, const int32_t* qstats, const int32_t* kstats, int B, int H, int nQt, int nKt,
                   int32_t* fwd_tab, int32_t* tiles, hipStream_t stream) {
  const int flags = take_flags(mode);
  if (!flags_ok(flags) || (mode != SCFA_DENSE && mode != SCFA_QK && mode != SCFA_HASH)) return SCFA_ERR_INVALID;
  const Reach rc = reach_of(flags);
  if (!qstats || !kstats || !fwd_tab || !tiles) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || nQt < 1 || nKt < 1) return SCFA_ERR_INVALID;
  hipLaunchKernelGGL(k_fwd_table, dim3(ceil_div(nQt, kTabWaves), B * H), dim3(64 * kTabWaves), 0, stream, mode, qstats,
                     kstats, nQt, nKt, fwd_tab, tiles, rc);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_bwd_table(const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, int B, int H, int nQt, int nKt,
                   int32_t* bwd_tab, int flags, hipStream_t stream) {
  if (!qstats || !kstats || !fwd_tab || !bwd_tab) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || nQt < 1 || nKt < 1 || !flags_ok(flags)) return SCFA_ERR_INVALID;
  hipLaunchKernelGGL(k_bwd_table, dim3(ceil_div(nKt, 4), B * H), dim3(256), 0, stream, qstats, kstats, fwd_tab, nQt, nKt,
                     bwd_tab, reach_of(flags));
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

// Groups of heads of a launch order: 8 when B*H is a multiple of 8 (one
// group per XCD), else the largest divisor of B*H not above 8, so that
// several workgroups share the building of the order.
static int order_groups(int BH) {
  if (BH % 8 == 0) return 8;
  for (int g = 7; g > 1; --g)
    if (BH % g == 0) return g;
  return 1;
}

// Work split of the one-launch table and order kernels: 8 runs of
// consecutive items when `runs_ok` and B*H is not a multiple of 8 (the hash
// modes, whose tiles carry similar work along a head; in the causal QK and
// dense modes a run that ends inside a head would carry less work than one
// that starts there), else the groups of scfa_work_order. heads / items:
// the most heads and items one workgroup handles.
struct OrderPlan {
  bool runs;
  int G, heads, items;
};
static OrderPlan order_plan(bool runs_ok, int BH, int nT) {
  OrderPlan op;
  op.runs = runs_ok && BH % 8 != 0;
  if (op.runs) {
    const long long N = static_cast<long long>(BH) * nT;
    const int c1 = static_cast<int>((N + 7) / 8);
    op.G = 8;
    op.items = c1;
    op.heads = min(BH, (c1 + nT - 1) / nT + 1);
  } else {
    op.G = order_groups(BH);
    op.heads = BH / op.G;
    op.items = op.heads * nT;
  }
  return op;
}

int scfa_work_order(const int32_t* tab, int B, int H, int ntiles, int span, int32_t* order, hipStream_t stream) {
  if (!tab || !order) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || ntiles < 1 || span < 1 || span > kMaxOrderSpan) return SCFA_ERR_INVALID;
  const int BH = B * H;
  const int G = order_groups(BH);
  const size_t lds = static_cast<size_t>(span + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(k_work_order, dim3(G), dim3(1024), lds, stream, reinterpret_cast<const int2*>(tab), BH, ntiles,
                     span, G, order);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_bwd_table_order(const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, int B, int H, int nQt,
                         int nKt, int32_t* bwd_tab, int32_t* order, int flags, hipStream_t stream) {
  if (!qstats || !kstats || !fwd_tab || !bwd_tab || !order) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || nQt < 1 || nKt < 1 || nQt > kMaxOrderSpan || !flags_ok(flags)) return SCFA_ERR_INVALID;
  const int BH = B * H;
  const OrderPlan op = order_plan(true, BH, nKt);
  const size_t lds = static_cast<size_t>(op.heads) * nQt * (sizeof(int2) + 4) +
                     static_cast<size_t>(nQt + 1 + op.items) * 4;
  if (op.heads > 64 || lds > kTableOrderLds) {  // too large for one workgroup's LDS: the two launches
    const int st = scfa_bwd_table(qstats, kstats, fwd_tab, B, H, nQt, nKt, bwd_tab, flags, stream);
    if (st != SCFA_OK) return st;
    return scfa_work_order(bwd_tab, B, H, nKt, nQt, order, stream);
  }
  hipLaunchKernelGGL(k_bwd_table_order, dim3(op.G), dim3(1024), lds, stream, reinterpret_cast<const int4*>(qstats),
                     reinterpret_cast<const int4*>(kstats), reinterpret_cast<const int2*>(fwd_tab), BH, nQt, nKt, op.G,
                     op.runs, reinterpret_cast<int2*>(bwd_tab), order, reach_of(flags));
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_fwd_table_order(int mode, const int32_t* qstats, const int32_t* kstats, int B, int H, int nQt, int nKt,
                         int32_t* fwd_tab, int32_t* tiles, int32_t* order, hipStream_t stream) {
  const int flags = take_flags(mode);
  if (!flags_ok(flags) || (mode != SCFA_DENSE && mode != SCFA_QK && mode != SCFA_HASH)) return SCFA_ERR_INVALID;
  if (!qstats || !kstats || !fwd_tab || !tiles || !order) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || nQt < 1 || nKt < 1 || nKt > kMaxOrderSpan) return SCFA_ERR_INVALID;
  const int BH = B * H;
  const OrderPlan op = order_plan(mode == SCFA_HASH, BH, nQt);
  const size_t lds = static_cast<size_t>(op.heads) * nKt * sizeof(int4) + static_cast<size_t>(nKt + 1 + op.items) * 4;
  if (op.heads > 64 || lds > kTableOrderLds) {  // too large for one workgroup's LDS: the two launches
    const int st = scfa_fwd_table(mode | flags, qstats, kstats, B, H, nQt, nKt, fwd_tab, tiles, stream);
    if (st != SCFA_OK) return st;
    return scfa_work_order(fwd_tab, B, H, nQt, nKt, order, stream);
  }
  hipLaunchKernelGGL(k_fwd_table_order, dim3(op.G), dim3(1024), lds, stream, mode,
                     reinterpret_cast<const int4*>(qstats), reinterpret_cast<const int4*>(kstats), BH, nQt, nKt, op.G,
                     op.runs, reinterpret_cast<int2*>(fwd_tab), tiles, order, reach_of(flags));
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

int scfa_count_visible(int mode, const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt,
                       int B, int H, int Tq, int Tk, int64_t* pairs, hipStream_t stream) {
  const int flags = take_flags(mode);
  if (!flags_ok(flags) || (mode != SCFA_DENSE && mode != SCFA_QK && mode != SCFA_HASH)) return SCFA_ERR_INVALID;
  const Reach rc = reach_of(flags);
  if (!pairs) return SCFA_ERR_INVALID;
  if (mode != SCFA_DENSE && (!q_idx || !k_idx)) return SCFA_ERR_INVALID;
  if (mode == SCFA_HASH && (!q_bkt || !k_bkt)) return SCFA_ERR_INVALID;
  if (B < 1 || H < 1 || Tq < 1 || Tk < 1) return SCFA_ERR_INVALID;
  hipLaunchKernelGGL(k_zero_i64, dim3(ceil_div(B * H, 256)), dim3(256), 0, stream, pairs, B * H);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  hipLaunchKernelGGL(k_count_visible, dim3(ceil_div(Tq, 256), B * H), dim3(256), 0, stream, mode, q_idx, k_idx, q_bkt,
                     k_bkt, Tq, Tk, pad_rows(Tq), pad_rows(Tk), pairs, rc);
  SCFA_RETURN_IF_LAUNCH_FAILED();
  return SCFA_OK;
}

}  // extern "C"
