/*
 * scfa.h -- C ABI of libscfa.so: sparse causal flash attention (SCFA) on
 * AMD MI355X (gfx950).
 *
 * The operations follow the explainer page "Faster Causal Attention Over
 * Large Sequences Through Sparse Flash Attention" (arXiv 2306.01160),
 * cited below as "SCFA explainer" with its section names.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers are DEVICE pointers unless stated otherwise; the caller
 *    owns and allocates all memory. The library never allocates, frees or
 *    synchronises, and keeps no pointer after returning.
 *  - Every call only enqueues work on `stream` (may be NULL = default
 *    stream) and returns; results are ready when the stream is.
 *  - Return value: SCFA_OK, or a negative status. Argument errors that the
 *    host can see (NULL pointer, bad size, unsupported dtype/mode) return
 *    SCFA_ERR_INVALID / SCFA_ERR_UNSUPPORTED before anything is enqueued.
 *    A failed kernel launch returns SCFA_ERR_HIP.
 *  - Data-dependent errors that only the device can see (a kept count above
 *    the compacted length, a bucket id outside [0, nb)) OR a bit into the
 *    caller's `dev_err` word (may be NULL) without a host sync; the affected
 *    outputs are then unspecified, but no access leaves its buffer.
 *  - Layouts: user tensors are (B, T, H, D) row-major ("3.2 Big-Picture
 *    Architecture", items 2 and 4); per-head index arrays are (B, H, n);
 *    compacted / sorted tensors are head-major. The attention calls address
 *    rows inside one batch entry's T x H x D block with 32-bit byte offsets:
 *    a block of 4 GiB or more returns SCFA_ERR_UNSUPPORTED.
 *  - Row buffers of compacted / sorted tensors hold Tpad = SCFA_PAD(n) rows,
 *    n = valid rows (Tc for QK compaction, T for hash sorting). Rows
 *    beyond n are zero; their index entries are the pads (-1 query,
 *    1000000000 key).
 *  - Supported: D = 64; dtype bf16 or fp32 (all operands of one call share
 *    the input dtype). The library is stateless and thread-safe.
 */
#ifndef SCFA_H_
#define SCFA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define SCFA_OK 0
#define SCFA_ERR_INVALID (-1)     /* bad argument (NULL, size, range)          */
#define SCFA_ERR_UNSUPPORTED (-2) /* valid but not built (e.g. D != 64)        */
#define SCFA_ERR_HIP (-3)         /* a HIP launch/runtime call failed          */
#define SCFA_ERR_TOO_LARGE (-4)   /* beyond the static scratch of a no-allocation entry point */

/* ---- device error bits (OR-ed into *dev_err) -------------------------- */
#define SCFA_DEVERR_COUNT_EXCEEDS_TC 1 /* a head keeps more tokens than Tc     */
#define SCFA_DEVERR_BUCKET_RANGE 2     /* a bucket id outside [0, nb)           */
#define SCFA_DEVERR_SEGMENT_OVERFLOW 4 /* a bucket-aligned layout exceeds Tseg  */

/* ---- enums ------------------------------------------------------------- */
#define SCFA_BF16 0 /* bfloat16 storage, fp32 accumulation */
#define SCFA_F32 1  /* float32 storage and accumulation     */

#define SCFA_DENSE 0 /* causal attention, positions 0..T-1 */
#define SCFA_QK 1    /* QK-drop: compacted keys/queries      */
#define SCFA_HASH 2  /* hash-sparse: bucket-sorted           */
/* Flag OR-ed into a mode (or passed as `flags`): strict causality, a key is
 * visible only strictly before its query (k_pos < q_pos), the explainer's
 * '>' variant of the causal test ("Design choice: >= vs >"); a query then
 * never attends to itself. Every call of one forward/backward pass must
 * agree on it (tables, attention, backward, pair count). */
#define SCFA_STRICT 16
/* Flag OR-ed into a mode (or passed as `flags`): no causal test, every kept
 * (QK) or same-bucket (hash) key is visible to every query -- bidirectional
 * attention, which the explainer names as untested ("Critical Assessment",
 * "Additional Weaknesses and Missing Experiments": causal attention only).
 * Every original position must lie below 2^28 (the attention entry points
 * check T; the table and pair-count calls rely on the caller). It excludes
 * SCFA_STRICT (SCFA_ERR_INVALID when both are set), and every call of one
 * pass must agree on it, as for SCFA_STRICT. */
#define SCFA_NONCAUSAL 32

#define SCFA_ROWS 0 /* (B, H, Tpad, D): one row per token           */
#define SCFA_COLS 1 /* (B, H, D, Tpad): transposed, one row per dim */

/* Sentinel indices for padded rows (SCFA explainer, 3.4, QK-Sparse
 * Attention, compaction step; Hyperparameters and Implementation Constants). */
#define SCFA_Q_PAD (-1)
#define SCFA_K_PAD 1000000000

/* Row padding of compacted/sorted buffers and the tile sizes of the
 * attention kernels (query tile SCFA_TILE_M rows, key tile SCFA_TILE_N). */
#define SCFA_ROW_ALIGN 128
#define SCFA_PAD(n) ((((n) + SCFA_ROW_ALIGN - 1) / SCFA_ROW_ALIGN) * SCFA_ROW_ALIGN)
#define SCFA_TILE_M 128
#define SCFA_TILE_N 64
#define SCFA_COUNT_CHUNK 64 /* positions per chunk of scfa_qk_count */

/* Human-readable text of a status code (static storage, never NULL). */
const char* scfa_status_string(int status);

/* Library ABI version (major*100 + minor). */
int scfa_version(void);

/* ------------------------------------------------------------------------
 * QK-drop preprocessing.
 * SCFA explainer, 3.4 "QK-Sparse Attention: Compaction and Index-Guided
 * Tiling", compaction step: per head the kept tokens are counted, kept in
 * position order (stable), gathered to the front and the index is padded.
 * ---------------------------------------------------------------------- */

/* Count kept tokens per head.
 *  keep          (B, T, H) uint8, nonzero = kept.
 *  count         out (B, H) int32: kept tokens of head (b, h).
 *  max_count     out (1) int32: max over all heads (read it back to size Tc).
 *  chunk_offsets out (B, H, ceil(T/64)) int32: kept tokens of head (b, h)
 *                before chunk c (positions [64c, 64c+64)) -- an exclusive
 *                prefix sum; input of scfa_qk_compact.                     */
int scfa_qk_count(const uint8_t* keep, int B, int T, int H, int32_t* count, int32_t* max_count,
                  int32_t* chunk_offsets, hipStream_t stream);

/* Compact one tensor. For r < count[b,h]: idx_c[b,h,r] = position of the
 * r-th kept token, x_c row r = x[b, idx_c[b,h,r], h, :] bit for bit. For
 * count <= r < Tc: idx_c = pad_idx and the row is zero.
 *  dtype         SCFA_BF16 / SCFA_F32 (element size of x and x_c).
 *  x             (B, T, H, D); may be NULL only if x_c is NULL.
 *  keep, count, chunk_offsets   as produced by scfa_qk_count on this keep.
 *  Tc            compacted length, a multiple of SCFA_ROW_ALIGN, >= max count
 *                (a head with more kept tokens sets COUNT_EXCEEDS_TC).
 *  pad_idx       SCFA_Q_PAD for queries, SCFA_K_PAD for keys.
 *  x_c           out (B, H, Tc, D) or NULL (index only).
 *  idx_c         out (B, H, Tc) int32.                                     */
int scfa_qk_compact(int dtype, const void* x, const uint8_t* keep, const int32_t* count,
                    const int32_t* chunk_offsets, int B, int T, int H, int D, int Tc, int32_t pad_idx,
                    void* x_c, int32_t* idx_c, int32_t* dev_err, hipStream_t stream);

/* The index compaction of the queries and of the keys, two launches for
 * both sides (grid dimension z selects the side): counts, max counts and
 * index arrays bit for bit as scfa_qk_count on keep_q and on keep_k
 * followed by scfa_qk_compact with x = x_c = NULL (index only), pad_idx
 * SCFA_Q_PAD for the queries and SCFA_K_PAD for the keys. Same definition
 * and citation. The second launch sums the chunk counts before each chunk
 * itself, so no prefix-sum array is written.
 *  keep_q (B, T, H), keep_k (B, T_kv, H) uint8, nonzero = kept.
 *  Tq, Tk            compacted lengths of the two sides (multiples of
 *                    SCFA_ROW_ALIGN, each >= its side's max count).
 *  count_q, count_k  out (B, H) int32.
 *  max_count         out (2) int32: max over heads of the query side, then
 *                    of the key side.
 *  chunk_counts_q    workspace (B, H, ceil(T/64)) int32, chunk_counts_k
 *                    (B, H, ceil(T_kv/64)): kept tokens per 64-position
 *                    chunk (left there on return).
 *  q_idx, k_idx      out (B, H, Tq), (B, H, Tk) int32.
 *  qstats, kstats, tiles
 *                    optional (all three or none): out (B, H, Tq/SCFA_TILE_M,
 *                    4), (B, H, Tk/SCFA_TILE_N, 4) and (B, H) -- the tile
 *                    statistics and zeroed processed-tile count that
 *                    scfa_range_table(SCFA_QK, q_idx, k_idx, ..., Tq, Tk,
 *                    SCFA_TILE_M, SCFA_TILE_N, ...) computes over these index
 *                    arrays (every row, pads included), bit for bit, for
 *                    scfa_fwd_table_order to take next.
 *  dev_err           as scfa_qk_compact (may be NULL).                      */
int scfa_qk_index_qk(const uint8_t* keep_q, const uint8_t* keep_k, int B, int T, int T_kv, int H, int Tq, int Tk,
                     int32_t* count_q, int32_t* count_k, int32_t* max_count, int32_t* chunk_counts_q,
                     int32_t* chunk_counts_k, int32_t* q_idx, int32_t* k_idx, int32_t* qstats, int32_t* kstats,
                     int32_t* tiles, int32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Hash-sparse preprocessing.
 * SCFA explainer, 3.4 "Hash-Sparse Attention: Sorting by Bucket and
 * Two-Dimensional Tiling": Reformer-style angular LSH buckets, a stable
 * per-head sort by bucket, and a gather into the sorted order.
 * ---------------------------------------------------------------------- */

/* LSH bucket of every token: c_j = sum_d x[b,t,h,d] * R[h,d,j] for
 * j < nb/2, accumulated in float64 in the order d = 0..D-1; bucket = the
 * first index of the maximum of [c ; -c].
 *  x       (B, T, H, D) bf16/fp32;  R (H, D, nb/2) fp32;  nb even, 2..64.
 *  bucket  out (B, H, T) int32 in [0, nb).                                  */
int scfa_hash_bucket(int dtype, const void* x, const float* R, int B, int T, int H, int D, int nb,
                     int32_t* bucket, hipStream_t stream);

/* scfa_hash_bucket plus the chunk histogram of the stable sort:
 *  chunk_counts  out (B, H, ceil(T / 256), nb) int32, the number of tokens
 *                of each bucket among positions [256 c, 256 c + 256) of each
 *                head (input of scfa_hash_layout).                          */
int scfa_hash_bucket_counts(int dtype, const void* x, const float* R, int B, int T, int H, int D, int nb,
                            int32_t* bucket, int32_t* chunk_counts, hipStream_t stream);

/* scfa_hash_bucket_counts of the queries and of the keys in one launch (the
 * two share R; grid dimension z selects the side): the same outputs, bit for
 * bit, as two calls. Same definition and citation.
 *  q, k                (B, T, H, D) of one dtype, device: one length T for
 *                      both (queries and keys of different lengths take
 *                      scfa_hash_bucket_counts per side, or
 *                      scfa_hash_bucket_counts_drop per side with keep
 *                      masks).
 *  keep_q, keep_k      optional (B, T, H) uint8 keep masks, both or neither:
 *                      hashing combined with within-bucket dropping (the SCFA
 *                      explainer's follow-up idea of a mask that is both
 *                      hash-based and drop-based). A dropped query takes
 *                      bucket nb and a dropped key bucket nb + 1, which match
 *                      nothing, so the rest of the hash path (sort and layout
 *                      with nb + 2 buckets, tables, attention, backward) runs
 *                      unchanged: dropped queries output zero with LSE -inf,
 *                      dropped keys are seen by no query. nb <= 62.
 *  bucket_q, bucket_k  out (B, H, T) int32.
 *  counts_q, counts_k  out chunk counts as in scfa_hash_bucket_counts, with
 *                      nb + 2 buckets per chunk when keep masks are given.
 * Argument errors as scfa_hash_bucket_counts (any NULL pointer other than
 * the keep masks, or only one keep mask: INVALID). */
int scfa_hash_bucket_qk(int dtype, const void* q, const void* k, const float* R, const uint8_t* keep_q,
                        const uint8_t* keep_k, int B, int T, int H, int D, int nb, int32_t* bucket_q, int32_t* bucket_k,
                        int32_t* counts_q, int32_t* counts_k, hipStream_t stream);

/* One side of scfa_hash_bucket_qk with its keep mask, for queries and keys of
 * different lengths (the SCFA explainer's decision tensors have lengths T_Q
 * and T_KV) combined with within-bucket dropping: the explainer's follow-up
 * idea of a mask that is both hash-based and drop-based. Kept tokens take
 * the scfa_hash_bucket bucket; a dropped token takes bucket nb + side, which
 * matches nothing on the other side. Bit for bit the same bucket and counts
 * as the corresponding side of scfa_hash_bucket_qk when the lengths agree.
 *  x             (B, T, H, D) bf16 or fp32, device: the queries (side 0) or
 *                the keys (side 1), T their own length.
 *  keep          (B, T, H) uint8, device, nonzero = kept; required.
 *  side          0 (queries: dropped -> nb) or 1 (keys: dropped -> nb + 1).
 *  bucket        out (B, H, T) int32.
 *  chunk_counts  out (B, H, ceil(T / 256), nb + 2) int32 (input of
 *                scfa_hash_layout with nb + 2 buckets).
 * Errors: NULL pointer, side not 0 or 1, bad sizes -> SCFA_ERR_INVALID;
 * D != 64 or nb > 62 -> SCFA_ERR_UNSUPPORTED. Asynchronous on `stream`. */
int scfa_hash_bucket_counts_drop(int dtype, const void* x, const float* R, const uint8_t* keep, int side, int B, int T,
                                 int H, int D, int nb, int32_t* bucket, int32_t* chunk_counts, hipStream_t stream);

/* Bytes of device workspace scfa_hash_sort needs. */
size_t scfa_hash_sort_workspace_bytes(int B, int H, int T, int nb);

/* Stable counting sort of each head's tokens by bucket.
 *  bucket        (B, H, T) int32 in [0, nb).
 *  perm          out (B, H, SCFA_PAD(T)): original positions ordered by
 *                (bucket, position); entries >= T hold pad_idx.
 *  bucket_sorted out (B, H, SCFA_PAD(T)): bucket[perm]; entries >= T hold -1.
 *  offsets       out (B, H, nb+1): offsets[v] = tokens with bucket < v.
 *  pad_idx       SCFA_Q_PAD when sorting queries, SCFA_K_PAD for keys.
 *  workspace     device scratch of scfa_hash_sort_workspace_bytes() bytes.  */
int scfa_hash_sort(const int32_t* bucket, int B, int H, int T, int nb, int32_t pad_idx, int32_t* perm,
                   int32_t* bucket_sorted, int32_t* offsets, void* workspace, size_t workspace_bytes,
                   int32_t* dev_err, hipStream_t stream);

/* Bucket-aligned layout of a sorted head. Same rows in the same order as
 * the stable sort, with pad rows inserted so that every bucket starts at a
 * multiple of `align`: tiles of `align` rows (the attention tiles) never hold
 * two buckets. This is a storage layout of the sorted order of "Hash-Sparse
 * Attention: Sorting by Bucket and Two-Dimensional Tiling" (SCFA explainer,
 * 3.4); it changes no result.
 *  perm, offsets  from scfa_hash_sort (perm has SCFA_PAD(T) rows per head).
 *  align          16, 32, 64 or 128.
 *  Tseg           rows per head of the outputs, a multiple of SCFA_ROW_ALIGN;
 *                 scfa_hash_segment_rows(T, nb, align) always suffices (a
 *                 smaller Tseg that a head overflows sets SEGMENT_OVERFLOW).
 *  idx_seg out (B, H, Tseg): bucket v's rows start at A_v = sum over u < v of
 *                 ceil(n_u / align) * align and hold perm[offsets[v] + r];
 *                 the rest of each segment holds pad_idx; rows from A_nb on
 *                 hold pad_idx.
 *  bkt_seg out (B, H, Tseg): v on the rows of segment v (pads included), nb
 *                 on the rows from A_nb on.
 *  seg_offsets out (B, H, nb+1) int32: A.                                    */
int scfa_hash_segment_rows(int T, int nb, int align);

int scfa_hash_segments(const int32_t* perm, const int32_t* offsets, int B, int H, int T, int nb, int align,
                       int32_t pad_idx, int Tseg, int32_t* idx_seg, int32_t* bkt_seg, int32_t* seg_offsets,
                       int32_t* dev_err, hipStream_t stream);

/* Sort and bucket-aligned layout in one launch, from the chunk counts of
 * scfa_hash_bucket_counts: the outputs of scfa_hash_sort followed by
 * scfa_hash_segments (same definitions, same bits). The explainer's hash
 * preprocessing (3.4, "Hash-Sparse Attention: Sorting by Bucket and
 * Two-Dimensional Tiling").
 *  bucket, nb, pad_idx, perm, bucket_sorted, offsets   as scfa_hash_sort.
 *  chunk_counts   (B, H, ceil(T / 256), nb): tokens of each bucket among
 *                 positions [256 c, 256 c + 256) of each head.
 *  align          0 (sort only: idx_seg, bkt_seg, seg_offsets unused and may
 *                 be NULL) or 16, 32, 64, 128 (as scfa_hash_segments).
 *  Tseg, idx_seg, bkt_seg, seg_offsets                 as scfa_hash_segments.
 * Data errors: BUCKET_RANGE (such tokens are left out), SEGMENT_OVERFLOW.  */
int scfa_hash_layout(const int32_t* bucket, const int32_t* chunk_counts, int B, int H, int T, int nb, int align,
                     int32_t pad_idx, int Tseg, int32_t* perm, int32_t* bucket_sorted, int32_t* offsets,
                     int32_t* idx_seg, int32_t* bkt_seg, int32_t* seg_offsets, int32_t* dev_err, hipStream_t stream);

/* scfa_hash_layout of both sides in one launch (grid dimension z selects the
 * side), with the attention's tiles: queries with align = SCFA_TILE_M and
 * pad_idx = SCFA_Q_PAD into Tseg_q rows per head, keys with align =
 * SCFA_TILE_N and pad_idx = SCFA_K_PAD into Tseg_k rows. The same outputs,
 * bit for bit, as the two calls; the same citation.
 *  *_q / *_k      the arguments of scfa_hash_layout for that side (every
 *                 pointer required); both sides have T tokens (different
 *                 lengths take scfa_hash_layout per side).
 *  qstats, kstats optional (both with tiles, or all three NULL): the tile
 *                 statistics of the two aligned layouts, (B, H, Tseg_q /
 *                 SCFA_TILE_M, 4) and (B, H, Tseg_k / SCFA_TILE_N, 4), the
 *                 same values scfa_range_table computes from idx_q, bkt_q,
 *                 idx_k, bkt_k in SCFA_HASH mode ("Kernel tiling logic for
 *                 Hash-sparse (Algorithm 2)" extrema), written by the threads
 *                 that place each tile's first and last token.
 *  tiles          (B*H) int32: set to 0, ready for scfa_fwd_table.
 *  dev_err        shared by both sides (may be NULL).
 * Argument errors as scfa_hash_layout; data errors of either side are OR-ed
 * into dev_err. */
int scfa_hash_layout_qk(const int32_t* bucket_q, const int32_t* bucket_k, const int32_t* counts_q,
                        const int32_t* counts_k, int B, int H, int T, int nb, int Tseg_q, int Tseg_k, int32_t* perm_q,
                        int32_t* perm_k, int32_t* bsorted_q, int32_t* bsorted_k, int32_t* offsets_q,
                        int32_t* offsets_k, int32_t* idx_q, int32_t* idx_k, int32_t* bkt_q, int32_t* bkt_k,
                        int32_t* seg_q, int32_t* seg_k, int32_t* qstats, int32_t* kstats, int32_t* tiles,
                        int32_t* dev_err, hipStream_t stream);

/* Gather rows into head-major order: out row r of head (b, h) is
 * x[b, idx[b,h,r], h, :] when 0 <= idx < T, else zero.
 *  layout  SCFA_ROWS -> x_p (B, H, Tp, D);  SCFA_COLS -> x_p (B, H, D, Tp).
 *  idx     (B, H, Tp) int32; Tp a multiple of SCFA_ROW_ALIGN.               */
int scfa_gather(int dtype, int layout, const void* x, const int32_t* idx, int B, int T, int H, int D, int Tp,
                void* x_p, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Tile range / skip table.
 * SCFA explainer, 3.4: "Kernel tiling logic (Algorithm 1)" (QK: key tiles
 * [0, end), end = number of key tiles whose smallest position is <= the
 * query tile's largest position); "Kernel tiling logic for Hash-sparse
 * (Algorithm 2)" (start skips key tiles whose largest bucket is below the
 * query tile's smallest bucket; the stop is the first tile whose smallest
 * bucket exceeds the query tile's largest, refined to one past the last tile
 * passing the causal extremum test); "Backward Pass Design" (per key tile,
 * the range of query tiles); "Design Choices" item 4 (dense = QK rule on
 * positions 0..T-1).
 *
 * A tile pair (i, j) is PROCESSED iff j is in fwd range of i and
 * kstats[j].minpos <= qstats[i].maxpos (minpos + 1 with SCFA_STRICT; with
 * SCFA_NONCAUSAL: tile i holds a real query and tile j a real key). bwd
 * range of j = [min, max+1) of the processed i (or [0, 0)).
 *  mode          SCFA_DENSE (q_idx, k_idx ignored, may be NULL), SCFA_QK,
 *                SCFA_HASH (q_bkt, k_bkt required); OR-ed with at most one
 *                of SCFA_STRICT, SCFA_NONCAUSAL.
 *  q_idx, q_bkt  (B, H, SCFA_PAD(Tq)); k_idx, k_bkt (B, H, SCFA_PAD(Tk)).
 *  Tq, Tk        valid rows (extrema are taken over rows < Tq / < Tk).
 *  Bm, Bn        tile sizes, each 16, 32, 64 or 128. The attention kernels
 *                require Bm = SCFA_TILE_M, Bn = SCFA_TILE_N.
 *  qstats out (B, H, nQt, 4), nQt = SCFA_PAD(Tq)/Bm:
 *                [min pos, max pos, min bucket, max bucket] (buckets 0 unless
 *                hash).
 *  kstats out (B, H, nKt, 4), nKt = SCFA_PAD(Tk)/Bn; a tile with no valid
 *                row holds [K_PAD, K_PAD, INT32_MAX, INT32_MAX].
 *  fwd_tab out (B, H, nQt, 2) [start, end), or NULL (then bwd_tab must be
 *                NULL too) for the statistics alone, with tiles zeroed:
 *                scfa_fwd_table_order then builds the ranges and the order.
 *  bwd_tab out (B, H, nKt, 2), or NULL to skip it (a forward-only call;
 *                scfa_bwd_table builds it later from the same statistics).
 *  tiles   out (B, H) int32: number of processed tile pairs.               */
int scfa_range_table(int mode, const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt,
                     const int32_t* k_bkt, int B, int H, int Tq, int Tk, int Bm, int Bn, int32_t* qstats,
                     int32_t* kstats, int32_t* fwd_tab, int32_t* bwd_tab, int32_t* tiles, hipStream_t stream);

/* The backward table alone, from the statistics and forward table of a
 * scfa_range_table call (nQt, nKt as there): the same bwd_tab. flags: the
 * SCFA_STRICT / SCFA_NONCAUSAL bit of that call (0 for none).             */
int scfa_bwd_table(const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, int B, int H, int nQt, int nKt,
                   int32_t* bwd_tab, int flags, hipStream_t stream);

/* The forward range table from tile statistics: the second half of
 * scfa_range_table (same rules, same citation), for statistics that another
 * call produced (scfa_hash_layout_qk).
 *  qstats, kstats  (B, H, nQt, 4), (B, H, nKt, 4) as scfa_range_table's.
 *  fwd_tab         out (B, H, nQt, 2).
 *  tiles           (B*H) int32, zero on entry: the processed-tile count is
 *                  added to it. */
int scfa_fwd_table(int mode, const int32_t* qstats, const int32_t* kstats, int B, int H, int nQt, int nKt,
                   int32_t* fwd_tab, int32_t* tiles, hipStream_t stream);

/* Launch order of the attention workgroups for one range table (the
 * forward table for the forward and dQ kernels, the backward table for the
 * dK/dV kernel): the B*H*ntiles items (item = (b*H + h)*ntiles + tile) sorted
 * by range length (end - start), longest first, so that the longest tiles
 * start first and the short ones fill the tail. The items are sorted within
 * G groups of heads (head bh in group bh % G) and interleaved,
 * order[slot*G + g]: G = 8 when B*H is a multiple of 8 (workgroup x runs on
 * XCD x % 8, so each XCD keeps to its own heads and their K/V tiles stay in
 * its L2), else the largest divisor of B*H not above 8 (one workgroup builds
 * each group). Items of equal length come in an unspecified order.
 *  tab     (B, H, ntiles, 2) [start, end) range table.
 *  ntiles  >= 1, tiles per head the table describes.
 *  span    1..16383, tiles per head its ranges index (key tiles for the
 *          forward table, query tiles for the backward table); lengths
 *          are clamped to [0, span].
 *  order   out (B*H*ntiles) int32, a permutation of the items.             */
int scfa_work_order(const int32_t* tab, int B, int H, int ntiles, int span, int32_t* order, hipStream_t stream);

/* The backward table and the launch order of the dK/dV workgroups in one
 * call: the results of scfa_bwd_table followed by scfa_work_order(bwd_tab,
 * ..., ntiles = nKt, span = nQt, ...), for the backward kernels' tile
 * ranges of the SCFA explainer, 3.4 "Backward Pass Design" (the same ranges
 * with queries and keys swapped). One launch: the group's forward ranges and
 * query extrema are held in LDS, and where a head's forward starts and ends
 * are both non-decreasing (the aligned hash layout, the QK and dense modes)
 * the query tiles whose range holds a key tile are found by two binary
 * searches; other tables are scanned tile by tile with the same rule, so any
 * table gives scfa_bwd_table's result. Groups too large for LDS fall back to
 * the two separate launches.
 *  qstats, kstats, fwd_tab   as for scfa_bwd_table.
 *  bwd_tab         out (B, H, nKt, 2).
 *  order           out (B*H*nKt) int32, sorted as scfa_work_order (items of
 *                  equal length in an unspecified order); when B*H is not a
 *                  multiple of 8, in the 8 runs of consecutive items that
 *                  scfa_fwd_table_order uses in SCFA_HASH mode (slot s of run
 *                  k at order[s*8 + k]); problems too large for one workgroup
 *                  per group or run take the two launches and
 *                  scfa_work_order's groups.
 *  nQt             1..16383.
 *  flags           the SCFA_STRICT / SCFA_NONCAUSAL bit of the tables (0
 *                  for none).                                             */
int scfa_bwd_table_order(const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, int B, int H, int nQt,
                         int nKt, int32_t* bwd_tab, int32_t* order, int flags, hipStream_t stream);

/* The forward range table and its launch order in one call: the results of
 * scfa_fwd_table followed by scfa_work_order(fwd_tab, ..., span = nKt, ...).
 * One launch: the group's key-tile statistics are held in LDS, and where a
 * head's key tiles are in layout order (one bucket per tile, buckets and,
 * within a bucket, smallest positions non-decreasing: the hash layout of
 * scfa_hash_layout_qk, and the compacted or dense rows of the QK and dense
 * modes) the range rules (explainer 3.4, Algorithms 1 and 2) become binary
 * searches; other statistics are scanned tile by tile with the same rules,
 * so any statistics give scfa_fwd_table's table. Groups too large for LDS
 * fall back to the two separate launches.
 *  mode            SCFA_DENSE, SCFA_QK or SCFA_HASH, optionally OR-ed with
 *                  SCFA_STRICT or SCFA_NONCAUSAL.
 *  qstats, kstats  (B, H, nQt, 4), (B, H, nKt, 4).
 *  fwd_tab         out (B, H, nQt, 2).
 *  tiles           (B*H) int32, zero on entry: the processed-tile count is
 *                  added to it.
 *  order           out (B*H*nQt) int32: the items sorted by range length,
 *                  longest first, as scfa_work_order (items of equal length
 *                  in an unspecified order), in scfa_work_order's groups of
 *                  heads, except in SCFA_HASH mode when B*H is not a
 *                  multiple of 8: then the N = B*H*nQt items (head-major)
 *                  form 8 runs of consecutive items of equal count (the
 *                  first N % 8 runs one item longer), each sorted on its
 *                  own, with slot s of run k at order[s*8 + k], so that each
 *                  XCD (workgroup x runs on XCD x % 8) works on about B*H/8
 *                  heads. Problems too large for one workgroup per run take
 *                  the two launches and scfa_work_order's groups.
 *  nKt             1..16383.                                              */
int scfa_fwd_table_order(int mode, const int32_t* qstats, const int32_t* kstats, int B, int H, int nQt, int nKt,
                         int32_t* fwd_tab, int32_t* tiles, int32_t* order, hipStream_t stream);

/* Exact number of visible (query, key) pairs per head, from the sorted /
 * compacted index arrays (a query row r < Tq with position p >= 0 sees the
 * key rows s < Tk with k_idx[s] <= p, and equal bucket in hash mode; the
 * mode may carry SCFA_STRICT, k_idx[s] < p, or SCFA_NONCAUSAL, every key row
 * with a real position).
 *  pairs out (B, H) int64.                                                  */
int scfa_count_visible(int mode, const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt,
                       const int32_t* k_bkt, int B, int H, int Tq, int Tk, int64_t* pairs, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Forward attention.
 * SCFA explainer, 3.4 "Kernel tiling logic (Algorithm 1)" / "(Algorithm 2)"
 * and "Softmax Statistics Accumulation with NaN Safety" (Algorithm 3);
 * "3.2 Big-Picture Architecture" item 4 (outputs scattered back to original
 * positions, dropped queries get a zero vector).
 *
 * For every query the output is softmax-weighted V over the VISIBLE keys:
 * key visible iff k_pos <= q_pos (QK), and same bucket (hash); scores are
 * scale * q.k. A query with no visible key -- and, in QK mode, a dropped
 * query -- gets O = 0 and LSE = -inf.
 *  flags         0, SCFA_STRICT (k_pos < q_pos) or SCFA_NONCAUSAL (no
 *                position test); the tables must have been built with the
 *                same flag.
 *  dtype_in      SCFA_BF16 / SCFA_F32 of q, k, v.
 *  dtype_out     SCFA_F32 / SCFA_BF16 of O.
 *  q             (B, T, H, D) and k, v (B, T_kv, H, D): the ORIGINAL,
 *                unpermuted tensors (D = 64). The gather of the
 *                preprocessing is fused into the loads: row r of a head
 *                reads token q_idx[r] of q (k_idx[r] of k and v); pad
 *                entries (any index outside [0, T) / [0, T_kv)) read token
 *                0, whose values must be finite.
 *  q_idx, k_idx  (B, H, Tpad) original positions with pads.
 *  q_bkt, k_bkt  (B, H, Tpad) sorted bucket ids (hash only).
 *  qstats, kstats, fwd_tab   from scfa_range_table with Bm = SCFA_TILE_M,
 *                Bn = SCFA_TILE_N, same mode and arrays.
 *  order         (B*H*nQt) launch order from scfa_work_order on fwd_tab, or
 *                NULL (then query tiles run in descending index order). Any
 *                permutation gives the same results; only the schedule moves.
 *  T             original query length (rows of O and LSE).
 *  T_kv          original key/value length; T_kv != T follows the
 *                explainer's separate decision-tensor lengths T_Q and T_KV
 *                ("QK-Sparse Attention: Compaction and Index-Guided
 *                Tiling"): query and key positions both count from 0 and the
 *                position test compares them unchanged.
 *  Tc            QK: compacted length (multiple of 128); Tpad = Tc.
 *  scale         score scale, normally 1/sqrt(D).
 *  O             out (B, T, H, D), every row written.
 *  lse           out (B, H, T) fp32 natural-log normaliser, every entry
 *                written (-inf for rows without a visible key).           */
int scfa_qk_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v,
                       const int32_t* q_idx, const int32_t* k_idx, const int32_t* qstats, const int32_t* kstats,
                       const int32_t* fwd_tab, const int32_t* order, int B, int H, int T, int T_kv, int Tc, int D,
                       float scale, int flags, void* O, float* lse, hipStream_t stream);

/* Hash-sparse: as above, with the sorted (or bucket-aligned) index arrays
 * and
 *  q_bkt, k_bkt  sorted bucket ids of the rows;
 *  Tq, Tk        query / key rows as passed to scfa_range_table (T for the
 *                sorted order, Tseg for the bucket-aligned layout); the
 *                index arrays hold SCFA_PAD(Tq) / SCFA_PAD(Tk) rows per head. */
int scfa_hash_sparse_fwd(int dtype_in, int dtype_out, const void* q, const void* k, const void* v,
                         const int32_t* q_idx, const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt,
                         const int32_t* qstats, const int32_t* kstats, const int32_t* fwd_tab, const int32_t* order,
                         int B, int H, int T, int T_kv, int Tq, int Tk, int D, float scale, int flags, void* O,
                         float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward attention (recomputation from the saved LSE).
 * SCFA explainer, 3.4 "Backward Pass Design": score tiles are recomputed
 * with the same index-guided tile ranges and local masks (queries and keys
 * swapped for dK/dV), and the same -inf guard as the forward: a query with
 * LSE = -inf contributes nothing. With P = exp(scale q.k - LSE) on visible
 * pairs: dV = P^T dO, dS = P (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 * dK = scale dS^T Q. Keep masks and buckets are constants.
 *
 *  mode          SCFA_QK (also dense: QK rule on positions 0..T-1) or
 *                SCFA_HASH, OR-ed with the forward call's SCFA_STRICT or
 *                SCFA_NONCAUSAL.
 *  dtype_in      SCFA_BF16 (the only backward build; fp32 returns
 *                SCFA_ERR_UNSUPPORTED).
 *  q             (B, T, H, D), k, v (B, T_kv, H, D): the original tensors
 *                of the forward call, read through q_idx / k_idx like the
 *                forward (pad entries read token 0).
 *  q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab
 *                exactly the index arrays and tables of the forward call.
 *  bwd_tab       the backward table of the same call (scfa_range_table or
 *                scfa_bwd_table).
 *  fwd_order     launch order of the dQ workgroups: scfa_work_order or
 *                scfa_fwd_table_order on fwd_tab (the forward call's
 *                order), or NULL (then query tiles run in descending index
 *                order).
 *  bwd_order     launch order of the dK/dV workgroups of the hash mode (one
 *                workgroup per key tile): scfa_work_order on bwd_tab with
 *                span = query tiles per head, or the order of
 *                scfa_bwd_table_order, or NULL (key tiles in index order). QK mode runs pairs of key tiles in index order
 *                and does not read it. Any permutation gives the same
 *                results; only the schedule moves.
 *  O             (B, T, H, D) fp32 forward output;  lse (B, H, T) fp32.
 *  dO            (B, T, H, D) upstream gradient, dtype_in.
 *  T, T_kv       original query and key/value lengths, as in the forward;
 *  Tq, Tk        query / key rows as
 *                passed to scfa_range_table (Tc and Tc for QK; T and T for the
 *                sorted hash order, Tseg_q and Tseg_k for the bucket-aligned
 *                layout); the buffers hold SCFA_PAD(Tq) / SCFA_PAD(Tk) rows.
 *  dQ            out (B, T, H, D), dK, dV out (B, T_kv, H, D): fp32 in
 *                original order, every row
 *                written (zero for dropped tokens and tokens without any
 *                visible pair).
 *  workspace     device scratch of scfa_bwd_workspace_bytes() bytes (Delta
 *                and log2 LSE per sorted query row).
 * Launches 2 kernels on `stream` (dQ, which also fills the workspace,
 * then dK/dV); no atomics, results are deterministic.                      */
size_t scfa_bwd_workspace_bytes(int mode, int B, int H, int Tq, int Tk, int D);

int scfa_bwd(int mode, int dtype_in, const void* q, const void* k, const void* v, const int32_t* q_idx,
             const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
             const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const int32_t* fwd_order,
             const int32_t* bwd_order, const float* O, const float* lse, const void* dO, int B, int H, int T, int T_kv,
             int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc). Same arguments, kernels and
 * results as scfa_bwd, bit for bit; the workspace (log2 LSE and Delta per
 * sorted query row, 8 bytes per row of B * H * SCFA_PAD(Tq)) lives in a
 * static device array of SCFA_NOALLOC_SCRATCH_BYTES that each device holds
 * for the life of the process. The call allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine.
 *  stream        must belong to the current device (else
 *                SCFA_ERR_INVALID); the first call on a device looks the
 *                array's address up on that device.
 * Errors: as scfa_bwd; a problem whose workspace exceeds the array
 * (B * H * SCFA_PAD(Tq) above about 2 million rows) -> SCFA_ERR_TOO_LARGE,
 * before anything is enqueued.
 * Every call on one device shares that device's array: calls that overlap
 * in time on one device (two streams, or two host threads) race and give
 * wrong gradients; calls in one stream order are safe. The array keeps the
 * last call's contents; every row a call reads it writes first, so nothing
 * needs clearing. */
#define SCFA_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)

int scfa_bwd_noalloc(int mode, int dtype_in, const void* q, const void* k, const void* v, const int32_t* q_idx,
                     const int32_t* k_idx, const int32_t* q_bkt, const int32_t* k_bkt, const int32_t* qstats,
                     const int32_t* kstats, const int32_t* fwd_tab, const int32_t* bwd_tab, const int32_t* fwd_order,
                     const int32_t* bwd_order, const float* O, const float* lse, const void* dO, int B, int H, int T,
                     int T_kv, int Tq, int Tk, int D, float scale, float* dQ, float* dK, float* dV, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SCFA_H_ */
