"""CPU oracle for Sparse Causal Flash Attention (SCFA).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: it exists so that tests, the smoke check and the benchmark's CPU
baseline can check the HIP path against a plain, slow, obviously correct
definition. It shares no code with the HIP path and imports nothing from it.

Source of every definition: the explainer page "Faster Causal Attention Over
Large Sequences Through Sparse Flash Attention" (arXiv 2306.01160),
hereafter "the SCFA explainer", sections named per function below.

Arithmetic: float64 throughout. Floating-point inputs are the exact values the
GPU sees (bf16 or fp32), widened to float64 by the caller. Attention is an
explicit masked softmax over whole rows in ORIGINAL token order (no tiling, no
online rescaling). Integer steps (compaction, LSH bucket, sort, tile tables)
are written from their definitions with scalar-order numpy operations.

Readings of points the pages leave open (each one is also listed in the design doc):
  * keep_p is the probability of KEEPING a token.
  * A query with no visible key, and a dropped query, outputs the zero vector
    and LSE = -inf.
  * LSE is the natural-log normaliser  ln sum_visible exp(tau * q.k).
  * Compaction pads: index -1 for queries, 1_000_000_000 for keys; padded rows
    of the compacted tensors are zero.
  * LSH: c_j = sum_d x_d R_dj accumulated in float64 in the order d = 0..D-1,
    each product and each sum separately rounded; bucket = first index of the
    maximum of [c ; -c].
  * Sort key: (bucket ascending, position ascending).
  * strict=True (every attention function): the explainer's '>' variant of
    the causal test, a key strictly before the query; a query then never
    sees itself, and the first token of a sequence sees nothing.
  * noncausal=True: no position test (bidirectional attention over the
    kept / same-bucket tokens); a tile holds a visible pair iff it holds a
    real key (position below the key pad).
  * Separate query and key lengths (the explainer's decision tensors of
    lengths T_Q and T_KV): queries at positions 0..T_Q-1, keys at
    0..T_KV-1, compared unchanged by the causal test. With T_KV > T_Q the
    keys after the last query are never visible (unless noncausal); with
    T_Q > T_KV the queries at T_KV and beyond see every key.
  * Hashing combined with within-bucket dropping (the explainer's follow-up
    idea): in hash mode with keep masks a pair is visible iff both tokens
    share a bucket, both are kept and the key does not come after the query.
  * Tile tables: see range_tables().

Pins: every function here is checked by tests/test_oracle_*.py against brute
force, closed forms, invariants, library routines or numbers the pages print
(the FLOP counts flops_fwd and flops_bwd against the teaching page's
per-product inventory). Parity pinned for all functions.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

Q_PAD = -1
K_PAD = 1_000_000_000
NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# QK-sparse preprocessing: compaction.
# SCFA explainer, 3.4 "QK-Sparse Attention: Compaction and Index-Guided
# Tiling", compaction step (count kept per head, stable order of the kept
# elements, gather, pad the index with sentinels).
# ---------------------------------------------------------------------------

def qk_count(keep: np.ndarray) -> np.ndarray:
    """Kept tokens per (b, h). keep: (B, T, H), nonzero = kept. -> (B, H) int32."""
    return (np.asarray(keep) != 0).sum(axis=1).astype(np.int32)


def qk_compact(x: Optional[np.ndarray], keep: np.ndarray, Tc: int, pad: int):
    """Compact the kept rows of each head to the front, in position order.

    x: (B, T, H, D) of any dtype (bit copies) or None; keep: (B, T, H).
    Returns (x_c (B, H, Tc, D) or None, idx (B, H, Tc) int32): for r < count,
    idx[r] is the r-th smallest kept position and x_c[r] = x[b, idx[r], h];
    for r >= count, idx[r] = pad and x_c[r] = 0.
    """
    keep = np.asarray(keep) != 0
    B, T, H = keep.shape
    idx = np.full((B, H, Tc), pad, dtype=np.int32)
    xc = None if x is None else np.zeros((B, H, Tc, x.shape[-1]), dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            pos = np.flatnonzero(keep[b, :, h])
            if len(pos) > Tc:
                raise ValueError("Tc is smaller than the kept count")
            idx[b, h, :len(pos)] = pos
            if xc is not None:
                xc[b, h, :len(pos)] = x[b, pos, h]
    return xc, idx


# ---------------------------------------------------------------------------
# Hash-sparse preprocessing.
# SCFA explainer, 3.4 "Hash-Sparse Attention: Sorting by Bucket and
# Two-Dimensional Tiling" (Reformer-style angular LSH; stable sort of the
# bucket ids per head; gather; original positions kept as q_idx/k_idx).
# ---------------------------------------------------------------------------

def hash_bucket(x: np.ndarray, R: np.ndarray, nb: int) -> np.ndarray:
    """Angular LSH bucket of every token.

    x: (B, T, H, D) float64 (exact widened input values); R: (H, D, nb/2)
    float64 (widened float32 rotations). -> (B, H, T) int32.
    c_j = (((0 + x_0 R_0j) + x_1 R_1j) + ...) in float64, every multiply and
    add a separate IEEE operation; bucket = argmax over [c_0..c_{nb/2-1},
    -c_0..-c_{nb/2-1}], smallest index on ties.
    """
    if nb % 2:
        raise ValueError("nb must be even")
    x = np.asarray(x, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    B, T, H, D = x.shape
    half = nb // 2
    c = np.zeros((B, T, H, half), dtype=np.float64)
    for d in range(D):
        prod = x[:, :, :, d:d + 1] * R[None, None, :, d, :]
        c = c + prod
    full = np.concatenate([c, -c], axis=-1)
    # np.argmax returns the first index of the maximum; -0.0 == +0.0.
    bucket = np.argmax(full, axis=-1).astype(np.int32)
    return np.ascontiguousarray(bucket.transpose(0, 2, 1))


def hash_sort(bucket: np.ndarray, nb: int):
    """Stable per-head sort of the tokens by bucket.

    bucket: (B, H, T) int. Returns perm (B, H, T) int32 (positions ordered by
    (bucket, position)), bucket_sorted (B, H, T) int32, offsets (B, H, nb+1)
    int32 with offsets[v] = number of tokens whose bucket < v.
    """
    bucket = np.asarray(bucket)
    B, H, T = bucket.shape
    perm = np.argsort(bucket, axis=-1, kind="stable").astype(np.int32)
    bsorted = np.take_along_axis(bucket, perm, axis=-1).astype(np.int32)
    offsets = np.zeros((B, H, nb + 1), dtype=np.int32)
    for v in range(nb + 1):
        offsets[:, :, v] = (bucket < v).sum(axis=-1)
    return perm, bsorted, offsets


def segment_rows(T: int, nb: int, align: int) -> int:
    """Rows of a bucket-aligned layout that any head of length T fits in:
    T real rows plus at most align - 1 pad rows per bucket, rounded up to a
    multiple of 128."""
    n = T + nb * (align - 1)
    return -(-n // 128) * 128


def hash_segments(perm: np.ndarray, offsets: np.ndarray, nb: int, align: int, pad: int, Tseg: int):
    """Bucket-aligned layout of a sorted head (a layout of the sorted order of
    the SCFA explainer, 3.4 "Hash-Sparse Attention: Sorting by Bucket and
    Two-Dimensional Tiling": it keeps every bucket's rows in sorted order and
    only inserts pad rows, so tiles of `align` rows never hold two buckets).

    perm: (B, H, >=T) sorted positions; offsets: (B, H, nb+1) from hash_sort.
    Bucket v starts at row A_v = sum_{u<v} ceil(n_u / align) * align, where
    n_u = offsets[u+1] - offsets[u]. Row A_v + r, r < n_v, holds
    perm[offsets[v] + r] with bucket v; rows A_v + n_v .. A_{v+1} - 1 hold
    `pad` with bucket v; rows A_nb .. Tseg - 1 hold `pad` with bucket nb.
    Returns idx (B, H, Tseg) int32, bkt (B, H, Tseg) int32, seg_off
    (B, H, nb+1) int32 = A.
    """
    B, H = offsets.shape[:2]
    idx = np.full((B, H, Tseg), pad, dtype=np.int32)
    bkt = np.full((B, H, Tseg), nb, dtype=np.int32)
    seg = np.zeros((B, H, nb + 1), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            a = 0
            for v in range(nb):
                lo, hi = int(offsets[b, h, v]), int(offsets[b, h, v + 1])
                n = hi - lo
                m = -(-n // align) * align
                if a + m > Tseg:
                    raise ValueError("Tseg too small")
                seg[b, h, v] = a
                idx[b, h, a:a + n] = perm[b, h, lo:hi]
                bkt[b, h, a:a + m] = v
                a += m
            seg[b, h, nb] = a
    return idx, bkt, seg


def gather_rows(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x: (B, T, H, D) any dtype; perm: (B, H, Tp). Row r of head (b,h) is
    x[b, perm[r], h] when 0 <= perm[r] < T, else a zero row. -> (B, H, Tp, D)."""
    B, T, H, D = x.shape
    Tp = perm.shape[-1]
    out = np.zeros((B, H, Tp, D), dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            p = perm[b, h]
            ok = (p >= 0) & (p < T)
            out[b, h, ok] = x[b, p[ok], h]
    return out


# ---------------------------------------------------------------------------
# Tile range / skip tables.
# SCFA explainer, 3.4: QK "Kernel tiling logic (Algorithm 1)" (end = number of
# key blocks whose smallest key index is <= the largest query index of the
# query block); Hash "Kernel tiling logic for Hash-sparse (Algorithm 2)"
# (start = blocks whose largest bucket is below the smallest query bucket,
# provisional stop at the first block whose smallest bucket exceeds the
# largest query bucket, then the stop refined by the causal extremum test);
# "Backward Pass Design" (the same extrema, roles of queries and keys swapped);
# "Design Choices" item 4 (dense: start = 0, stop = i + 1).
# ---------------------------------------------------------------------------

def tile_stats(pos: np.ndarray, bkt: Optional[np.ndarray], tile: int) -> np.ndarray:
    """Per-tile extrema over the rows that exist (r < len).

    pos: (B, H, Tp) int; bkt: (B, H, Tp) int or None (then buckets are 0).
    -> (B, H, ceil(Tp/tile), 4) int32: [min pos, max pos, min bucket, max bucket].
    Sentinel positions (pads) are included as ordinary values.
    """
    B, H, Tp = pos.shape
    n = -(-Tp // tile)
    st = np.zeros((B, H, n, 4), dtype=np.int64)
    for t in range(n):
        sl = slice(t * tile, min((t + 1) * tile, Tp))
        st[:, :, t, 0] = pos[:, :, sl].min(axis=-1)
        st[:, :, t, 1] = pos[:, :, sl].max(axis=-1)
        if bkt is not None:
            st[:, :, t, 2] = bkt[:, :, sl].min(axis=-1)
            st[:, :, t, 3] = bkt[:, :, sl].max(axis=-1)
    return st.astype(np.int32)


def range_tables(mode: str, q_idx: np.ndarray, k_idx: np.ndarray, q_bkt: Optional[np.ndarray],
                 k_bkt: Optional[np.ndarray], Bm: int, Bn: int, strict: bool = False,
                 noncausal: bool = False) -> dict:
    """Forward and backward tile ranges and the processed tile set.

    q_idx: (B, H, Tq), k_idx: (B, H, Tk) original positions (with pads);
    q_bkt/k_bkt: (B, H, Tq/Tk) sorted bucket ids (hash mode only).
    Dense mode ignores q_idx/k_idx contents and uses positions 0..T-1.

    Returns dict with
      qstats (B,H,nQt,4), kstats (B,H,nKt,4)  per-tile extrema (tile_stats);
      fwd    (B,H,nQt,2) [start, end) of key tiles per query tile;
      bwd    (B,H,nKt,2) [start, end) of query tiles per key tile;
      P      (B,H,nQt,nKt) bool, the processed tile set;
      tiles  (B,H) int32, |P|.
    A tile pair (i, j) is processed iff j lies in the forward range of i and
    kminpos_j <= qmaxpos_i (the causal extremum test; kminpos_j < qmaxpos_i
    with strict=True, the explainer's '>' variant). The backward range of
    key tile j is [min, max+1) of {i : (i, j) processed}, or [0, 0).
    """
    q_idx = np.asarray(q_idx)
    k_idx = np.asarray(k_idx)
    if mode == "dense":
        B, H, Tq = q_idx.shape
        Tk = k_idx.shape[-1]
        q_idx = np.broadcast_to(np.arange(Tq, dtype=np.int64), (B, H, Tq))
        k_idx = np.broadcast_to(np.arange(Tk, dtype=np.int64), (B, H, Tk))
    use_b = mode == "hash"
    qs = tile_stats(q_idx, q_bkt if use_b else None, Bm)
    ks = tile_stats(k_idx, k_bkt if use_b else None, Bn)
    B, H, nQt, _ = qs.shape
    nKt = ks.shape[2]
    sh = 1 if strict else 0

    def reach(kmin, qmax):
        """Tile-level position test. Causal: the key tile's smallest position
        (+1 when strict) does not exceed the query tile's largest. Without
        causality: the query tile holds a real query (largest position not
        the pad -1) and the key tile a real key (smallest below the pad)."""
        if noncausal:
            return (kmin < K_PAD) & (qmax >= 0)
        return kmin + sh <= qmax

    fwd = np.zeros((B, H, nQt, 2), dtype=np.int32)
    P = np.zeros((B, H, nQt, nKt), dtype=bool)
    for b in range(B):
        for h in range(H):
            kmin = ks[b, h, :, 0]
            for i in range(nQt):
                qmax = qs[b, h, i, 1]
                if mode in ("qk", "dense"):
                    # Algorithm 1: end = number of key tiles whose minimum
                    # position does not exceed the query tile's maximum.
                    start = 0
                    end = int(reach(kmin, qmax).sum())
                else:
                    qminb, qmaxb = qs[b, h, i, 2], qs[b, h, i, 3]
                    kminb, kmaxb = ks[b, h, :, 2], ks[b, h, :, 3]
                    # Algorithm 2: start skips tiles whose largest bucket is
                    # below the smallest query bucket.
                    start = int((kmaxb < qminb).sum())
                    # provisional stop: first tile at/after start whose
                    # smallest bucket exceeds the largest query bucket.
                    eh = start
                    while eh < nKt and not (kminb[eh] > qmaxb):
                        eh += 1
                    # refined stop: one past the last tile in [start, eh)
                    # that passes the causal extremum test.
                    end = start
                    for j in range(start, eh):
                        if reach(kmin[j], qmax):
                            end = j + 1
                fwd[b, h, i] = (start, end)
                for j in range(start, end):
                    if reach(kmin[j], qmax):
                        P[b, h, i, j] = True
    bwd = np.zeros((B, H, nKt, 2), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for j in range(nKt):
                ii = np.flatnonzero(P[b, h, :, j])
                if len(ii):
                    bwd[b, h, j] = (ii[0], ii[-1] + 1)
    return {"qstats": qs, "kstats": ks, "fwd": fwd, "bwd": bwd, "P": P,
            "tiles": P.sum(axis=(2, 3)).astype(np.int32)}


# ---------------------------------------------------------------------------
# Attention: visibility, forward, backward.
# Visibility: SCFA explainer 3.4 -- QK: a query attends to a key iff both are
# kept and q_idx >= k_idx (local mask of Algorithm 1); Hash: additionally the
# buckets are equal (combined mask of Algorithm 2); dense: the causal
# lower-triangular mask ("FlashAttention's Tiling Strategy").
# Scores: tau * q.k with tau = 1/sqrt(D) ("Hyperparameters and Implementation
# Constants"). Rows with no visible key output the zero vector ("Softmax
# Statistics Accumulation with NaN Safety"); dropped queries output the zero
# vector ("3.2 Big-Picture Architecture", item 4).
# ---------------------------------------------------------------------------

def _vis_rows(mode: str, rows: np.ndarray, T: int, kq, kk, bq, bk, strict: bool = False,
              noncausal: bool = False) -> np.ndarray:
    """Visibility of query rows `rows` (original positions) against all T keys
    of one head (strict: a key strictly before the query, the explainer's
    '>' variant of the causal test; noncausal: no position test at all, the
    bidirectional attention the explainer mentions as an extension).
    Returns (len(rows), T) bool."""
    j = np.arange(T)
    if noncausal:
        vis = np.ones((len(rows), T), dtype=bool)
    else:
        vis = (j[None, :] < rows[:, None]) if strict else (j[None, :] <= rows[:, None])
    if mode == "qk":
        vis &= (kq[rows] != 0)[:, None] & (kk != 0)[None, :]
    elif mode == "hash":
        vis &= bq[rows][:, None] == bk[None, :]
        # hashing combined with within-bucket dropping (the explainer's
        # follow-up, "Combined hashing and within-bucket dropping"): a pair
        # must also have both tokens kept
        if kq is not None:
            vis &= (kq[rows] != 0)[:, None]
        if kk is not None:
            vis &= (kk != 0)[None, :]
    elif mode != "dense":
        raise ValueError(mode)
    return vis


def _heads(B: int, H: int, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def attention_fwd(mode: str, q, k, v, keep_q=None, keep_k=None, bkt_q=None, bkt_k=None,
                  scale: Optional[float] = None, heads: Optional[Sequence[Tuple[int, int]]] = None,
                  rows: Optional[np.ndarray] = None, block: int = 512, strict: bool = False,
                  noncausal: bool = False):
    """Explicit masked-softmax causal attention in original token order.

    q: (B, Tq, H, D), k, v: (B, Tk, H, D) float64; Tq and Tk may differ (the
    explainer's decision tensors have lengths T_Q and T_KV): queries sit at
    positions 0..Tq-1 and keys at 0..Tk-1, and the causal test compares
    these positions unchanged. keep_q (B, Tq, H) / keep_k (B, Tk, H) (qk
    mode; in hash mode optional, for hashing combined with within-bucket
    dropping). bkt_q (B, H, Tq) / bkt_k (B, H, Tk) bucket ids (hash mode).
    strict: keys strictly before the query (the explainer's '>' variant);
    noncausal: no position test (bidirectional).
    heads: optional list of (b, h) to compute (others left at 0 / -inf).
    rows: optional query positions to compute (others left at 0 / -inf).
    Returns O (B, Tq, H, D) float64 and LSE (B, H, Tq) float64.
    For a row with n visible keys: O = sum_j softmax_j v_j, LSE = m + ln sum
    exp(s - m); with n = 0: O = 0, LSE = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, D = q.shape
    Tk = k.shape[1]
    tau = 1.0 / math.sqrt(D) if scale is None else scale
    O = np.zeros((B, T, H, v.shape[-1]))
    LSE = np.full((B, H, T), NEG_INF)
    all_rows = np.arange(T) if rows is None else np.asarray(rows)
    for b, h in _heads(B, H, heads):
        kq = None if keep_q is None else keep_q[b, :, h]
        kk = None if keep_k is None else keep_k[b, :, h]
        bq = None if bkt_q is None else bkt_q[b, h]
        bk = None if bkt_k is None else bkt_k[b, h]
        Kh, Vh = k[b, :, h], v[b, :, h]
        for s0 in range(0, len(all_rows), block):
            r = all_rows[s0:s0 + block]
            vis = _vis_rows(mode, r, Tk, kq, kk, bq, bk, strict, noncausal)
            S = tau * (q[b, r, h] @ Kh.T)
            S = np.where(vis, S, NEG_INF)
            has = vis.any(axis=1)
            m = np.where(has, S.max(axis=1), 0.0)
            with np.errstate(invalid="ignore"):
                e = np.where(vis, np.exp(S - m[:, None]), 0.0)
            l = e.sum(axis=1)
            lse = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
            P = np.where(vis, np.exp(S - np.where(has, lse, 0.0)[:, None]), 0.0)
            O[b, r, h] = P @ Vh
            LSE[b, h, r] = lse
    return O, LSE


def attention_bwd(mode: str, q, k, v, dO, keep_q=None, keep_k=None, bkt_q=None, bkt_k=None,
                  scale: Optional[float] = None, heads: Optional[Sequence[Tuple[int, int]]] = None,
                  block: int = 512, strict: bool = False, noncausal: bool = False):
    """Gradients of L = sum(O * dO) w.r.t. the original-order q, k, v.

    With P_ij = exp(s_ij - LSE_i) on visible pairs (0 elsewhere):
      dV_j = sum_i P_ij dO_i;   dP_ij = dO_i . v_j;   Delta_i = dO_i . O_i;
      dS_ij = P_ij (dP_ij - Delta_i);   dQ_i = tau sum_j dS_ij k_j;
      dK_j = tau sum_i dS_ij q_i.
    Keep masks and buckets are constants. Returns dQ (shaped like q) and dK,
    dV (shaped like k) float64 (zero for heads not in `heads`).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    B, T, H, D = q.shape
    Tk = k.shape[1]
    tau = 1.0 / math.sqrt(D) if scale is None else scale
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b, h in _heads(B, H, heads):
        O, LSE = attention_fwd(mode, q, k, v, keep_q, keep_k, bkt_q, bkt_k, tau, heads=[(b, h)], block=block,
                               strict=strict, noncausal=noncausal)
        kq = None if keep_q is None else keep_q[b, :, h]
        kk = None if keep_k is None else keep_k[b, :, h]
        bq = None if bkt_q is None else bkt_q[b, h]
        bk = None if bkt_k is None else bkt_k[b, h]
        Qh, Kh, Vh = q[b, :, h], k[b, :, h], v[b, :, h]
        for s0 in range(0, T, block):
            r = np.arange(s0, min(T, s0 + block))
            vis = _vis_rows(mode, r, Tk, kq, kk, bq, bk, strict, noncausal)
            lse = LSE[b, h, r]
            has = np.isfinite(lse)
            S = tau * (Qh[r] @ Kh.T)
            P = np.where(vis & has[:, None], np.exp(S - np.where(has, lse, 0.0)[:, None]), 0.0)
            dOr = dO[b, r, h]
            dV[b, :, h] += P.T @ dOr
            dP = dOr @ Vh.T
            delta = (dOr * O[b, r, h]).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dQ[b, r, h] = tau * (dS @ Kh)
            dK[b, :, h] += tau * (dS.T @ Qh[r])
    return dQ, dK, dV


def attention_rows(q, k, v, q_pos, k_pos, q_bkt=None, k_bkt=None, scale: Optional[float] = None):
    """Attention of ONE head over rows that carry explicit original positions
    (and buckets), in whatever order the rows come: a key row s is visible to
    query row r iff k_pos[s] <= q_pos[r] (and q_bkt[r] == k_bkt[s] when
    buckets are given). This is the form the compacted / sorted tensors take
    (SCFA explainer 3.4, "What the compaction achieves"; Hash-sparse,
    "Hashing and sorting"). q: (Tq, D), k, v: (Tk, D) float64.
    Returns O (Tq, D), LSE (Tq,)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    tau = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    if q_bkt is not None:
        vis &= np.asarray(q_bkt)[:, None] == np.asarray(k_bkt)[None, :]
    S = np.where(vis, tau * (q @ k.T), NEG_INF)
    has = vis.any(axis=1)
    m = np.where(has, S.max(axis=1), 0.0)
    e = np.where(vis, np.exp(np.where(vis, S, 0.0) - m[:, None]), 0.0)
    l = e.sum(axis=1)
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
    P = np.where(vis, np.exp(np.where(vis, S, 0.0) - np.where(has, lse, 0.0)[:, None]), 0.0)
    return P @ v, lse


def visible_pairs(mode: str, T: int, B: int, H: int, keep_q=None, keep_k=None, bkt_q=None, bkt_k=None,
                  strict: bool = False, noncausal: bool = False, Tk: Optional[int] = None) -> np.ndarray:
    """Exact number of visible (query, key) pairs per (b, h), T queries and
    Tk keys (default T). -> (B, H) int64."""
    Tk = T if Tk is None else Tk
    out = np.zeros((B, H), dtype=np.int64)
    sh = 1 if strict else 0
    qpos = np.arange(T)

    def upto(c):
        """Per query position i < T: the count c holds (inclusive cumsum over
        the Tk key positions) at key positions <= i (strict: < i;
        noncausal: all)."""
        if noncausal:
            return np.full(T, c[-1])
        last = np.minimum(qpos - sh, Tk - 1)  # last visible key position
        return np.where(last >= 0, c[np.maximum(last, 0)], 0)

    for b in range(B):
        for h in range(H):
            if mode == "dense":
                out[b, h] = int(upto(np.arange(1, Tk + 1)).sum())
            elif mode == "qk":
                kk = (keep_k[b, :, h] != 0).astype(np.int64)
                before = upto(np.cumsum(kk))  # kept keys visible to query position i
                out[b, h] = int(before[keep_q[b, :, h] != 0].sum())
            else:
                tot = 0
                bq, bk = bkt_q[b, h], bkt_k[b, h]
                kq = np.ones(T, bool) if keep_q is None else keep_q[b, :, h] != 0
                kk = np.ones(Tk, bool) if keep_k is None else keep_k[b, :, h] != 0
                for val in np.union1d(np.unique(bq), np.unique(bk)):
                    kin = upto(np.cumsum((bk == val) & kk))
                    tot += int(kin[(bq == val) & kq].sum())
                out[b, h] = tot
    return out


def flops_fwd(pairs: int, D: int) -> int:
    """Algorithmic forward FLOPs: 2*D for q.k plus 2*D for p*v per visible pair
    (the per-pair form of the 2*B*H*N^2*d inventory on the efficient-attention
    teaching page, section on compute/memory arithmetic)."""
    return 4 * D * int(pairs)


def flops_bwd(pairs: int, D: int) -> int:
    """Algorithmic backward FLOPs per visible pair: the five products of the
    recomputation backward (the scores S again, dP, dV, dQ, dK), each costing
    2*D per pair as the teaching page's per-product inventory counts Q K^T
    (section on compute/memory arithmetic): 10*D."""
    return 10 * D * int(pairs)
