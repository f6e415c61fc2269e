"""Python binding of libscfa.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libscfa.so. torch is used for device memory and streams. The
low-level functions carry the C names and take torch CUDA tensors; sizes are
read from the tensor shapes. The pipeline helpers at the bottom allocate the
intermediate buffers and chain the C calls for the three modes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libscfa.so")

SCFA_OK, SCFA_ERR_INVALID, SCFA_ERR_UNSUPPORTED, SCFA_ERR_HIP, SCFA_ERR_TOO_LARGE = 0, -1, -2, -3, -4
SCFA_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024
SCFA_DEVERR_COUNT_EXCEEDS_TC, SCFA_DEVERR_BUCKET_RANGE, SCFA_DEVERR_SEGMENT_OVERFLOW = 1, 2, 4
SCFA_BF16, SCFA_F32 = 0, 1
SCFA_DENSE, SCFA_QK, SCFA_HASH = 0, 1, 2
SCFA_STRICT = 16  # flag: a key is visible only strictly before its query
SCFA_NONCAUSAL = 32  # flag: no causal test (bidirectional attention)
SCFA_ROWS, SCFA_COLS = 0, 1
SCFA_Q_PAD, SCFA_K_PAD = -1, 1_000_000_000
SCFA_ROW_ALIGN = 128
SCFA_TILE_M, SCFA_TILE_N = 128, 64
SCFA_COUNT_CHUNK = 64

MODE_IDS = {"dense": SCFA_DENSE, "qk": SCFA_QK, "hash": SCFA_HASH}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes)
_SIGS = {
    "scfa_status_string": (ctypes.c_char_p, [_i]),
    "scfa_version": (_i, []),
    "scfa_qk_count": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "scfa_qk_compact": (_i, [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_int32, _vp, _vp, _vp, _vp]),
    "scfa_hash_bucket": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "scfa_hash_sort_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "scfa_hash_sort": (_i, [_vp, _i, _i, _i, _i, ctypes.c_int32, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "scfa_hash_segment_rows": (_i, [_i, _i, _i]),
    "scfa_hash_segments": (_i, [_vp, _vp, _i, _i, _i, _i, _i, ctypes.c_int32, _i, _vp, _vp, _vp, _vp, _vp]),
    "scfa_hash_layout": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "scfa_hash_bucket_counts": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "scfa_hash_bucket_counts_drop": (_i, [_i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "scfa_hash_bucket_qk": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "scfa_hash_layout_qk": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i] + [_vp] * 17),
    "scfa_fwd_table": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "scfa_bwd_table": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _vp]),
    "scfa_gather": (_i, [_i, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "scfa_range_table": (_i, [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "scfa_count_visible": (_i, [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "scfa_work_order": (_i, [_vp, _i, _i, _i, _i, _vp, _vp]),
    "scfa_bwd_table_order": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _i, _vp]),
    "scfa_fwd_table_order": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "scfa_qk_index_qk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i] + [_vp] * 12),
    "scfa_qk_sparse_fwd": (_i, [_i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                _vp, _vp, _vp]),
    "scfa_hash_sparse_fwd": (_i, [_i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                  _i, _i, _f, _i, _vp, _vp, _vp]),
    "scfa_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "scfa_bwd": (_i, [_i, _i] + [_vp] * 16 + [_i] * 7 + [_f, _vp, _vp, _vp, _vp, _sz, _vp]),
    "scfa_bwd_noalloc": (_i, [_i, _i] + [_vp] * 16 + [_i] * 7 + [_f, _vp, _vp, _vp, _vp]),
}

_LIB = None


class ScfaError(RuntimeError):
    pass


def lib():
    """Load libscfa.so (built in-tree by __graft_entry__.build()). Fails loudly
    when the library is missing: there is no fallback path."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ScfaError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name, None)
            if fn is None:
                continue
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def exported_symbols():
    L = lib()
    return [n for n in _SIGS if getattr(L, n, None) is not None]


def _check(status: int, name: str):
    if status != SCFA_OK:
        msg = lib().scfa_status_string(status).decode()
        raise ScfaError(f"{name} failed: {msg}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ScfaError("expected a device tensor")
    if not t.is_contiguous():
        raise ScfaError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref: Optional[torch.Tensor] = None):
    if stream is None:
        dev = ref.device if ref is not None else torch.device("cuda")
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SCFA_BF16
    if t.dtype == torch.float32:
        return SCFA_F32
    raise ScfaError(f"unsupported dtype {t.dtype}")


def pad_rows(n: int) -> int:
    return ((n + SCFA_ROW_ALIGN - 1) // SCFA_ROW_ALIGN) * SCFA_ROW_ALIGN


# ---------------------------------------------------------------------------
# Low-level calls (same names as the C ABI).
# ---------------------------------------------------------------------------

def scfa_status_string(status: int) -> str:
    return lib().scfa_status_string(status).decode()


def scfa_version() -> int:
    return lib().scfa_version()


def scfa_qk_count(keep, count, max_count, chunk_offsets, stream=None):
    B, T, H = keep.shape
    _check(lib().scfa_qk_count(_p(keep), B, T, H, _p(count), _p(max_count), _p(chunk_offsets), _stream(stream, keep)),
           "scfa_qk_count")


def scfa_qk_compact(x, keep, count, chunk_offsets, Tc, pad_idx, x_c, idx_c, dev_err=None, stream=None):
    B, T, H = keep.shape
    D = x.shape[-1] if x is not None else 64
    dt = _dt(x) if x is not None else SCFA_BF16
    _check(lib().scfa_qk_compact(dt, _p(x), _p(keep), _p(count), _p(chunk_offsets), B, T, H, D, Tc, pad_idx, _p(x_c),
                                 _p(idx_c), _p(dev_err), _stream(stream, keep)), "scfa_qk_compact")


def scfa_qk_index_qk(keep_q, keep_k, Tq, Tk, count_q, count_k, max_count, chunk_counts_q, chunk_counts_k, q_idx,
                     k_idx, dev_err=None, stream=None, qstats=None, kstats=None, tiles=None):
    """Index compaction of the queries and of the keys in two launches
    (counts and index arrays of both sides; the chunk counts are workspace),
    optionally with the tile statistics of the attention tiles."""
    B, T, H = keep_q.shape
    T_kv = keep_k.shape[1]
    if keep_k.shape[0] != B or keep_k.shape[2] != H:
        raise ScfaError("keep_q and keep_k must share B and H")
    _check(lib().scfa_qk_index_qk(_p(keep_q), _p(keep_k), B, T, T_kv, H, Tq, Tk, _p(count_q), _p(count_k),
                                  _p(max_count), _p(chunk_counts_q), _p(chunk_counts_k), _p(q_idx), _p(k_idx),
                                  _p(qstats), _p(kstats), _p(tiles), _p(dev_err), _stream(stream, keep_q)),
           "scfa_qk_index_qk")


def scfa_hash_bucket(x, R, nb, bucket, stream=None):
    B, T, H, D = x.shape
    _check(lib().scfa_hash_bucket(_dt(x), _p(x), _p(R), B, T, H, D, nb, _p(bucket), _stream(stream, x)),
           "scfa_hash_bucket")


def scfa_hash_bucket_counts(x, R, nb, bucket, chunk_counts, stream=None):
    B, T, H, D = x.shape
    _check(lib().scfa_hash_bucket_counts(_dt(x), _p(x), _p(R), B, T, H, D, nb, _p(bucket), _p(chunk_counts),
                                         _stream(stream, x)), "scfa_hash_bucket_counts")


def scfa_hash_bucket_counts_drop(x, R, keep, side, nb, bucket, chunk_counts, stream=None):
    """One side with its keep mask (side 0: queries, dropped -> nb; side 1:
    keys, dropped -> nb + 1); chunk counts over nb + 2 buckets."""
    B, T, H, D = x.shape
    if keep is None or tuple(keep.shape) != (B, T, H):
        raise ScfaError("keep must be (B, T, H) for the side's own length T")
    _check(lib().scfa_hash_bucket_counts_drop(_dt(x), _p(x), _p(R), _p(keep), side, B, T, H, D, nb, _p(bucket),
                                              _p(chunk_counts), _stream(stream, x)), "scfa_hash_bucket_counts_drop")


def scfa_hash_bucket_qk(q, k, R, nb, bucket_q, bucket_k, counts_q, counts_k, stream=None, keep_q=None, keep_k=None):
    """scfa_hash_bucket_counts of queries and keys in one launch; with keep
    masks, dropped queries take bucket nb and dropped keys bucket nb + 1
    (chunk counts then have nb + 2 buckets)."""
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ScfaError("queries and keys must have the same shape and dtype")
    if (keep_q is None) != (keep_k is None):
        raise ScfaError("give both keep masks or neither")
    B, T, H, D = q.shape
    _check(lib().scfa_hash_bucket_qk(_dt(q), _p(q), _p(k), _p(R), _p(keep_q), _p(keep_k), B, T, H, D, nb,
                                     _p(bucket_q), _p(bucket_k), _p(counts_q), _p(counts_k), _stream(stream, q)),
           "scfa_hash_bucket_qk")


def scfa_hash_sort_workspace_bytes(B, H, T, nb) -> int:
    return lib().scfa_hash_sort_workspace_bytes(B, H, T, nb)


def scfa_hash_sort(bucket, nb, pad_idx, perm, bucket_sorted, offsets, workspace, dev_err=None, stream=None):
    B, H, T = bucket.shape
    _check(lib().scfa_hash_sort(_p(bucket), B, H, T, nb, pad_idx, _p(perm), _p(bucket_sorted), _p(offsets),
                                _p(workspace), workspace.numel() * workspace.element_size(), _p(dev_err),
                                _stream(stream, bucket)), "scfa_hash_sort")


def scfa_hash_segment_rows(T, nb, align) -> int:
    return lib().scfa_hash_segment_rows(T, nb, align)


def scfa_hash_segments(perm, offsets, T, nb, align, pad_idx, idx_seg, bkt_seg, seg_offsets, dev_err=None,
                       stream=None):
    B, H, Tseg = idx_seg.shape
    _check(lib().scfa_hash_segments(_p(perm), _p(offsets), B, H, T, nb, align, pad_idx, Tseg, _p(idx_seg),
                                    _p(bkt_seg), _p(seg_offsets), _p(dev_err), _stream(stream, perm)),
           "scfa_hash_segments")


def scfa_hash_layout(bucket, chunk_counts, nb, align, pad_idx, perm, bucket_sorted, offsets, idx_seg=None,
                     bkt_seg=None, seg_offsets=None, dev_err=None, stream=None):
    """Sort by bucket and (align > 0) the bucket-aligned layout in one launch,
    from the chunk counts of scfa_hash_bucket_counts."""
    B, H, T = bucket.shape
    Tseg = idx_seg.shape[-1] if idx_seg is not None else 0
    _check(lib().scfa_hash_layout(_p(bucket), _p(chunk_counts), B, H, T, nb, align, pad_idx, Tseg, _p(perm),
                                  _p(bucket_sorted), _p(offsets), _p(idx_seg), _p(bkt_seg), _p(seg_offsets),
                                  _p(dev_err), _stream(stream, bucket)), "scfa_hash_layout")


def scfa_hash_layout_qk(bucket_q, bucket_k, counts_q, counts_k, nb, perm_q, perm_k, bs_q, bs_k, off_q, off_k, idx_q,
                        idx_k, bkt_q, bkt_k, seg_q, seg_k, dev_err, qstats=None, kstats=None, tiles=None, stream=None):
    """scfa_hash_layout of queries (query-tile alignment, query pads) and keys
    (key-tile alignment, key pads) in one launch; optionally also the tile
    statistics of both layouts and a zeroed processed-tile counter."""
    B, H, T = bucket_q.shape
    if bucket_k.shape != bucket_q.shape:
        raise ScfaError("query and key buckets must have the same shape")
    _check(lib().scfa_hash_layout_qk(_p(bucket_q), _p(bucket_k), _p(counts_q), _p(counts_k), B, H, T, nb,
                                     idx_q.shape[-1], idx_k.shape[-1], _p(perm_q), _p(perm_k), _p(bs_q), _p(bs_k),
                                     _p(off_q), _p(off_k), _p(idx_q), _p(idx_k), _p(bkt_q), _p(bkt_k), _p(seg_q),
                                     _p(seg_k), _p(qstats), _p(kstats), _p(tiles), _p(dev_err),
                                     _stream(stream, bucket_q)), "scfa_hash_layout_qk")


def scfa_fwd_table(mode, qstats, kstats, fwd_tab, tiles, stream=None):
    """Forward range table from tile statistics (tiles must be zero on entry)."""
    B, H, nQt, _ = qstats.shape
    nKt = kstats.shape[2]
    _check(lib().scfa_fwd_table(mode, _p(qstats), _p(kstats), B, H, nQt, nKt, _p(fwd_tab), _p(tiles),
                                _stream(stream, qstats)), "scfa_fwd_table")


def scfa_fwd_table_order(mode, qstats, kstats, fwd_tab, tiles, order, stream=None):
    """Forward range table and its launch order in one launch (tiles must be
    zero on entry)."""
    B, H, nQt, _ = qstats.shape
    nKt = kstats.shape[2]
    _check(lib().scfa_fwd_table_order(mode, _p(qstats), _p(kstats), B, H, nQt, nKt, _p(fwd_tab), _p(tiles), _p(order),
                                      _stream(stream, qstats)), "scfa_fwd_table_order")


def chunk_count_shape(B, H, T, nb):
    """Shape of the chunk counts of scfa_hash_bucket_counts."""
    return (B, H, (T + 255) // 256, nb)


def scfa_gather(x, idx, layout, x_p, stream=None):
    B, T, H, D = x.shape
    Tp = idx.shape[-1]
    _check(lib().scfa_gather(_dt(x), layout, _p(x), _p(idx), B, T, H, D, Tp, _p(x_p), _stream(stream, x)),
           "scfa_gather")


def scfa_range_table(mode, q_idx, k_idx, q_bkt, k_bkt, B, H, Tq, Tk, Bm, Bn, qstats, kstats, fwd_tab, bwd_tab, tiles,
                     stream=None):
    _check(lib().scfa_range_table(mode, _p(q_idx), _p(k_idx), _p(q_bkt), _p(k_bkt), B, H, Tq, Tk, Bm, Bn, _p(qstats),
                                  _p(kstats), _p(fwd_tab), _p(bwd_tab), _p(tiles), _stream(stream, qstats)),
           "scfa_range_table")


def scfa_bwd_table(qstats, kstats, fwd_tab, bwd_tab, stream=None, flags=0):
    B, H, nQt = fwd_tab.shape[:3]
    nKt = bwd_tab.shape[2]
    _check(lib().scfa_bwd_table(_p(qstats), _p(kstats), _p(fwd_tab), B, H, nQt, nKt, _p(bwd_tab), flags,
                                _stream(stream, fwd_tab)), "scfa_bwd_table")


def scfa_bwd_table_order(qstats, kstats, fwd_tab, bwd_tab, order, stream=None, flags=0):
    """scfa_bwd_table and scfa_work_order(bwd_tab, span = nQt) in one launch."""
    B, H, nQt = fwd_tab.shape[:3]
    nKt = bwd_tab.shape[2]
    _check(lib().scfa_bwd_table_order(_p(qstats), _p(kstats), _p(fwd_tab), B, H, nQt, nKt, _p(bwd_tab), _p(order),
                                      flags, _stream(stream, fwd_tab)), "scfa_bwd_table_order")


def scfa_count_visible(mode, q_idx, k_idx, q_bkt, k_bkt, B, H, Tq, Tk, pairs, stream=None):
    _check(lib().scfa_count_visible(mode, _p(q_idx), _p(k_idx), _p(q_bkt), _p(k_bkt), B, H, Tq, Tk, _p(pairs),
                                    _stream(stream, pairs)), "scfa_count_visible")


def scfa_work_order(tab, span, order, stream=None):
    B, H, n, _ = tab.shape
    _check(lib().scfa_work_order(_p(tab), B, H, n, span, _p(order), _stream(stream, tab)), "scfa_work_order")


def _kv_len(q, k, v) -> int:
    """Tokens of the original k and v tensors (B, T_kv, H, D)."""
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ScfaError("k and v must be (B, T_kv, H, D) with the B, H, D of q")
    return k.shape[1]


def scfa_qk_sparse_fwd(q, k, v, q_idx, k_idx, qstats, kstats, fwd_tab, T, O, lse, scale=None, stream=None,
                       order=None, flags=0):
    """q: original (B,T,H,D), k, v: original (B,T_kv,H,D) tensors; q_idx,
    k_idx (B,H,Tc) compacted."""
    B, Tq_, H, D = q.shape
    if Tq_ != T:
        raise ScfaError("q must be the original (B,T,H,D) tensor")
    Tc = q_idx.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(lib().scfa_qk_sparse_fwd(_dt(q), _dt(O), _p(q), _p(k), _p(v), _p(q_idx), _p(k_idx), _p(qstats),
                                    _p(kstats), _p(fwd_tab), _p(order), B, H, T, _kv_len(q, k, v), Tc, D, scale, flags,
                                    _p(O), _p(lse), _stream(stream, q)), "scfa_qk_sparse_fwd")


def scfa_hash_sparse_fwd(q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, T, O, lse, scale=None,
                         stream=None, order=None, Tq=None, Tk=None, flags=0):
    """q: original (B,T,H,D), k, v: original (B,T_kv,H,D) tensors. Tq / Tk:
    query / key rows as passed to the range table (default: T, T_kv)."""
    B, Tq_, H, D = q.shape
    if Tq_ != T:
        raise ScfaError("q must be the original (B,T,H,D) tensor")
    T_kv = _kv_len(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    Tq = T if Tq is None else Tq
    Tk = T_kv if Tk is None else Tk
    _check(lib().scfa_hash_sparse_fwd(_dt(q), _dt(O), _p(q), _p(k), _p(v), _p(q_idx), _p(k_idx), _p(q_bkt),
                                      _p(k_bkt), _p(qstats), _p(kstats), _p(fwd_tab), _p(order), B, H, T, T_kv, Tq, Tk,
                                      D, scale, flags, _p(O), _p(lse), _stream(stream, q)), "scfa_hash_sparse_fwd")


def scfa_bwd_workspace_bytes(mode, B, H, Tq, Tk, D=64) -> int:
    return lib().scfa_bwd_workspace_bytes(mode, B, H, Tq, Tk, D)


def scfa_bwd(mode, q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, bwd_tab, O, lse, dO, T, Tq, Tk, dQ,
             dK, dV, workspace, scale=None, stream=None, fwd_order=None, bwd_order=None):
    """q, dO: original (B,T,H,D), k, v: original (B,T_kv,H,D) bf16 tensors
    (read through the index arrays); fwd_order / bwd_order: optional launch
    orders from scfa_work_order."""
    B, Tq_, H, D = q.shape
    if Tq_ != T:
        raise ScfaError("q must be the original (B,T,H,D) tensor")
    T_kv = _kv_len(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(lib().scfa_bwd(mode, _dt(q), _p(q), _p(k), _p(v), _p(q_idx), _p(k_idx), _p(q_bkt), _p(k_bkt), _p(qstats),
                          _p(kstats), _p(fwd_tab), _p(bwd_tab), _p(fwd_order), _p(bwd_order), _p(O), _p(lse), _p(dO), B,
                          H, T, T_kv, Tq, Tk, D, scale, _p(dQ), _p(dK), _p(dV), _p(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream, q)), "scfa_bwd")


def scfa_bwd_noalloc(mode, q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, bwd_tab, O, lse, dO, T, Tq,
                     Tk, dQ, dK, dV, scale=None, stream=None, fwd_order=None, bwd_order=None):
    """scfa_bwd without a workspace argument: the library's static per-device
    scratch holds it (for callers that cannot allocate)."""
    B, Tq_, H, D = q.shape
    if Tq_ != T:
        raise ScfaError("q must be the original (B,T,H,D) tensor")
    T_kv = _kv_len(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(lib().scfa_bwd_noalloc(mode, _dt(q), _p(q), _p(k), _p(v), _p(q_idx), _p(k_idx), _p(q_bkt), _p(k_bkt),
                                  _p(qstats), _p(kstats), _p(fwd_tab), _p(bwd_tab), _p(fwd_order), _p(bwd_order),
                                  _p(O), _p(lse), _p(dO), B, H, T, T_kv, Tq, Tk, D, scale, _p(dQ), _p(dK), _p(dV),
                                  _stream(stream, q)),
           "scfa_bwd_noalloc")


# ---------------------------------------------------------------------------
# Pipelines: allocate intermediates and chain the calls.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Prepared:
    """Index arrays of one attention call (head-major) and its operands.

    Forward and backward read q_in, k_in, v_in (original (B,T,H,D) order)
    through q_idx / k_idx. Head-major copies q, k (rows) and v_t
    (transposed) exist only on request (gather_operands(), or the compacted
    rows of prepare_qk(rows=True)).
    Tq, Tk are the query / key rows as passed to the range table; the index
    arrays hold pad_rows(Tq) / pad_rows(Tk) rows per head."""
    mode: str
    B: int
    H: int
    T: int
    D: int
    Tq: int
    Tk: int
    q_in: torch.Tensor
    k_in: torch.Tensor
    v_in: torch.Tensor
    q_idx: torch.Tensor
    k_idx: torch.Tensor
    q_bkt: Optional[torch.Tensor] = None
    k_bkt: Optional[torch.Tensor] = None
    q: Optional[torch.Tensor] = None  # (B,H,pad(Tq),D) rows
    k: Optional[torch.Tensor] = None  # (B,H,pad(Tk),D) rows
    v_t: Optional[torch.Tensor] = None  # (B,H,D,pad(Tk)) transposed
    extra: dict = dataclasses.field(default_factory=dict)
    strict: bool = False  # keys strictly before the query (SCFA_STRICT)
    noncausal: bool = False  # no causal test (SCFA_NONCAUSAL)


def gather_operands(pre: Prepared, stream=None) -> Prepared:
    """Head-major copies of the operands in index order (pad rows zero); a
    no-op for the ones already present."""
    B, H, D = pre.B, pre.H, pre.D
    TqP, TkP = pad_rows(pre.Tq), pad_rows(pre.Tk)
    if pre.q is None:
        pre.q = _empty((B, H, TqP, D), pre.q_in.dtype, pre.q_in)
        scfa_gather(pre.q_in, pre.q_idx, SCFA_ROWS, pre.q, stream)
    if pre.k is None:
        pre.k = _empty((B, H, TkP, D), pre.k_in.dtype, pre.k_in)
        scfa_gather(pre.k_in, pre.k_idx, SCFA_ROWS, pre.k, stream)
    if pre.v_t is None:
        pre.v_t = _empty((B, H, D, TkP), pre.v_in.dtype, pre.v_in)
        scfa_gather(pre.v_in, pre.k_idx, SCFA_COLS, pre.v_t, stream)
    return pre


@dataclasses.dataclass
class Tables:
    qstats: torch.Tensor
    kstats: torch.Tensor
    fwd: torch.Tensor
    bwd: torch.Tensor
    tiles: torch.Tensor
    Bm: int
    Bn: int
    fwd_order: Optional[torch.Tensor] = None  # launch order of the forward / dQ workgroups
    bwd_order: Optional[torch.Tensor] = None  # launch order of the dK/dV workgroups (hash mode)
    bwd_ready: bool = True  # bwd (and bwd_order) hold the ranges of the current forward tables


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def prepare_qk(q, k, v, keep_q, keep_k, Tc: Optional[int] = None, rows: bool = False, stream=None,
               strict: bool = False, noncausal: bool = False) -> Prepared:
    """QK-drop preprocessing: counts and the compacted index arrays (with
    rows=True also the compacted Q and K rows). Reads the max kept count back
    to the host once (to size Tc) unless Tc is given."""
    B, T, H, D = q.shape
    T_kv = _kv_len(q, k, v)
    dev = q
    i32 = torch.int32
    nCq = (T + SCFA_COUNT_CHUNK - 1) // SCFA_COUNT_CHUNK
    nCk = (T_kv + SCFA_COUNT_CHUNK - 1) // SCFA_COUNT_CHUNK
    cq, ck = _empty((B, H), i32, dev), _empty((B, H), i32, dev)
    mq, mk = _empty((1,), i32, dev), _empty((1,), i32, dev)
    oq, ok = _empty((B, H, nCq), i32, dev), _empty((B, H, nCk), i32, dev)
    scfa_qk_count(keep_q, cq, mq, oq, stream)
    scfa_qk_count(keep_k, ck, mk, ok, stream)
    if Tc is None:
        Tc = pad_rows(max(1, int(torch.maximum(mq, mk).item())))
    dev_err = torch.zeros((1,), dtype=i32, device=q.device)
    q_c = _empty((B, H, Tc, D), q.dtype, dev) if rows else None
    k_c = _empty((B, H, Tc, D), k.dtype, dev) if rows else None
    q_idx, k_idx = _empty((B, H, Tc), i32, dev), _empty((B, H, Tc), i32, dev)
    scfa_qk_compact(q, keep_q, cq, oq, Tc, SCFA_Q_PAD, q_c, q_idx, dev_err, stream)
    scfa_qk_compact(k, keep_k, ck, ok, Tc, SCFA_K_PAD, k_c, k_idx, dev_err, stream)
    return Prepared("qk", B, H, T, D, Tc, Tc, q, k, v, q_idx, k_idx, q=q_c, k=k_c,
                    extra={"count_q": cq, "count_k": ck, "max_q": mq, "max_k": mk, "dev_err": dev_err}, strict=strict,
                    noncausal=noncausal)


def prepare_hash(q, k, v, R, nb: int, aligned: bool = True, stream=None, keep_q=None, keep_k=None,
                 strict: bool = False, noncausal: bool = False) -> Prepared:
    """Hash-sparse preprocessing: LSH buckets of Q and K, stable counting sort
    per head and (aligned=True) the bucket-aligned layout in one launch per
    side (query buckets start at multiples of the query tile, key buckets at
    multiples of the key tile). The operands stay in original order (gathered
    on load). With keep masks (hashing combined with within-bucket dropping)
    dropped queries take bucket nb and dropped keys bucket nb + 1 (two-side
    launch, or one launch per side when the lengths differ), and the sort has
    nb + 2 buckets."""
    B, T, H, D = q.shape
    T_kv = _kv_len(q, k, v)
    dev = q
    i32 = torch.int32
    Tp, Tkp = pad_rows(T), pad_rows(T_kv)
    if (keep_q is None) != (keep_k is None):
        raise ScfaError("give both keep masks or neither")
    nbs = nb if keep_q is None else nb + 2  # buckets of the sort
    bq, bk = _empty((B, H, T), i32, dev), _empty((B, H, T_kv), i32, dev)
    cq, ck = _empty(chunk_count_shape(B, H, T, nbs), i32, dev), _empty(chunk_count_shape(B, H, T_kv, nbs), i32, dev)
    if nbs == nb:
        scfa_hash_bucket_counts(q, R, nb, bq, cq, stream)
        scfa_hash_bucket_counts(k, R, nb, bk, ck, stream)
    elif T_kv == T:
        scfa_hash_bucket_qk(q, k, R, nb, bq, bk, cq, ck, stream, keep_q, keep_k)
    else:  # two lengths: one launch per side
        scfa_hash_bucket_counts_drop(q, R, keep_q, 0, nb, bq, cq, stream)
        scfa_hash_bucket_counts_drop(k, R, keep_k, 1, nb, bk, ck, stream)
    nb = nbs
    dev_err = torch.zeros((1,), dtype=i32, device=q.device)
    perm_q, perm_k = _empty((B, H, Tp), i32, dev), _empty((B, H, Tkp), i32, dev)
    bs_q, bs_k = _empty((B, H, Tp), i32, dev), _empty((B, H, Tkp), i32, dev)
    offq, offk = _empty((B, H, nb + 1), i32, dev), _empty((B, H, nb + 1), i32, dev)
    extra = {"bucket_q": bq, "bucket_k": bk, "chunk_counts_q": cq, "chunk_counts_k": ck, "perm_q": perm_q,
             "perm_k": perm_k, "sorted_bkt_q": bs_q, "sorted_bkt_k": bs_k, "offsets_q": offq, "offsets_k": offk,
             "dev_err": dev_err, "sort_buckets": nb}
    if aligned:
        Tq = scfa_hash_segment_rows(T, nb, SCFA_TILE_M)
        Tk = scfa_hash_segment_rows(T_kv, nb, SCFA_TILE_N)
        q_idx, q_bkt = _empty((B, H, Tq), i32, dev), _empty((B, H, Tq), i32, dev)
        k_idx, k_bkt = _empty((B, H, Tk), i32, dev), _empty((B, H, Tk), i32, dev)
        sq, sk = _empty((B, H, nb + 1), i32, dev), _empty((B, H, nb + 1), i32, dev)
        scfa_hash_layout(bq, cq, nb, SCFA_TILE_M, SCFA_Q_PAD, perm_q, bs_q, offq, q_idx, q_bkt, sq, dev_err, stream)
        scfa_hash_layout(bk, ck, nb, SCFA_TILE_N, SCFA_K_PAD, perm_k, bs_k, offk, k_idx, k_bkt, sk, dev_err, stream)
        extra.update(seg_offsets_q=sq, seg_offsets_k=sk)
    else:
        scfa_hash_layout(bq, cq, nb, 0, SCFA_Q_PAD, perm_q, bs_q, offq, dev_err=dev_err, stream=stream)
        scfa_hash_layout(bk, ck, nb, 0, SCFA_K_PAD, perm_k, bs_k, offk, dev_err=dev_err, stream=stream)
        Tq, Tk = T, T_kv
        q_idx, k_idx, q_bkt, k_bkt = perm_q, perm_k, bs_q, bs_k
    return Prepared("hash", B, H, T, D, Tq, Tk, q, k, v, q_idx, k_idx, q_bkt, k_bkt, extra=extra, strict=strict,
                    noncausal=noncausal)


def prepare_dense(q, k, v, stream=None, strict: bool = False, noncausal: bool = False) -> Prepared:
    """Dense causal attention on the same kernel: positions 0..T-1 for the
    queries and 0..T_kv-1 for the keys (the QK path with nothing dropped;
    both index arrays padded to one length, as the QK path's compacted ones)."""
    B, T, H, D = q.shape
    T_kv = _kv_len(q, k, v)
    Tp = pad_rows(max(T, T_kv))
    ar = torch.arange(Tp, dtype=torch.int32, device=q.device)
    q_idx = torch.where(ar < T, ar, torch.full_like(ar, SCFA_Q_PAD)).expand(B, H, Tp).contiguous()
    k_idx = torch.where(ar < T_kv, ar, torch.full_like(ar, SCFA_K_PAD)).expand(B, H, Tp).contiguous()
    return Prepared("dense", B, H, T, D, Tp, Tp, q, k, v, q_idx, k_idx, strict=strict, noncausal=noncausal)


def _table_mode(mode: str) -> int:
    return SCFA_HASH if mode == "hash" else SCFA_QK


def _flags(pre: "Prepared") -> int:
    if pre.strict and pre.noncausal:
        raise ScfaError("strict and noncausal exclude each other")
    return (SCFA_STRICT if pre.strict else 0) | (SCFA_NONCAUSAL if pre.noncausal else 0)


def build_tables(pre: Prepared, Bm: int = SCFA_TILE_M, Bn: int = SCFA_TILE_N, stream=None) -> Tables:
    """Tile extrema, range tables and the forward launch order. Dense inputs
    use the QK rule on their arange positions (identical to the dense rule,
    and it keeps the ragged tail's pads out of the causal ranges)."""
    B, H = pre.B, pre.H
    nQt, nKt = pad_rows(pre.Tq) // Bm, pad_rows(pre.Tk) // Bn
    i32 = torch.int32
    d = pre.q_idx
    t = Tables(_empty((B, H, nQt, 4), i32, d), _empty((B, H, nKt, 4), i32, d), _empty((B, H, nQt, 2), i32, d),
               _empty((B, H, nKt, 2), i32, d), _empty((B, H), i32, d), Bm, Bn)
    scfa_range_table(_table_mode(pre.mode) | _flags(pre), pre.q_idx, pre.k_idx, pre.q_bkt, pre.k_bkt, B, H, pre.Tq,
                     pre.Tk, Bm, Bn, t.qstats, t.kstats, t.fwd, t.bwd, t.tiles, stream)
    t.fwd_order = _empty((B * H * nQt,), i32, d)
    scfa_work_order(t.fwd, nKt, t.fwd_order, stream)
    t.bwd_order = _empty((B * H * nKt,), i32, d)
    scfa_work_order(t.bwd, nQt, t.bwd_order, stream)
    return t


def count_visible(pre: Prepared, stream=None) -> torch.Tensor:
    pairs = _empty((pre.B, pre.H), torch.int64, pre.q_idx)
    scfa_count_visible(_table_mode(pre.mode) | _flags(pre), pre.q_idx, pre.k_idx, pre.q_bkt, pre.k_bkt, pre.B, pre.H,
                       pre.Tq, pre.Tk, pairs, stream)
    return pairs


def forward(pre: Prepared, tab: Tables, out_dtype=torch.float32, scale=None, O=None, lse=None, stream=None):
    """Attention forward on the original operands through the prepared index
    arrays. Returns O (B,T,H,D) in original order and LSE (B,H,T) float32."""
    B, H, T, D = pre.B, pre.H, pre.T, pre.D
    if O is None:
        O = _empty((B, T, H, D), out_dtype, pre.q_in)
    if lse is None:
        lse = _empty((B, H, T), torch.float32, pre.q_in)
    if pre.mode == "hash":
        scfa_hash_sparse_fwd(pre.q_in, pre.k_in, pre.v_in, pre.q_idx, pre.k_idx, pre.q_bkt, pre.k_bkt, tab.qstats, tab.kstats,
                             tab.fwd, T, O, lse, scale, stream, order=tab.fwd_order, Tq=pre.Tq, Tk=pre.Tk,
                             flags=_flags(pre))
    else:
        scfa_qk_sparse_fwd(pre.q_in, pre.k_in, pre.v_in, pre.q_idx, pre.k_idx, tab.qstats, tab.kstats, tab.fwd, T, O, lse,
                           scale, stream, order=tab.fwd_order, flags=_flags(pre))
    return O, lse


def backward(pre: Prepared, tab: Tables, O, lse, dO, scale=None, grads=None, workspace=None, stream=None):
    """Gradients w.r.t. the original-order q, k, v (fp32, (B,T,H,D)); the
    backward kernels read q, k, v and dO through the index arrays."""
    if not tab.bwd_ready:  # the dK/dV kernel reads bwd (and bwd_order)
        raise ScfaError("the backward table of these tables is not built (a plan builds it in its backward())")
    B, H, T, D = pre.B, pre.H, pre.T, pre.D
    mode = _table_mode(pre.mode)
    if grads is None:
        T_kv = pre.k_in.shape[1]
        grads = tuple(_empty((B, n, H, D), torch.float32, pre.q_in) for n in (T, T_kv, T_kv))
    if workspace is None:
        workspace = _empty((scfa_bwd_workspace_bytes(mode, B, H, pre.Tq, pre.Tk, D),), torch.uint8, pre.q_in)
    dQ, dK, dV = grads
    scfa_bwd(mode | _flags(pre), pre.q_in, pre.k_in, pre.v_in, pre.q_idx, pre.k_idx, pre.q_bkt, pre.k_bkt, tab.qstats,
             tab.kstats, tab.fwd, tab.bwd, O, lse, dO, T, pre.Tq, pre.Tk, dQ, dK, dV, workspace, scale, stream,
             fwd_order=tab.fwd_order, bwd_order=tab.bwd_order)
    return dQ, dK, dV


def qk_sparse_attention(q, k, v, keep_q, keep_k, out_dtype=torch.float32, scale=None):
    pre = prepare_qk(q, k, v, keep_q, keep_k)
    return forward(pre, build_tables(pre), out_dtype, scale)


def hash_sparse_attention(q, k, v, R, nb, out_dtype=torch.float32, scale=None):
    pre = prepare_hash(q, k, v, R, nb)
    return forward(pre, build_tables(pre), out_dtype, scale)


def dense_causal_attention(q, k, v, out_dtype=torch.float32, scale=None):
    pre = prepare_dense(q, k, v)
    return forward(pre, build_tables(pre), out_dtype, scale)


# ---------------------------------------------------------------------------
# Plans: every buffer allocated once, run() only launches kernels (no host
# synchronisation, no allocation), so a plan can be timed or graph-captured.
# ---------------------------------------------------------------------------

class Plan:
    """Preallocated pipeline for one shape and mode.

    mode "hash": bucket -> sort -> bucket-aligned layout -> tables -> forward.
    mode "hash_drop": hash with the keep masks of the inputs as well (hashing
                 combined with within-bucket dropping: dropped queries and
                 keys take buckets nb and nb + 1, which match nothing).
    mode "qk":   count -> compact (index arrays) -> tables -> forward, with a
                 fixed compacted length Tc (default: pad_rows(T), which always
                 fits).
    mode "dense": tables -> forward on positions 0..T-1.
    T_kv: key/value length when it differs from the query length T (keys at
    positions 0..T_kv-1); hash mode then runs the one-side bucket and layout
    launches per side and builds the tile statistics with the tables.
    Forward and backward read the operands through the index arrays (no
    gathered copies). Each stage is a separate method so it can be timed on
    its own.
    """

    def __init__(self, mode, B, H, T, D=64, dtype=torch.bfloat16, nb=16, Tc=None, out_dtype=torch.float32,
                 device="cuda", scale=None, strict=False, noncausal=False, T_kv=None):
        self.drop = mode == "hash_drop"
        self.T_kv = T if T_kv is None else T_kv
        self.two_side = self.T_kv == T  # queries and keys bucketed and laid out in one launch each
        if self.drop:
            mode = "hash"
            if nb > 62:
                raise ScfaError("hash_drop supports nb <= 62")
        if mode not in MODE_IDS:
            raise ScfaError(f"unknown mode {mode}")
        self.mode, self.B, self.H, self.T, self.D, self.nb = mode, B, H, T, D, nb
        self.nbs = nb + 2 if self.drop else nb  # buckets of the sort and layout
        self.strict = bool(strict)  # keys strictly before the query (SCFA_STRICT)
        self.noncausal = bool(noncausal)  # no causal test (SCFA_NONCAUSAL)
        if self.strict and self.noncausal:
            raise ScfaError("strict and noncausal exclude each other")
        self.flags = (SCFA_STRICT if self.strict else 0) | (SCFA_NONCAUSAL if self.noncausal else 0)
        self.dtype, self.out_dtype = dtype, out_dtype
        self.scale = 1.0 / math.sqrt(D) if scale is None else scale
        d = torch.device(device)
        i32 = torch.int32
        e = lambda shape, dt=i32: torch.empty(shape, dtype=dt, device=d)  # noqa: E731
        Tkv = self.T_kv
        if mode == "qk":
            Tc = Tc if Tc is not None else pad_rows(max(T, Tkv))
            if Tc % SCFA_ROW_ALIGN:
                raise ScfaError("Tc must be a multiple of 128")
            self.Tq = self.Tk = Tc
            nC = [(n + SCFA_COUNT_CHUNK - 1) // SCFA_COUNT_CHUNK for n in (T, Tkv)]
            self.cnt = [e((B, H)), e((B, H))]
            self.mx2 = e((2,))  # max counts of the query and key sides
            self.mx = [self.mx2[0:1], self.mx2[1:2]]
            self.choff = [e((B, H, nC[0])), e((B, H, nC[1]))]
        elif mode == "hash":
            self.Tq = scfa_hash_segment_rows(T, self.nbs, SCFA_TILE_M)
            self.Tk = scfa_hash_segment_rows(Tkv, self.nbs, SCFA_TILE_N)
        else:
            self.Tq = self.Tk = pad_rows(max(T, Tkv))
        TqP, TkP = pad_rows(self.Tq), pad_rows(self.Tk)
        self.x = None  # operands of the last prepare()
        self.device = d
        self.q_idx, self.k_idx = e((B, H, TqP)), e((B, H, TkP))
        self.q_bkt = self.k_bkt = None
        self.dev_err = torch.zeros((1,), dtype=i32, device=d)
        if mode == "hash":
            Tp, Tkp = pad_rows(T), pad_rows(Tkv)
            self.bq, self.bk = e((B, H, T)), e((B, H, Tkv))
            self.perm_q, self.perm_k = e((B, H, Tp)), e((B, H, Tkp))
            self.bs_q, self.bs_k = e((B, H, Tp)), e((B, H, Tkp))
            nbs = self.nbs
            self.offq, self.offk = e((B, H, nbs + 1)), e((B, H, nbs + 1))
            self.segq, self.segk = e((B, H, nbs + 1)), e((B, H, nbs + 1))
            self.q_bkt, self.k_bkt = e((B, H, TqP)), e((B, H, TkP))
            self.cq, self.ck = e(chunk_count_shape(B, H, T, nbs)), e(chunk_count_shape(B, H, Tkv, nbs))
        if mode == "dense":
            ar = torch.arange(TqP, dtype=i32, device=d)
            self.q_idx.copy_(torch.where(ar < T, ar, torch.full_like(ar, SCFA_Q_PAD)).expand(B, H, TqP))
            self.k_idx.copy_(torch.where(ar < Tkv, ar, torch.full_like(ar, SCFA_K_PAD)).expand(B, H, TkP))
        Bm, Bn = SCFA_TILE_M, SCFA_TILE_N
        nQt, nKt = TqP // Bm, TkP // Bn
        self.tab = Tables(e((B, H, nQt, 4)), e((B, H, nKt, 4)), e((B, H, nQt, 2)), e((B, H, nKt, 2)), e((B, H)), Bm, Bn,
                          e((B * H * nQt,)), e((B * H * nKt,)) if mode == "hash" else None, bwd_ready=False)
        self.O = e((B, T, H, D), out_dtype)
        self.lse = e((B, H, T), torch.float32)
        self.pairs = e((B, H), torch.int64)
        self._grads = None
        self._bws = None

    # -- stages ---------------------------------------------------------------
    def bucket(self, q, k, R, stream=None, keep_q=None, keep_k=None):
        """LSH buckets and the chunk counts of the sort (queries and keys in
        one launch); the keep masks are required in hash_drop mode."""
        if self.drop and (keep_q is None or keep_k is None):
            raise ScfaError("hash_drop needs the keep masks")
        if not self.two_side:  # queries and keys of different lengths: one launch per side
            if self.drop:
                scfa_hash_bucket_counts_drop(q, R, keep_q, 0, self.nb, self.bq, self.cq, stream)
                scfa_hash_bucket_counts_drop(k, R, keep_k, 1, self.nb, self.bk, self.ck, stream)
            else:
                scfa_hash_bucket_counts(q, R, self.nb, self.bq, self.cq, stream)
                scfa_hash_bucket_counts(k, R, self.nb, self.bk, self.ck, stream)
            return
        scfa_hash_bucket_qk(q, k, R, self.nb, self.bq, self.bk, self.cq, self.ck, stream,
                            keep_q if self.drop else None, keep_k if self.drop else None)

    def sort(self, stream=None):
        """Stable sort by bucket, the bucket-aligned layout and its tile
        statistics (both sides in one launch)."""
        t = self.tab
        if not self.two_side:  # one launch per side; tables() computes the tile statistics
            scfa_hash_layout(self.bq, self.cq, self.nbs, SCFA_TILE_M, SCFA_Q_PAD, self.perm_q, self.bs_q, self.offq,
                             self.q_idx, self.q_bkt, self.segq, self.dev_err, stream)
            scfa_hash_layout(self.bk, self.ck, self.nbs, SCFA_TILE_N, SCFA_K_PAD, self.perm_k, self.bs_k, self.offk,
                             self.k_idx, self.k_bkt, self.segk, self.dev_err, stream)
            return
        scfa_hash_layout_qk(self.bq, self.bk, self.cq, self.ck, self.nbs, self.perm_q, self.perm_k, self.bs_q, self.bs_k,
                            self.offq, self.offk, self.q_idx, self.k_idx, self.q_bkt, self.k_bkt, self.segq, self.segk,
                            self.dev_err, t.qstats, t.kstats, t.tiles, stream)

    def compact(self, q, k, keep_q, keep_k, stream=None):
        """Counts, index arrays and tile statistics of both sides (two
        launches; the operands are read through the index arrays, no
        compacted copies)."""
        t = self.tab
        scfa_qk_index_qk(keep_q, keep_k, self.Tq, self.Tk, self.cnt[0], self.cnt[1], self.mx2, self.choff[0],
                         self.choff[1], self.q_idx, self.k_idx, self.dev_err, stream, t.qstats, t.kstats, t.tiles)

    def tables(self, stream=None):
        """Forward ranges and the launch order, after the tile statistics
        (computed here, or by sort() in hash mode and by compact() in QK
        mode, which also zero the processed-tile counter that this call adds
        to); the backward table is built by backward()."""
        t = self.tab
        t.bwd_ready = False  # new forward ranges: backward() rebuilds the backward table
        mode = _table_mode(self.mode) | self.flags
        # the tile statistics come from the layout launch (hash, one length)
        # or from the compaction (QK); otherwise from a statistics-only call
        if self.mode == "dense" or (self.mode == "hash" and not self.two_side):
            scfa_range_table(mode, self.q_idx, self.k_idx, self.q_bkt, self.k_bkt, self.B, self.H, self.Tq, self.Tk,
                             t.Bm, t.Bn, t.qstats, t.kstats, None, None, t.tiles, stream)
        scfa_fwd_table_order(mode, t.qstats, t.kstats, t.fwd, t.tiles, t.fwd_order, stream)

    def forward(self, stream=None):
        forward(self.prepared(), self.tab, self.out_dtype, self.scale, self.O, self.lse, stream)

    def backward(self, dO, stream=None):
        """Gradients of the last forward() w.r.t. q, k, v (fp32, original order):
        the backward table, then the backward kernels."""
        if self.x is None:
            raise ScfaError("backward needs a prepared forward")
        if self.out_dtype != torch.float32:
            raise ScfaError("backward needs the fp32 forward output")
        if self.mode == "hash":  # one dK/dV workgroup per key tile: longest query ranges first
            scfa_bwd_table_order(self.tab.qstats, self.tab.kstats, self.tab.fwd, self.tab.bwd, self.tab.bwd_order,
                                 stream, self.flags)
        else:
            scfa_bwd_table(self.tab.qstats, self.tab.kstats, self.tab.fwd, self.tab.bwd, stream, self.flags)
        self.tab.bwd_ready = True
        if self._grads is None:
            d = self.device
            self._grads = tuple(torch.empty((self.B, n, self.H, self.D), dtype=torch.float32, device=d)
                                for n in (self.T, self.T_kv, self.T_kv))
            self._bws = torch.empty((scfa_bwd_workspace_bytes(_table_mode(self.mode), self.B, self.H, self.Tq, self.Tk,
                                                              self.D),), dtype=torch.uint8, device=d)
        return backward(self.prepared(), self.tab, self.O, self.lse, dO, self.scale, self._grads, self._bws, stream)

    def count_visible(self, stream=None):
        scfa_count_visible(_table_mode(self.mode) | self.flags, self.q_idx, self.k_idx, self.q_bkt, self.k_bkt, self.B,
                           self.H, self.Tq, self.Tk, self.pairs, stream)
        return self.pairs

    def prepare(self, x: dict, stream=None):
        """All preprocessing stages for inputs x (q, k, v, keep_q, keep_k, R)."""
        if self.mode == "hash":
            if self.drop:
                self.bucket(x["q"], x["k"], x["R"], stream, x["keep_q"], x["keep_k"])
            else:
                self.bucket(x["q"], x["k"], x["R"], stream)
            self.sort(stream)
        elif self.mode == "qk":
            self.compact(x["q"], x["k"], x["keep_q"], x["keep_k"], stream)
        self.x = x
        self.tables(stream)

    def run(self, x: dict, stream=None):
        """Whole forward path: preprocessing, tables, attention."""
        self.prepare(x, stream)
        self.forward(stream)
        return self.O, self.lse

    def capture(self, x: dict):
        """A HIP graph of run(x) (all stages launch on the capturing stream;
        none allocates, synchronises or records a memset). Replay it with
        graph.replay(); the inputs must stay at the same addresses."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):  # warm-up launch on the capture stream
            self.run(x)
        torch.cuda.current_stream(self.device).wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(x)
        return graph

    def prepared(self) -> Prepared:
        if self.x is None:
            raise ScfaError("call prepare() first")
        x = self.x
        return Prepared(self.mode, self.B, self.H, self.T, self.D, self.Tq, self.Tk, x["q"], x["k"], x["v"],
                        self.q_idx, self.k_idx, self.q_bkt, self.k_bkt, strict=self.strict,
                        noncausal=self.noncausal)
