"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects host-visible argument errors before enqueueing anything
(no compute call is made here)."""
import ctypes
import os
import re

import pytest
import torch

import io_aware_attention_head_amd.scfa as scfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scfa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(scfa.LIB_PATH), reason="libscfa.so not built (run __graft_entry__.build())")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(scfa_[a-z0-9_]+)\s*\(", txt)))


def test_header_symbols_exported():
    L = scfa.lib()
    names = _declared()
    assert "scfa_qk_sparse_fwd" in names and "scfa_hash_sparse_fwd" in names
    missing = [n for n in names if getattr(L, n, None) is None]
    assert not missing, missing
    # every declared symbol has a binding signature
    assert not [n for n in names if n not in scfa._SIGS]


def test_status_strings_and_version():
    assert scfa.scfa_status_string(0) == "SCFA_OK"
    for s in (-1, -2, -3):
        assert scfa.scfa_status_string(s).startswith("SCFA_ERR")
    assert scfa.scfa_version() >= 100


def test_invalid_arguments_rejected_without_gpu():
    L = scfa.lib()
    null = None
    dummy = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # NULL pointers
    assert L.scfa_qk_count(null, 1, 8, 1, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    # bad sizes
    assert L.scfa_qk_count(dummy, 0, 8, 1, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    # Tc not a multiple of 128
    assert L.scfa_qk_compact(0, dummy, dummy, dummy, dummy, 1, 8, 1, 64, 100, -1, dummy, dummy, null,
                             null) == scfa.SCFA_ERR_INVALID
    # D != 64
    assert L.scfa_qk_compact(0, dummy, dummy, dummy, dummy, 1, 8, 1, 32, 128, -1, dummy, dummy, null,
                             null) == scfa.SCFA_ERR_UNSUPPORTED
    # odd nb / unsupported nb
    assert L.scfa_hash_bucket(0, dummy, dummy, 1, 8, 1, 64, 15, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_bucket(0, dummy, dummy, 1, 8, 1, 64, 128, dummy, null) == scfa.SCFA_ERR_UNSUPPORTED
    # one-side bucket launch with a keep mask: the mask and the counts are
    # required, side is 0 or 1, nb + 2 buckets must fit 64
    drop = L.scfa_hash_bucket_counts_drop
    assert drop(0, dummy, dummy, null, 0, 1, 8, 1, 64, 16, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert drop(0, dummy, dummy, dummy, 0, 1, 8, 1, 64, 16, dummy, null, null) == scfa.SCFA_ERR_INVALID
    assert drop(0, dummy, dummy, dummy, 2, 1, 8, 1, 64, 16, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert drop(0, dummy, dummy, dummy, -1, 1, 8, 1, 64, 16, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert drop(0, dummy, dummy, dummy, 1, 1, 0, 1, 64, 16, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert drop(0, dummy, dummy, dummy, 1, 1, 8, 1, 64, 64, dummy, dummy, null) == scfa.SCFA_ERR_UNSUPPORTED
    # bad dtype
    assert L.scfa_gather(7, 0, dummy, dummy, 1, 8, 1, 64, 128, dummy, null) == scfa.SCFA_ERR_INVALID
    # bad layout
    assert L.scfa_gather(0, 5, dummy, dummy, 1, 8, 1, 64, 128, dummy, null) == scfa.SCFA_ERR_INVALID
    # workspace too small
    assert L.scfa_hash_sort(dummy, 1, 1, 1000, 16, -1, dummy, dummy, dummy, dummy, 4, null,
                            null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_sort_workspace_bytes(1, 1, 1000, 16) == 4 * 16 * 4
    # tile sizes
    assert L.scfa_range_table(1, dummy, dummy, null, null, 1, 1, 8, 8, 48, 64, dummy, dummy, dummy, dummy, dummy,
                              null) == scfa.SCFA_ERR_INVALID
    # hash mode needs buckets
    assert L.scfa_range_table(2, dummy, dummy, null, null, 1, 1, 8, 8, 128, 64, dummy, dummy, dummy, dummy, dummy,
                              null) == scfa.SCFA_ERR_INVALID
    # forward: bad scale, D, Tc (the launch order may be NULL)
    args = [0, 1] + [dummy] * 8 + [null]
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 8, 128, 64, ctypes.c_float(0.0), 0, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 8, 128, 128, ctypes.c_float(0.125), 0, dummy, dummy,
                                null) == scfa.SCFA_ERR_UNSUPPORTED
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 8, 120, 64, ctypes.c_float(0.125), 0, dummy, dummy,
                                null) == scfa.SCFA_ERR_INVALID
    # one batch entry's T x H x D block of 4 GiB or more (32-bit row offsets)
    assert L.scfa_qk_sparse_fwd(*args, 1, 64, 1 << 20, 1 << 20, 1 << 20, 64, ctypes.c_float(0.125), 0, dummy, dummy,
                                null) == scfa.SCFA_ERR_UNSUPPORTED
    # separate key/value length: zero is rejected, and so is a k/v block of 4 GiB or more
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 0, 128, 64, ctypes.c_float(0.125), 0, dummy, dummy,
                                null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_qk_sparse_fwd(*args, 1, 64, 8, 1 << 20, 128, 64, ctypes.c_float(0.125), 0, dummy, dummy,
                                null) == scfa.SCFA_ERR_UNSUPPORTED
    # flags other than SCFA_STRICT / SCFA_NONCAUSAL, and the two together
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 8, 128, 64, ctypes.c_float(0.125), 4, dummy, dummy,
                                null) == scfa.SCFA_ERR_INVALID
    both = scfa.SCFA_STRICT | scfa.SCFA_NONCAUSAL
    assert L.scfa_qk_sparse_fwd(*args, 1, 1, 8, 8, 128, 64, ctypes.c_float(0.125), both, dummy, dummy,
                                null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table(dummy, dummy, dummy, 1, 1, 2, 2, dummy, 3, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table(dummy, dummy, dummy, 1, 1, 2, 2, dummy, both, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_range_table(1 | both, dummy, dummy, null, null, 1, 1, 8, 8, 128, 64, dummy, dummy, dummy, dummy,
                              dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_count_visible(1 | both, dummy, dummy, null, null, 1, 1, 8, 8, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_workspace_bytes(1 | both, 1, 1, 128, 128, 64) == 0
    assert L.scfa_bwd_workspace_bytes(1 | scfa.SCFA_NONCAUSAL, 1, 1, 128, 128, 64) == \
        L.scfa_bwd_workspace_bytes(1, 1, 1, 128, 128, 64) > 0
    # a mode with the strict flag is accepted where a mode is (argument errors still caught)
    assert L.scfa_range_table(2 | scfa.SCFA_STRICT, dummy, dummy, null, null, 1, 1, 8, 8, 128, 64, dummy, dummy,
                              dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_range_table(7 | scfa.SCFA_STRICT, dummy, dummy, dummy, dummy, 1, 1, 8, 8, 128, 64, dummy, dummy,
                              dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    hargs = [0, 1] + [dummy] * 10
    # hash forward: a NULL table is rejected
    assert L.scfa_hash_sparse_fwd(*hargs[:-1], null, null, 1, 1, 8, 8, 8, 8, 64, ctypes.c_float(0.125), 0, dummy, dummy,
                                  null) == scfa.SCFA_ERR_INVALID
    # bucket-aligned layout: bad alignment, rows below T, size helper
    assert L.scfa_hash_segments(dummy, dummy, 1, 1, 100, 16, 48, -1, 128, dummy, dummy, dummy, null,
                                null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_segments(dummy, dummy, 1, 1, 300, 16, 64, -1, 256, dummy, dummy, dummy, null,
                                null) == scfa.SCFA_ERR_INVALID
    # one-launch sort and layout: bad alignment, rows below T, missing counts or layout outputs, nb above 64
    assert L.scfa_hash_layout(dummy, dummy, 1, 1, 100, 16, 48, -1, 128, dummy, dummy, dummy, dummy, dummy, dummy,
                              null, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout(dummy, dummy, 1, 1, 300, 16, 64, -1, 256, dummy, dummy, dummy, dummy, dummy, dummy,
                              null, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout(dummy, dummy, 1, 1, 300, 16, 64, -1, 512, dummy, dummy, dummy, null, dummy, dummy,
                              null, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout(dummy, null, 1, 1, 300, 16, 0, -1, 0, dummy, dummy, dummy, null, null, null, null,
                              null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout(dummy, dummy, 1, 1, 300, 65, 0, -1, 0, dummy, dummy, dummy, null, null, null, null,
                              null) == scfa.SCFA_ERR_UNSUPPORTED
    assert L.scfa_hash_bucket_counts(0, dummy, dummy, 1, 8, 1, 64, 16, dummy, null, null) == scfa.SCFA_ERR_INVALID
    # two-side entry points: missing counts, NULL key side, rows below T, nb above 64
    assert L.scfa_hash_bucket_qk(0, dummy, dummy, dummy, null, null, 1, 8, 1, 64, 16, dummy, dummy, dummy, null,
                                 null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_bucket_qk(0, dummy, null, dummy, null, null, 1, 8, 1, 64, 16, dummy, dummy, dummy, dummy,
                                 null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_bucket_qk(0, dummy, dummy, dummy, null, null, 1, 8, 1, 32, 16, dummy, dummy, dummy, dummy,
                                 null) == scfa.SCFA_ERR_UNSUPPORTED
    # keep masks: both or neither; nb + 2 sort buckets must fit 64
    assert L.scfa_hash_bucket_qk(0, dummy, dummy, dummy, dummy, null, 1, 8, 1, 64, 16, dummy, dummy, dummy, dummy,
                                 null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_bucket_qk(0, dummy, dummy, dummy, dummy, dummy, 1, 8, 1, 64, 64, dummy, dummy, dummy, dummy,
                                 null) == scfa.SCFA_ERR_UNSUPPORTED
    qk_out = [dummy] * 12 + [null] * 3 + [dummy]  # layouts, no statistics, dev_err
    assert L.scfa_hash_layout_qk(dummy, dummy, dummy, dummy, 1, 1, 300, 16, 256, 384, *qk_out,
                                 null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout_qk(dummy, dummy, dummy, dummy, 1, 1, 300, 16, 384, 384, *qk_out[:11], null,
                                 *qk_out[12:], null) == scfa.SCFA_ERR_INVALID
    # statistics: all three or none
    assert L.scfa_hash_layout_qk(dummy, dummy, dummy, dummy, 1, 1, 300, 16, 384, 384, *qk_out[:12], dummy, null, null,
                                 dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_layout_qk(dummy, dummy, dummy, dummy, 1, 1, 300, 65, 384, 384, *qk_out,
                                 null) == scfa.SCFA_ERR_UNSUPPORTED
    # forward table from statistics: bad mode, NULL counter, bad sizes
    assert L.scfa_fwd_table(7, dummy, dummy, 1, 1, 2, 2, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table(2, dummy, dummy, 1, 1, 2, 2, dummy, null, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table(2, dummy, dummy, 1, 1, 0, 2, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_hash_segment_rows(16384, 16, 128) == 18432
    assert L.scfa_hash_segment_rows(16384, 16, 48) == 0
    # work order: bad sizes, NULL pointers
    assert L.scfa_work_order(dummy, 1, 1, 0, 8, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_work_order(dummy, 1, 1, 8, 16384, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_work_order(null, 1, 1, 8, 8, dummy, null) == scfa.SCFA_ERR_INVALID
    # two-side QK index compaction: NULL pointers, compacted lengths not multiples of 128, too many heads
    qk = [dummy] * 2 + [1, 8, 8, 2, 128, 128] + [dummy] * 7 + [null, null, null, null, null]
    bad = list(qk)
    bad[0] = null
    assert L.scfa_qk_index_qk(*bad) == scfa.SCFA_ERR_INVALID
    bad = list(qk)
    bad[6] = 100
    assert L.scfa_qk_index_qk(*bad) == scfa.SCFA_ERR_INVALID
    bad = list(qk)
    bad[5] = 129
    assert L.scfa_qk_index_qk(*bad) == scfa.SCFA_ERR_INVALID
    bad = list(qk)
    bad[14] = null
    assert L.scfa_qk_index_qk(*bad) == scfa.SCFA_ERR_INVALID
    bad = list(qk)
    bad[15] = dummy  # statistics: all three outputs or none
    assert L.scfa_qk_index_qk(*bad) == scfa.SCFA_ERR_INVALID
    # forward table and order in one launch: bad mode, NULL outputs, bad sizes
    assert L.scfa_fwd_table_order(7, dummy, dummy, 1, 1, 2, 2, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table_order(3, dummy, dummy, 1, 1, 2, 2, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    # range table: statistics only (no forward table) cannot ask for a backward table
    assert L.scfa_range_table(1, dummy, dummy, null, null, 1, 1, 8, 8, 128, 64, dummy, dummy, null, dummy, dummy,
                              null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table_order(2, dummy, dummy, 1, 1, 2, 2, dummy, dummy, null, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table_order(2, dummy, dummy, 1, 1, 2, 16384, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_fwd_table_order(2 | 48, dummy, dummy, 1, 1, 2, 2, dummy, dummy, dummy, null) == scfa.SCFA_ERR_INVALID
    # backward table and order in one launch: NULL inputs or outputs, bad sizes, bad flags
    assert L.scfa_bwd_table_order(dummy, dummy, dummy, 1, 1, 2, 2, dummy, null, 0, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table_order(dummy, dummy, null, 1, 1, 2, 2, dummy, dummy, 0, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table_order(dummy, dummy, dummy, 1, 1, 16384, 2, dummy, dummy, 0, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table_order(dummy, dummy, dummy, 1, 0, 2, 2, dummy, dummy, 0, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table_order(dummy, dummy, dummy, 1, 1, 2, 2, dummy, dummy, both, null) == scfa.SCFA_ERR_INVALID
    assert L.scfa_bwd_table_order(dummy, dummy, dummy, 1, 1, 2, 2, dummy, dummy, 3, null) == scfa.SCFA_ERR_INVALID


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 8, 1, 64)
    with pytest.raises(scfa.ScfaError):
        scfa.scfa_gather(x, torch.zeros(1, 1, 128, dtype=torch.int32), scfa.SCFA_ROWS, torch.zeros(1, 1, 128, 64))
    with pytest.raises(scfa.ScfaError):  # queries and keys of different shapes
        scfa.scfa_hash_bucket_qk(x, torch.zeros(1, 9, 1, 64), torch.zeros(1, 64, 8), 16, *[None] * 4)
    with pytest.raises(scfa.ScfaError):  # one keep mask without the other
        scfa.scfa_hash_bucket_qk(x, x, torch.zeros(1, 64, 8), 16, *[None] * 4, keep_q=torch.ones(1, 8, 1))


def test_header_constants_match_binding():
    txt = open(HEADER).read()
    for name in ("SCFA_TILE_M", "SCFA_TILE_N", "SCFA_ROW_ALIGN", "SCFA_COUNT_CHUNK", "SCFA_K_PAD", "SCFA_STRICT",
                 "SCFA_NONCAUSAL"):
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", txt)
        assert m and int(m.group(1)) == getattr(scfa, name), name


def test_plan_rejects_strict_with_noncausal():
    with pytest.raises(scfa.ScfaError):
        scfa.Plan("hash", 1, 1, 128, strict=True, noncausal=True, device="cpu")


def test_bwd_noalloc_rejects_without_gpu():
    """The no-allocation backward checks its arguments and the size of its
    static scratch before it touches the device."""
    L = scfa.lib()
    null = None
    d = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    f = L.scfa_bwd_noalloc
    # q, k, v, q_idx, k_idx, q_bkt, k_bkt, qstats, kstats, fwd_tab, bwd_tab, fwd_order, bwd_order (optional),
    # O, lse, dO
    ptrs = [d] * 11 + [null, null] + [d] * 3

    def call(mode, ps, B, H, T, Tq, Tk, D=64, dtype=scfa.SCFA_BF16, scale=0.125):
        return f(mode, dtype, *ps, B, H, T, T, Tq, Tk, D, scale, d, d, d, null)

    # NULL operand, NULL gradient, bad mode, fp32, D != 64
    assert call(scfa.SCFA_HASH, [null] + ptrs[1:], 1, 1, 256, 256, 256) == scfa.SCFA_ERR_INVALID
    assert f(scfa.SCFA_HASH, 0, *ptrs, 1, 1, 256, 256, 256, 256, 64, 0.125, null, d, d, null) == scfa.SCFA_ERR_INVALID
    assert call(7, ptrs, 1, 1, 256, 256, 256) == scfa.SCFA_ERR_INVALID
    assert call(scfa.SCFA_HASH | 64, ptrs, 1, 1, 256, 256, 256) == scfa.SCFA_ERR_INVALID
    assert call(scfa.SCFA_HASH, ptrs, 1, 1, 256, 256, 256, dtype=scfa.SCFA_F32) == scfa.SCFA_ERR_UNSUPPORTED
    assert call(scfa.SCFA_HASH, ptrs, 1, 1, 256, 256, 256, D=32) == scfa.SCFA_ERR_UNSUPPORTED
    # workspace beyond the static scratch: 8 bytes per query row of B*H*pad(Tq)
    rows_max = scfa.SCFA_NOALLOC_SCRATCH_BYTES // 8
    assert call(scfa.SCFA_QK, ptrs, 1, 17, 131072, 131072, 131072) == scfa.SCFA_ERR_TOO_LARGE
    assert 17 * 131072 > rows_max
    assert scfa.scfa_status_string(scfa.SCFA_ERR_TOO_LARGE).startswith("SCFA_ERR_TOO_LARGE")


def test_plan_tables_need_backward_table_before_dkdv():
    """A plan's tables carry no backward ranges until the plan's backward()
    builds them: a backward on them is refused on the host (its dK/dV kernel
    would read unwritten ranges)."""
    plan = scfa.Plan("hash", 1, 2, 300, device="cpu")
    q = torch.zeros(1, 300, 2, 64, dtype=torch.bfloat16)
    plan.x = dict(q=q, k=q, v=q, R=torch.zeros(64, 8))
    assert not plan.tab.bwd_ready
    with pytest.raises(scfa.ScfaError, match="backward table"):
        scfa.backward(plan.prepared(), plan.tab, plan.O, plan.lse, q)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more (flag or WORLD_SIZE) it exits
    with status 2 and a message, before it imports torch or touches a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
