"""GPU parity of the integer steps: compaction, LSH bucket, counting sort,
gathers, tile tables and visible-pair counts must equal the oracle BIT FOR
BIT (calls go through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs, small
from gpu_util import announce, f64, need_gpu, np_bits, oracle_buckets, to_dev

pytestmark = pytest.mark.gpu

QK_CASES = [small("qk", 2, 3, 777, keep_p=0.6, seed=21), small("qk", 1, 2, 256, dtype="f32", keep_p=0.7, seed=1),
            small("qk", 1, 1, 1, keep_p=1.0, seed=22), small("qk", 2, 2, 300, keep_p=0.0, seed=23),
            small("qk", 1, 12, 2048, keep_p=0.5, seed=24)]
HASH_CASES = [small("hash", 2, 3, 1000, nb=16, seed=31), small("hash", 1, 2, 1, nb=16, seed=32),
              small("hash", 1, 2, 333, dtype="f32", nb=8, seed=33), small("hash", 1, 4, 4096, nb=64, seed=34),
              small("hash", 2, 2, 700, nb=2, seed=35), small("hash", 1, 2, 700, nb=32, seed=36),
              small("hash", 1, 2, 500, dtype="f32", nb=24, seed=37), small("hash", 1, 3, 600, nb=6, seed=38)]


def _tables_match(mode, pre, tab, Tq, Bm, Bn, q_bkt=None, k_bkt=None, Tk=None):
    Tk = Tq if Tk is None else Tk
    qi = pre.q_idx.cpu().numpy()[:, :, :Tq]
    ki = pre.k_idx.cpu().numpy()[:, :, :Tk]
    qb = None if q_bkt is None else q_bkt.cpu().numpy()[:, :, :Tq]
    kb = None if k_bkt is None else k_bkt.cpu().numpy()[:, :, :Tk]
    ref = oracle.range_tables(mode, qi, ki, qb, kb, Bm, Bn)
    nQ, nK = ref["fwd"].shape[2], ref["bwd"].shape[2]
    qs, ks = tab.qstats.cpu().numpy(), tab.kstats.cpu().numpy()
    fwd, bwd = tab.fwd.cpu().numpy(), tab.bwd.cpu().numpy()
    assert np.array_equal(qs[:, :, :nQ], ref["qstats"])
    assert np.array_equal(ks[:, :, :nK], ref["kstats"])
    assert np.array_equal(fwd[:, :, :nQ], ref["fwd"])
    assert np.array_equal(bwd[:, :, :nK], ref["bwd"])
    assert np.array_equal(tab.tiles.cpu().numpy(), ref["tiles"])
    # tiles beyond the valid rows are empty and never processed
    assert (fwd[:, :, nQ:, 0] == fwd[:, :, nQ:, 1]).all()
    assert (bwd[:, :, nK:] == 0).all()
    assert (ks[:, :, nK:, 0] == scfa.SCFA_K_PAD).all()
    if tab.fwd_order is not None:
        check_order(tab.fwd_order.cpu().numpy(), fwd)
    return ref


def check_order(order, tab, layout="groups"):
    """A launch order is a permutation of the (head, tile) items, longest range
    first within each part, in one of two layouts:
    groups: G groups of heads (head bh in group bh % G; G = 8 when B*H is a
    multiple of 8, else the largest divisor of B*H not above 8), slot s of
    group g at s*G + g;
    runs: 8 runs of consecutive items of equal count (the first N % 8 one
    longer), slot s of run k at s*8 + k."""
    B, H, n, _ = tab.shape
    BH = B * H
    N = BH * n
    assert sorted(order.tolist()) == list(range(N))
    lens = (tab[..., 1] - tab[..., 0]).reshape(N)
    if layout == "groups":
        G = 8 if BH % 8 == 0 else max(g for g in range(1, 8) if BH % g == 0)
        for g in range(G):
            items = order[g::G]
            assert ((items // n) % G == g).all()
            assert (np.diff(lens[items]) <= 0).all()
    else:
        c, r = divmod(N, 8)
        for k in range(8):
            lo, cnt = k * c + min(k, r), c + (1 if k < r else 0)
            items = order[k::8]
            assert len(items) == cnt
            assert sorted(items.tolist()) == list(range(lo, lo + cnt))
            assert (np.diff(lens[items]) <= 0).all()


@pytest.mark.parametrize("w", QK_CASES, ids=lambda w: w.name)
def test_qk_compaction_bitexact(w):
    need_gpu()
    announce(f"qk compaction {w.name}")
    x = make_inputs(w)
    g = to_dev(x)
    pre = scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"], rows=True)
    scfa.gather_operands(pre)  # v_t only: compaction wrote the q and k rows
    torch.cuda.synchronize()
    assert int(pre.extra["dev_err"].item()) == 0
    kq, kk = x["keep_q"].numpy(), x["keep_k"].numpy()
    cq, ck = oracle.qk_count(kq), oracle.qk_count(kk)
    assert np.array_equal(pre.extra["count_q"].cpu().numpy(), cq)
    assert np.array_equal(pre.extra["count_k"].cpu().numpy(), ck)
    assert int(pre.extra["max_q"].item()) == cq.max() and int(pre.extra["max_k"].item()) == ck.max()
    Tc = pre.Tq
    assert Tc == scfa.pad_rows(max(1, int(max(cq.max(), ck.max()))))
    qc, qi = oracle.qk_compact(np_bits(x["q"]), kq, Tc, oracle.Q_PAD)
    kc, ki = oracle.qk_compact(np_bits(x["k"]), kk, Tc, oracle.K_PAD)
    assert np.array_equal(pre.q_idx.cpu().numpy(), qi)
    assert np.array_equal(pre.k_idx.cpu().numpy(), ki)
    assert np.array_equal(np_bits(pre.q), qc)
    assert np.array_equal(np_bits(pre.k), kc)
    vref = oracle.gather_rows(np_bits(x["v"]), ki)
    assert np.array_equal(np_bits(pre.v_t), vref.transpose(0, 1, 3, 2))
    # the same rows through the plain gather (pads zero, as compaction writes them)
    pre2 = scfa.gather_operands(scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"]))
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(pre2.q), qc)
    assert np.array_equal(np_bits(pre2.k), kc)
    tab = scfa.build_tables(pre)
    torch.cuda.synchronize()
    _tables_match("qk", pre, tab, Tc, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N)
    pairs = scfa.count_visible(pre).cpu().numpy()
    assert np.array_equal(pairs, oracle.visible_pairs("qk", w.T, w.B, w.H, kq, kk))


@pytest.mark.parametrize("w", HASH_CASES, ids=lambda w: w.name)
def test_hash_bucket_sort_gather_bitexact(w):
    need_gpu()
    announce(f"hash preprocessing {w.name}")
    x = make_inputs(w)
    g = to_dev(x)
    pre = scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb)
    torch.cuda.synchronize()
    assert int(pre.extra["dev_err"].item()) == 0
    bq, bk = oracle_buckets(w, x)
    assert np.array_equal(pre.extra["bucket_q"].cpu().numpy(), bq)
    assert np.array_equal(pre.extra["bucket_k"].cpu().numpy(), bk)
    assert np.array_equal(pre.extra["chunk_counts_q"].cpu().numpy(), chunk_counts_np(bq, w.nb))
    assert np.array_equal(pre.extra["chunk_counts_k"].cpu().numpy(), chunk_counts_np(bk, w.nb))
    T = w.T
    ex = pre.extra
    sides = ((bq, ex["perm_q"], ex["sorted_bkt_q"], ex["offsets_q"], oracle.Q_PAD, pre.q_idx, pre.q_bkt,
              ex["seg_offsets_q"], scfa.SCFA_TILE_M, pre.Tq),
             (bk, ex["perm_k"], ex["sorted_bkt_k"], ex["offsets_k"], oracle.K_PAD, pre.k_idx, pre.k_bkt,
              ex["seg_offsets_k"], scfa.SCFA_TILE_N, pre.Tk))
    for b_, pperm, pbs, off, pad, sidx, sbkt, soff, align, Tseg in sides:
        perm, bs, offs = oracle.hash_sort(b_, w.nb)
        gi, gb = pperm.cpu().numpy(), pbs.cpu().numpy()
        assert np.array_equal(gi[:, :, :T], perm)
        assert (gi[:, :, T:] == pad).all()
        assert np.array_equal(gb[:, :, :T], bs)
        assert (gb[:, :, T:] == -1).all()
        assert np.array_equal(off.cpu().numpy(), offs)
        # bucket-aligned layout
        assert Tseg == oracle.segment_rows(T, w.nb, align)
        ri, rb, ro = oracle.hash_segments(perm, offs, w.nb, align, pad, Tseg)
        assert np.array_equal(sidx.cpu().numpy(), ri)
        assert np.array_equal(sbkt.cpu().numpy(), rb)
        assert np.array_equal(soff.cpu().numpy(), ro)
    scfa.gather_operands(pre)
    qi, ki = pre.q_idx.cpu().numpy(), pre.k_idx.cpu().numpy()
    assert np.array_equal(np_bits(pre.q), oracle.gather_rows(np_bits(x["q"]), qi))
    assert np.array_equal(np_bits(pre.k), oracle.gather_rows(np_bits(x["k"]), ki))
    assert np.array_equal(np_bits(pre.v_t), oracle.gather_rows(np_bits(x["v"]), ki).transpose(0, 1, 3, 2))
    tab = scfa.build_tables(pre)
    torch.cuda.synchronize()
    _tables_match("hash", pre, tab, pre.Tq, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N, pre.q_bkt, pre.k_bkt, pre.Tk)
    pairs = scfa.count_visible(pre).cpu().numpy()
    assert np.array_equal(pairs, oracle.visible_pairs("hash", T, w.B, w.H, bkt_q=bq, bkt_k=bk))


@pytest.mark.parametrize("Bm,Bn", [(16, 16), (32, 64), (64, 128), (128, 32), (128, 128)])
def test_tables_any_tile_size(Bm, Bn):
    """Tile-size invariance of the table rules: the GPU tables equal the
    oracle's for every supported tile shape, in all three modes."""
    need_gpu()
    announce(f"tables Bm={Bm} Bn={Bn}")
    for w in (small("hash", 1, 2, 900, nb=8, seed=41), small("qk", 1, 2, 900, keep_p=0.5, seed=42)):
        x = make_inputs(w)
        g = to_dev(x)
        pre = (scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb) if w.mode == "hash"
               else scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"]))
        tab = scfa.build_tables(pre, Bm, Bn)
        torch.cuda.synchronize()
        ref = _tables_match(w.mode, pre, tab, pre.Tq, Bm, Bn, pre.q_bkt, pre.k_bkt, pre.Tk)
        assert ref["tiles"].sum() > 0
    # dense mode of the table call (positions = row numbers, no index arrays)
    T = 1000
    B, H = 1, 2
    nQt, nKt = scfa.pad_rows(T) // Bm, scfa.pad_rows(T) // Bn
    i32 = torch.int32
    d = torch.device("cuda:0")
    t = [torch.empty(s, dtype=i32, device=d) for s in ((B, H, nQt, 4), (B, H, nKt, 4), (B, H, nQt, 2), (B, H, nKt, 2),
                                                      (B, H))]
    scfa.scfa_range_table(scfa.SCFA_DENSE, None, None, None, None, B, H, T, T, Bm, Bn, *t)
    torch.cuda.synchronize()
    a = np.broadcast_to(np.arange(T, dtype=np.int32), (B, H, T)).copy()
    ref = oracle.range_tables("dense", a, a, None, None, Bm, Bn)
    nQ, nK = ref["fwd"].shape[2], ref["bwd"].shape[2]
    assert np.array_equal(t[2].cpu().numpy()[:, :, :nQ], ref["fwd"])
    assert np.array_equal(t[3].cpu().numpy()[:, :, :nK], ref["bwd"])
    assert np.array_equal(t[4].cpu().numpy(), ref["tiles"])


def test_backward_table_separately():
    """A forward-only table call (no backward table) followed by
    scfa_bwd_table gives the backward table of the full call."""
    need_gpu()
    announce("backward table separately")
    w = small("hash", 1, 2, 3000, nb=8, seed=44)
    x = make_inputs(w)
    g = to_dev(x)
    pre = scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb)
    tab = scfa.build_tables(pre)
    t2 = [torch.full_like(a, -5) for a in (tab.qstats, tab.kstats, tab.fwd, tab.bwd, tab.tiles)]
    scfa.scfa_range_table(scfa.SCFA_HASH, pre.q_idx, pre.k_idx, pre.q_bkt, pre.k_bkt, w.B, w.H, pre.Tq, pre.Tk,
                          tab.Bm, tab.Bn, t2[0], t2[1], t2[2], None, t2[4])
    torch.cuda.synchronize()
    assert (t2[3] == -5).all()  # not written
    scfa.scfa_bwd_table(t2[0], t2[1], t2[2], t2[3])
    torch.cuda.synchronize()
    for a, b in zip((tab.qstats, tab.kstats, tab.fwd, tab.bwd, tab.tiles), t2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode,T", [("hash", 9000), ("qk", 9000), ("hash", 17000)])
def test_tables_more_than_512_tiles(mode, T):
    """More than 512 tiles per head on both sides: the table kernels' chunked
    loop (instead of the register path) against the oracle, plus the launch
    order."""
    need_gpu()
    announce(f"tables >512 tiles {mode} T={T}")
    w = small(mode, 1, 2, T, nb=16, keep_p=0.95, seed=43)
    x = make_inputs(w)
    g = to_dev(x)
    pre = (scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb) if mode == "hash"
           else scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"]))
    tab = scfa.build_tables(pre, 16, 16)
    torch.cuda.synchronize()
    assert tab.fwd.shape[2] > 512 and tab.bwd.shape[2] > 512
    ref = _tables_match(mode, pre, tab, pre.Tq, 16, 16, pre.q_bkt, pre.k_bkt, pre.Tk)
    assert ref["tiles"].sum() > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hash_bucket_near_ties(dtype):
    """LSH buckets on inputs built to sit at or near ties, bit-exact against
    the float64 definition: rotations with two equal columns (exact ties
    between buckets 0 and 1 for every token), a column equal to minus another
    (ties between a positive and a negative candidate), tokens whose two
    largest projections differ by rounding only, and all-zero tokens (every
    candidate equal). These are the tokens the float32 pass must hand to the
    float64 one."""
    need_gpu()
    announce(f"hash bucket near ties {dtype}")
    rng = np.random.default_rng(91)
    B, T, H, D, nb = 1, 3000, 2, 64, 16
    half = nb // 2
    R = rng.standard_normal((H, D, half)).astype(np.float32)
    R[0, :, 1] = R[0, :, 0]   # c_1 == c_0 exactly
    R[1, :, 3] = -R[1, :, 2]  # -c_3 == c_2 exactly
    x = rng.standard_normal((B, T, H, D))
    for h in range(H):
        for t in range(0, T, 3):  # every third token: two columns nearly tied as the largest
            # two columns whose difference is nonzero (head 0 has two equal
            # columns: that pair is tied for every token already)
            while True:
                j1, j2 = rng.choice(half, 2, replace=False)
                u = R[h, :, j1].astype(np.float64) - R[h, :, j2]
                if u @ u > 0:
                    break
            v = R[h, :, j1].astype(np.float64) + R[h, :, j2] + 0.1 * rng.standard_normal(D)
            x[0, t, h] = v - (v @ u) / (u @ u) * u
        x[0, 7::97, h] = 0.0  # all-zero tokens
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt = torch.from_numpy(x.astype(np.float32)).to(tdt)
    x64 = xt.double().numpy()
    assert np.isfinite(x64).all()
    ref = oracle.hash_bucket(x64, R.astype(np.float64), nb)
    d = torch.device("cuda:0")
    got = torch.empty((B, H, T), dtype=torch.int32, device=d)
    cnt = torch.empty(scfa.chunk_count_shape(B, H, T, nb), dtype=torch.int32, device=d)
    scfa.scfa_hash_bucket_counts(xt.to(d), torch.from_numpy(R).to(d), nb, got, cnt)
    got2 = torch.empty_like(got)
    scfa.scfa_hash_bucket(xt.to(d), torch.from_numpy(R).to(d), nb, got2)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(g, ref), f"{int((g != ref).sum())} buckets differ"
    assert torch.equal(got, got2)
    assert np.array_equal(cnt.cpu().numpy(), chunk_counts_np(ref, nb))
    # exact ties go to the first candidate: head 0 never picks 1 or 9 (tied
    # with 0 and 8), head 1 never 10 or 11 (tied with 3 and 2); zero tokens
    # pick 0
    assert not np.isin(ref[0, 0], [1, half + 1]).any()
    assert not np.isin(ref[0, 1], [half + 2, half + 3]).any()
    assert (ref[:, :, 7::97] == 0).all()


def chunk_counts_np(b_np, nb):
    """Tokens of each bucket among positions [256 c, 256 c + 256) of each head."""
    B, H, T = b_np.shape
    nC = (T + 255) // 256
    out = np.zeros((B, H, nC, nb), dtype=np.int32)
    for c in range(nC):
        blk = b_np[:, :, 256 * c:256 * (c + 1)]
        for v in range(nb):
            out[:, :, c, v] = (blk == v).sum(-1)
    return out


@pytest.mark.parametrize("T,nb,align,dist", [(1, 1, 0, "uniform"), (63, 3, 16, "uniform"), (300, 16, 128, "uniform"),
                                              (1000, 64, 64, "uniform"), (4100, 16, 64, "skewed"),
                                              (16384, 16, 128, "uniform"), (777, 8, 32, "one"),
                                              (2049, 5, 0, "skewed"), (40000, 16, 64, "uniform")])
def test_hash_layout_bitexact(T, nb, align, dist):
    """The one-launch sort and layout against the oracle's sort and
    bucket-aligned layout, and against the two-stage entry points
    (scfa_hash_sort then scfa_hash_segments) on the same buckets: ragged
    lengths, empty buckets, one bucket holding everything, nb up to 64."""
    need_gpu()
    announce(f"hash layout T={T} nb={nb} align={align} {dist}")
    d = torch.device("cuda:0")
    B, H = 2, 3
    rng = np.random.default_rng(T * 131 + nb)
    if dist == "uniform":
        b_np = rng.integers(0, nb, (B, H, T)).astype(np.int32)
    elif dist == "skewed":  # most tokens in bucket 0, a few elsewhere, some buckets empty
        b_np = np.where(rng.random((B, H, T)) < 0.9, 0, rng.integers(0, nb, (B, H, T))).astype(np.int32)
    else:
        b_np = np.full((B, H, T), nb - 1, dtype=np.int32)
    bucket = torch.from_numpy(b_np).to(d)
    counts = torch.from_numpy(chunk_counts_np(b_np, nb)).to(d)
    Tp = scfa.pad_rows(T)
    i32 = torch.int32
    out = {k: torch.full(shape, -7, dtype=i32, device=d) for k, shape in
           (("perm", (B, H, Tp)), ("bs", (B, H, Tp)), ("off", (B, H, nb + 1)))}
    err = torch.zeros(1, dtype=i32, device=d)
    pad = oracle.K_PAD
    perm, bs, offs = oracle.hash_sort(b_np, nb)
    if align:
        Tseg = scfa.scfa_hash_segment_rows(T, nb, align)
        seg = {k: torch.full(shape, -7, dtype=i32, device=d) for k, shape in
               (("idx", (B, H, Tseg)), ("bkt", (B, H, Tseg)), ("so", (B, H, nb + 1)))}
        scfa.scfa_hash_layout(bucket, counts, nb, align, pad, out["perm"], out["bs"], out["off"], seg["idx"],
                              seg["bkt"], seg["so"], err)
    else:
        scfa.scfa_hash_layout(bucket, counts, nb, 0, pad, out["perm"], out["bs"], out["off"], dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    gp, gb = out["perm"].cpu().numpy(), out["bs"].cpu().numpy()
    assert np.array_equal(gp[:, :, :T], perm) and (gp[:, :, T:] == pad).all()
    assert np.array_equal(gb[:, :, :T], bs) and (gb[:, :, T:] == -1).all()
    assert np.array_equal(out["off"].cpu().numpy(), offs)
    # the two-stage entry points give the same bits
    ws = torch.empty(max(1, scfa.scfa_hash_sort_workspace_bytes(B, H, T, nb)), dtype=torch.uint8, device=d)
    p2, b2, o2 = torch.empty_like(out["perm"]), torch.empty_like(out["bs"]), torch.empty_like(out["off"])
    scfa.scfa_hash_sort(bucket, nb, pad, p2, b2, o2, ws, err)
    if align:
        ri, rb, ro = oracle.hash_segments(perm, offs, nb, align, pad, Tseg)
        i2, k2, s2 = torch.empty_like(seg["idx"]), torch.empty_like(seg["bkt"]), torch.empty_like(seg["so"])
        scfa.scfa_hash_segments(p2, o2, T, nb, align, pad, i2, k2, s2, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(p2, out["perm"]) and torch.equal(b2, out["bs"]) and torch.equal(o2, out["off"])
    if align:
        assert np.array_equal(seg["idx"].cpu().numpy(), ri)
        assert np.array_equal(seg["bkt"].cpu().numpy(), rb)
        assert np.array_equal(seg["so"].cpu().numpy(), ro)
        assert torch.equal(i2, seg["idx"]) and torch.equal(k2, seg["bkt"]) and torch.equal(s2, seg["so"])


def test_hash_layout_device_errors():
    """scfa_hash_layout flags a bucket outside [0, nb) and a layout that
    overflows the given rows."""
    need_gpu()
    announce("hash layout device errors")
    d = torch.device("cuda:0")
    i32 = torch.int32
    T, nb = 300, 16
    Tp = scfa.pad_rows(T)
    perm, bs = torch.empty((1, 1, Tp), dtype=i32, device=d), torch.empty((1, 1, Tp), dtype=i32, device=d)
    off = torch.empty((1, 1, nb + 1), dtype=i32, device=d)
    err = torch.zeros(1, dtype=i32, device=d)
    bucket = (torch.arange(T, dtype=i32, device=d) % nb).reshape(1, 1, T).contiguous()
    bucket[0, 0, 5] = -2
    counts = torch.from_numpy(chunk_counts_np(bucket.cpu().numpy(), nb)).to(d)
    scfa.scfa_hash_layout(bucket, counts, nb, 0, -1, perm, bs, off, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == scfa.SCFA_DEVERR_BUCKET_RANGE
    bucket[0, 0, 5] = 5
    counts = torch.from_numpy(chunk_counts_np(bucket.cpu().numpy(), nb)).to(d)
    seg_i = torch.empty((1, 1, 384), dtype=i32, device=d)
    seg_b, seg_o = torch.empty_like(seg_i), torch.empty((1, 1, nb + 1), dtype=i32, device=d)
    err.zero_()
    scfa.scfa_hash_layout(bucket, counts, nb, 128, -1, perm, bs, off, seg_i, seg_b, seg_o, err)
    torch.cuda.synchronize()
    assert int(err.item()) == scfa.SCFA_DEVERR_SEGMENT_OVERFLOW
    assert seg_o.cpu().numpy()[0, 0, nb] == nb * 128


def test_device_error_flags():
    """Data errors only the device sees set dev_err (no host sync needed)."""
    need_gpu()
    announce("device error flags")
    d = torch.device("cuda:0")
    # a bucket id outside [0, nb)
    B, H, T, nb = 1, 1, 300, 8
    bucket = torch.randint(0, nb, (B, H, T), dtype=torch.int32, device=d)
    bucket[0, 0, 17] = nb + 3
    ws = torch.empty(scfa.scfa_hash_sort_workspace_bytes(B, H, T, nb), dtype=torch.uint8, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    Tp = scfa.pad_rows(T)
    perm = torch.empty((B, H, Tp), dtype=torch.int32, device=d)
    bs = torch.empty_like(perm)
    off = torch.empty((B, H, nb + 1), dtype=torch.int32, device=d)
    scfa.scfa_hash_sort(bucket, nb, -1, perm, bs, off, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) & scfa.SCFA_DEVERR_BUCKET_RANGE
    # a bucket-aligned layout that does not fit the given number of rows: 16
    # buckets of about 19 tokens each need 16 x 128 rows, 256 are given
    bucket = (torch.arange(300, dtype=torch.int32, device=d) % 16).reshape(1, 1, 300).contiguous()
    ws16 = torch.empty(scfa.scfa_hash_sort_workspace_bytes(1, 1, 300, 16), dtype=torch.uint8, device=d)
    off16 = torch.empty((1, 1, 17), dtype=torch.int32, device=d)
    err.zero_()
    scfa.scfa_hash_sort(bucket, 16, -1, perm, bs, off16, ws16, err)
    seg_i = torch.empty((1, 1, 384), dtype=torch.int32, device=d)
    seg_b, seg_o = torch.empty_like(seg_i), torch.empty((1, 1, 17), dtype=torch.int32, device=d)
    scfa.scfa_hash_segments(perm, off16, 300, 16, 128, -1, seg_i, seg_b, seg_o, err)
    torch.cuda.synchronize()
    assert int(err.item()) == scfa.SCFA_DEVERR_SEGMENT_OVERFLOW
    assert seg_o.cpu().numpy()[0, 0, 16] == 16 * 128
    # a kept count above the compacted length
    keep = torch.ones((1, 200, 1), dtype=torch.uint8, device=d)
    x = torch.zeros((1, 200, 1, 64), dtype=torch.bfloat16, device=d)
    cnt = torch.empty((1, 1), dtype=torch.int32, device=d)
    mx = torch.empty((1,), dtype=torch.int32, device=d)
    co = torch.empty((1, 1, 4), dtype=torch.int32, device=d)
    scfa.scfa_qk_count(keep, cnt, mx, co)
    err.zero_()
    xc = torch.empty((1, 1, 128, 64), dtype=torch.bfloat16, device=d)
    idx = torch.empty((1, 1, 128), dtype=torch.int32, device=d)
    scfa.scfa_qk_compact(x, keep, cnt, co, 128, -1, xc, idx, err)
    torch.cuda.synchronize()
    assert int(err.item()) & scfa.SCFA_DEVERR_COUNT_EXCEEDS_TC
    assert idx.cpu().numpy().tolist()[0][0] == list(range(128))


@pytest.mark.parametrize("name", ["qk_bf16_t8192_keep0.7", "qk_bf16_t8192_keep0.5", "hash_bf16_t16384_nb16"])
def test_full_size_preprocessing_bitexact(name):
    """Full-size workloads: every integer output bit-exact against the oracle."""
    need_gpu()
    w = WORKLOADS[name]
    announce(f"full-size preprocessing {name}")
    x = make_inputs(w)
    g = to_dev(x)
    if w.mode == "hash":
        pre = scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb)
        torch.cuda.synchronize()
        bq, bk = oracle_buckets(w, x)
        assert np.array_equal(pre.extra["bucket_q"].cpu().numpy(), bq)
        assert np.array_equal(pre.extra["bucket_k"].cpu().numpy(), bk)
        perm, bs, offs = oracle.hash_sort(bk, w.nb)
        assert np.array_equal(pre.extra["perm_k"].cpu().numpy()[:, :, :w.T], perm)
        ri, rb, _ = oracle.hash_segments(perm, offs, w.nb, scfa.SCFA_TILE_N, oracle.K_PAD, pre.Tk)
        assert np.array_equal(pre.k_idx.cpu().numpy(), ri)
        assert np.array_equal(pre.k_bkt.cpu().numpy(), rb)
        mode = "hash"
    else:
        pre = scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"])
        torch.cuda.synchronize()
        _, ki = oracle.qk_compact(None, x["keep_k"].numpy(), pre.Tq, oracle.K_PAD)
        assert np.array_equal(pre.k_idx.cpu().numpy(), ki)
        mode = "qk"
    tab = scfa.build_tables(pre)
    torch.cuda.synchronize()
    _tables_match(mode, pre, tab, pre.Tq, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N, pre.q_bkt, pre.k_bkt, pre.Tk)


def _qk_stats(rng, BH, nQt, nKt, ordered=True):
    """Tile statistics shaped like the QK and dense modes' (buckets 0): real
    tiles with ascending positions, then pad tiles; or, unordered, real tiles
    with random positions."""
    qs = np.empty((BH, nQt, 4), np.int32)
    ks = np.empty((BH, nKt, 4), np.int32)
    for st, n, pad, zw, rows in ((qs, nQt, oracle.Q_PAD, (2**31 - 1, -2**31), scfa.SCFA_TILE_M),
                                 (ks, nKt, oracle.K_PAD, (2**31 - 1, 2**31 - 1), scfa.SCFA_TILE_N)):
        for h in range(BH):
            nreal = int(rng.integers(1, n + 1))
            lo = np.sort(rng.integers(0, 40 * n * rows, nreal)) if ordered else rng.integers(0, 40 * n * rows, nreal)
            st[h, :nreal, 0] = lo
            st[h, :nreal, 1] = lo + rng.integers(0, 3 * rows, nreal)
            st[h, :nreal, 2:] = 0
            st[h, nreal:] = (pad, pad, zw[0], zw[1])
    return qs, ks


@pytest.mark.parametrize("case", [(1, 12, 64, 128, scfa.SCFA_QK), (2, 12, 64, 128, scfa.SCFA_QK | scfa.SCFA_STRICT),
                                  (2, 4, 33, 70, scfa.SCFA_QK | scfa.SCFA_NONCAUSAL), (1, 3, 40, 4000, scfa.SCFA_QK),
                                  (1, 2, 16, 32, scfa.SCFA_DENSE), (1, 5, 9, 1, scfa.SCFA_QK)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("kind", ["ordered", "random"])
def test_fwd_table_order_qk_matches_two_launches(case, kind):
    """The one-launch forward table and order in the QK and dense modes
    (Algorithm 1) against scfa_fwd_table followed by scfa_work_order: the
    same table and tile count bit for bit and a valid longest-first order,
    on position-ordered statistics (the searched path) and on unordered ones
    (the tile-by-tile count); (1, 3, 40, 4000) takes the two-launch
    fallback."""
    need_gpu()
    B, H, nQt, nKt, mode = case
    announce(f"fwd table + order qk {kind} {case}")
    rng = np.random.default_rng(sum(case) + (5 if kind == "random" else 2))
    qs, ks = _qk_stats(rng, B * H, nQt, nKt, ordered=(kind == "ordered"))
    dev = torch.device("cuda:0")
    qst = torch.from_numpy(qs).reshape(B, H, nQt, 4).to(dev)
    kst = torch.from_numpy(ks).reshape(B, H, nKt, 4).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ref_tab, ref_tiles, ref_order = (torch.empty((B, H, nQt, 2), **i32), torch.zeros((B, H), **i32),
                                     torch.empty((B * H * nQt,), **i32))
    scfa.scfa_fwd_table(mode, qst, kst, ref_tab, ref_tiles)
    scfa.scfa_work_order(ref_tab, nKt, ref_order)
    tab, tiles, order = (torch.empty((B, H, nQt, 2), **i32), torch.zeros((B, H), **i32),
                         torch.empty((B * H * nQt,), **i32))
    scfa.scfa_fwd_table_order(mode, qst, kst, tab, tiles, order)
    torch.cuda.synchronize()
    assert torch.equal(tab, ref_tab)
    assert torch.equal(tiles, ref_tiles)
    check_order(order.cpu().numpy(), tab.cpu().numpy())


@pytest.mark.parametrize("w", [WORKLOADS["hash_bf16_t16384_nb16"], small("hash", 1, 2, 700, dtype="f32", nb=24, seed=81),
                               small("hash", 2, 2, 1000, nb=64, seed=82), small("hash", 1, 3, 1, nb=16, seed=83)],
                         ids=lambda w: w.name)
def test_plan_two_side_launches_bitexact(w):
    """The Plan's one-launch-per-stage entry points (queries and keys in one
    grid): buckets, chunk counts, sort and both aligned layouts bit-exact
    against the oracle, as the one-side entry points are."""
    need_gpu()
    announce(f"two-side preprocessing {w.name}")
    x = make_inputs(w)
    g = to_dev(x)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, dt, nb=w.nb)
    plan.prepare(g)
    torch.cuda.synchronize()
    assert int(plan.dev_err.item()) == 0
    bq, bk = oracle_buckets(w, x)
    for b_, bg, cg, pg, bsg, og, ig, kg, sg, align, pad, Tseg in (
            (bq, plan.bq, plan.cq, plan.perm_q, plan.bs_q, plan.offq, plan.q_idx, plan.q_bkt, plan.segq,
             scfa.SCFA_TILE_M, oracle.Q_PAD, plan.Tq),
            (bk, plan.bk, plan.ck, plan.perm_k, plan.bs_k, plan.offk, plan.k_idx, plan.k_bkt, plan.segk,
             scfa.SCFA_TILE_N, oracle.K_PAD, plan.Tk)):
        assert np.array_equal(bg.cpu().numpy(), b_)
        assert np.array_equal(cg.cpu().numpy(), chunk_counts_np(b_, w.nb))
        perm, bs, offs = oracle.hash_sort(b_, w.nb)
        assert np.array_equal(pg.cpu().numpy()[:, :, :w.T], perm)
        assert np.array_equal(bsg.cpu().numpy()[:, :, :w.T], bs)
        assert np.array_equal(og.cpu().numpy(), offs)
        ri, rb, ro = oracle.hash_segments(perm, offs, w.nb, align, pad, Tseg)
        assert np.array_equal(ig.cpu().numpy()[:, :, :Tseg], ri)
        assert np.array_equal(kg.cpu().numpy()[:, :, :Tseg], rb)
        assert np.array_equal(sg.cpu().numpy(), ro)
    # tile statistics from the layout launch and the forward table built on
    # them: the same as the tables built from the index arrays
    ref = scfa.build_tables(plan.prepared())
    torch.cuda.synchronize()
    for name in ("qstats", "kstats", "fwd", "tiles"):
        assert torch.equal(getattr(plan.tab, name), getattr(ref, name)), name
    # the Plan's launch order over its forward table
    check_order(plan.tab.fwd_order.cpu().numpy(), plan.tab.fwd.cpu().numpy(),
                "groups" if (w.B * w.H) % 8 == 0 else "runs")


def _layout_stats(rng, BH, nQt, nKt, nb):
    """Tile statistics shaped like the bucket-aligned layout's: every tile one
    bucket, buckets non-decreasing, positions ascending within a bucket, pad
    tiles (bucket nb) at the end of each side."""
    qs = np.empty((BH, nQt, 4), np.int32)
    ks = np.empty((BH, nKt, 4), np.int32)
    for st, n, pad, rows in ((qs, nQt, oracle.Q_PAD, scfa.SCFA_TILE_M), (ks, nKt, oracle.K_PAD, scfa.SCFA_TILE_N)):
        for h in range(BH):
            nreal = int(rng.integers(max(1, n // 2), n + 1))
            bk = np.sort(rng.integers(0, nb, nreal))
            pos = np.empty(nreal, np.int64)
            for v in range(nb):  # positions ascend within each bucket
                m = bk == v
                pos[m] = np.sort(rng.integers(0, 50 * n * rows, int(m.sum())))
            st[h, :nreal, 0] = pos
            st[h, :nreal, 1] = pos + rng.integers(0, 3 * rows, nreal)
            st[h, :nreal, 2] = bk
            st[h, :nreal, 3] = bk
            st[h, nreal:] = (pad, pad, nb, nb)
    return qs, ks


@pytest.mark.parametrize("case", [(2, 12, 144, 272, 16, 0), (1, 3, 20, 40, 8, 0), (2, 4, 64, 130, 4, scfa.SCFA_STRICT),
                                  (1, 8, 30, 70, 6, scfa.SCFA_NONCAUSAL), (1, 3, 40, 4000, 16, 0), (1, 3, 40, 1300, 16, 0),
                                  (1, 5, 9, 2, 2, 0)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("kind", ["layout", "random"])
def test_fwd_table_order_matches_two_launches(case, kind):
    """The one-launch forward table and order against scfa_fwd_table followed
    by scfa_work_order: the same table and tile count, bit for bit, and a
    valid longest-first order, on statistics shaped like the aligned layout's
    (the searched path) and on random statistics (the tile-by-tile path);
    (1, 3, 40, 4000) is too large for one workgroup's LDS (the two-launch
    fallback inside the call, with scfa_work_order's groups); the other
    cases with B*H not a multiple of 8 take the runs layout."""
    need_gpu()
    B, H, nQt, nKt, nb, flags = case
    announce(f"fwd table + order {kind} {case}")
    rng = np.random.default_rng(sum(case) + (7 if kind == "random" else 0))
    if kind == "layout":
        qs, ks = _layout_stats(rng, B * H, nQt, nKt, nb)
    else:
        qs = rng.integers(-5, 4000, (B * H, nQt, 4)).astype(np.int32)
        ks = rng.integers(-5, 4000, (B * H, nKt, 4)).astype(np.int32)
        qs[..., 2:] = np.sort(rng.integers(0, nb, (B * H, nQt, 2)), axis=-1)
        ks[..., 2:] = np.sort(rng.integers(0, nb, (B * H, nKt, 2)), axis=-1)
    dev = torch.device("cuda:0")
    qst = torch.from_numpy(qs).reshape(B, H, nQt, 4).to(dev)
    kst = torch.from_numpy(ks).reshape(B, H, nKt, 4).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    mode = scfa.SCFA_HASH | flags
    ref_tab, ref_tiles, ref_order = (torch.empty((B, H, nQt, 2), **i32), torch.zeros((B, H), **i32),
                                     torch.empty((B * H * nQt,), **i32))
    scfa.scfa_fwd_table(mode, qst, kst, ref_tab, ref_tiles)
    scfa.scfa_work_order(ref_tab, nKt, ref_order)
    tab, tiles, order = (torch.empty((B, H, nQt, 2), **i32), torch.zeros((B, H), **i32),
                         torch.empty((B * H * nQt,), **i32))
    scfa.scfa_fwd_table_order(mode, qst, kst, tab, tiles, order)
    torch.cuda.synchronize()
    assert torch.equal(tab, ref_tab)
    assert torch.equal(tiles, ref_tiles)
    fallback = nKt >= 4000  # too large for one workgroup: scfa_work_order's groups
    check_order(order.cpu().numpy(), tab.cpu().numpy(), "groups" if fallback or (B * H) % 8 == 0 else "runs")


@pytest.mark.parametrize("case", [(2, 8192, 8192, 12, 0.5, 8192, 8192), (1, 300, 777, 3, 0.6, 384, 896),
                                  (1, 1, 1, 2, 1.0, 128, 128), (2, 1000, 200, 5, 0.0, 1024, 256),
                                  (1, 777, 300, 16, 0.9, 896, 384), (2, 100, 130, 4, 0.7, 512, 256)],
                         ids=lambda c: "x".join(map(str, c)))
def test_qk_index_two_sides_matches_one_side_calls(case):
    """The two-side index compaction against scfa_qk_count and scfa_qk_compact
    (index only) per side: counts, max counts and index arrays bit for bit,
    with compacted lengths above the kept counts and above T."""
    need_gpu()
    B, T, Tkv, H, p, Tq, Tk = case
    announce(f"qk index two sides {case}")
    g = torch.Generator().manual_seed(sum(case[:4]))
    dev = torch.device("cuda:0")
    keep_q = (torch.rand((B, T, H), generator=g) < p).to(torch.uint8).to(dev)
    keep_k = (torch.rand((B, Tkv, H), generator=g) < p).to(torch.uint8).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    nCq, nCk = (T + 63) // 64, (Tkv + 63) // 64
    ref = {"cq": torch.empty((B, H), **i32), "ck": torch.empty((B, H), **i32), "mq": torch.empty((1,), **i32),
           "mk": torch.empty((1,), **i32), "oq": torch.empty((B, H, nCq), **i32), "ok": torch.empty((B, H, nCk), **i32),
           "iq": torch.empty((B, H, Tq), **i32), "ik": torch.empty((B, H, Tk), **i32)}
    scfa.scfa_qk_count(keep_q, ref["cq"], ref["mq"], ref["oq"])
    scfa.scfa_qk_count(keep_k, ref["ck"], ref["mk"], ref["ok"])
    scfa.scfa_qk_compact(None, keep_q, ref["cq"], ref["oq"], Tq, scfa.SCFA_Q_PAD, None, ref["iq"])
    scfa.scfa_qk_compact(None, keep_k, ref["ck"], ref["ok"], Tk, scfa.SCFA_K_PAD, None, ref["ik"])
    # tile statistics of the attention tiles over every row of the index arrays
    nQt, nKt = Tq // scfa.SCFA_TILE_M, Tk // scfa.SCFA_TILE_N
    ref["qs"], ref["ks"] = torch.empty((B, H, nQt, 4), **i32), torch.empty((B, H, nKt, 4), **i32)
    ref["tiles"] = torch.full((B, H), -7, **i32)
    scfa.scfa_range_table(scfa.SCFA_QK, ref["iq"], ref["ik"], None, None, B, H, Tq, Tk, scfa.SCFA_TILE_M,
                          scfa.SCFA_TILE_N, ref["qs"], ref["ks"], None, None, ref["tiles"])
    got = {k: torch.full_like(v, -7) for k, v in ref.items()}
    mx = torch.full((2,), -7, **i32)
    err = torch.zeros((1,), **i32)
    scfa.scfa_qk_index_qk(keep_q, keep_k, Tq, Tk, got["cq"], got["ck"], mx, got["oq"], got["ok"], got["iq"], got["ik"],
                          err, qstats=got["qs"], kstats=got["ks"], tiles=got["tiles"])
    torch.cuda.synchronize()
    for name in ("cq", "ck", "iq", "ik", "qs", "ks", "tiles"):
        assert torch.equal(got[name], ref[name]), name
    assert int(mx[0]) == int(ref["mq"][0]) and int(mx[1]) == int(ref["mk"][0])
    assert int(err.item()) == 0


@pytest.mark.parametrize("case", [(1, 12, 135, 272, 16, 0, "layout"), (2, 12, 144, 272, 16, 0, "layout"),
                                  (1, 3, 20, 40, 8, scfa.SCFA_STRICT, "layout"),
                                  (1, 8, 30, 70, 6, scfa.SCFA_NONCAUSAL, "layout"), (1, 1, 9, 2, 2, 0, "layout"),
                                  (1, 12, 40, 80, 4, 0, "random"), (2, 4, 33, 70, 4, scfa.SCFA_STRICT, "random"),
                                  (1, 5, 64, 128, 1, 0, "qk"), (2, 3, 33, 65, 1, scfa.SCFA_NONCAUSAL, "qk"),
                                  (65, 8, 1, 2, 2, 0, "layout"), (1, 1, 4000, 8000, 16, 0, "layout"),
                                  (1, 1, 3000, 6000, 16, 0, "layout")],
                         ids=lambda c: "x".join(map(str, c)))
def test_bwd_table_order_matches_two_launches(case):
    """The one-launch backward table and dK/dV launch order against
    scfa_bwd_table followed by scfa_work_order (span = nQt): the same table
    bit for bit and a valid longest-first order, on forward tables of
    statistics shaped like the aligned hash layout and the QK mode (starts
    and ends in order: the searched path) and of random statistics (the
    tile-by-tile path); (65, 8, ...) and (1, 1, 4000, 8000, ...) are too
    large for one workgroup (the two-launch fallback inside the call, with
    scfa_work_order's groups); the other cases with B*H not a multiple of 8
    take the runs layout."""
    need_gpu()
    B, H, nQt, nKt, nb, flags, kind = case
    announce(f"bwd table + order {case}")
    rng = np.random.default_rng(sum(case[:6]) + 11)
    if kind == "layout":
        qs, ks = _layout_stats(rng, B * H, nQt, nKt, nb)
        mode = scfa.SCFA_HASH
    elif kind == "qk":
        qs, ks = _qk_stats(rng, B * H, nQt, nKt)
        mode = scfa.SCFA_QK
    else:
        qs = rng.integers(-5, 4000, (B * H, nQt, 4)).astype(np.int32)
        ks = rng.integers(-5, 4000, (B * H, nKt, 4)).astype(np.int32)
        qs[..., 2:] = np.sort(rng.integers(0, nb, (B * H, nQt, 2)), axis=-1)
        ks[..., 2:] = np.sort(rng.integers(0, nb, (B * H, nKt, 2)), axis=-1)
        mode = scfa.SCFA_HASH
    dev = torch.device("cuda:0")
    qst = torch.from_numpy(qs).reshape(B, H, nQt, 4).to(dev)
    kst = torch.from_numpy(ks).reshape(B, H, nKt, 4).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    fwd, tiles = torch.empty((B, H, nQt, 2), **i32), torch.zeros((B, H), **i32)
    scfa.scfa_fwd_table(mode | flags, qst, kst, fwd, tiles)
    ref_bwd, ref_order = torch.empty((B, H, nKt, 2), **i32), torch.empty((B * H * nKt,), **i32)
    scfa.scfa_bwd_table(qst, kst, fwd, ref_bwd, flags=flags)
    scfa.scfa_work_order(ref_bwd, nQt, ref_order)
    bwd, order = torch.empty((B, H, nKt, 2), **i32), torch.empty((B * H * nKt,), **i32)
    scfa.scfa_bwd_table_order(qst, kst, fwd, bwd, order, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(bwd, ref_bwd)
    if kind != "random":
        assert int((bwd[..., 1] > bwd[..., 0]).sum()) > 0  # the tables hold work
    fallback = (B, H) == (65, 8) or nQt >= 4000  # too large for one workgroup: scfa_work_order's groups
    check_order(order.cpu().numpy(), bwd.cpu().numpy(), "groups" if fallback or (B * H) % 8 == 0 else "runs")


def test_plan_orders_training_workload_runs():
    """The hash training workload (B*H = 12, not a multiple of 8): the Plan's
    forward order (forward and dQ) and its dK/dV order are longest-first
    orders in 8 runs of consecutive items, one run per XCD."""
    need_gpu()
    w = WORKLOADS["train_hash_bf16_t16384_nb16"]
    announce(f"plan orders {w.name}")
    x = {k: v.to("cuda:0") for k, v in make_inputs(w).items()}
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb)
    plan.run(x)
    plan.backward(x["dO"])
    torch.cuda.synchronize()
    check_order(plan.tab.fwd_order.cpu().numpy(), plan.tab.fwd.cpu().numpy(), "runs")
    check_order(plan.tab.bwd_order.cpu().numpy(), plan.tab.bwd.cpu().numpy(), "runs")
