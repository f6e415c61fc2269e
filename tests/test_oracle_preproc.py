"""Pins of the oracle's integer steps: compaction, LSH bucket, sort, gather,
visible-pair counts (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_head_amd.inputs import make_inputs, small, WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def test_pages_constants_match_oracle():
    g = json.load(open(GOLDEN))
    kc = g["kernel_constants"]
    assert oracle.Q_PAD == kc["q_pad"] and oracle.K_PAD == kc["k_pad"]
    assert 1.0 / math.sqrt(kc["D"]) == kc["tau"]
    im = g["index_tensor_memory"]
    idx = np.zeros((im["B"], im["H"], im["T"]), dtype=np.int32)
    assert idx.nbytes == im["bytes"] and round(idx.nbytes / 1e6, 1) == im["approx_MB"]
    fi = g["flop_inventory"]
    pairs = fi["N"] * fi["N"]  # dense, non-causal square
    assert oracle.flops_fwd(pairs, fi["d_h"]) == fi["qk_flops"] + fi["av_flops"]
    # The backward by recomputation evaluates five products of the same
    # (N x d)(d x N) or (N x N)(N x d) shape over the same pairs: the scores
    # Q K^T again, dP = dO V^T, dV = P^T dO, dQ = dS K and dK = dS^T Q. Each
    # costs what the inventory gives for Q K^T (d_h = d_v here).
    assert fi["d_h"] == fi["d_v"]
    assert oracle.flops_bwd(pairs, fi["d_h"]) == 5 * fi["qk_flops"]
    # forward + backward per visible pair: 14 * D
    assert oracle.flops_fwd(1, 64) + oracle.flops_bwd(1, 64) == 14 * 64
    w = WORKLOADS["hash_bf16_t16384_nb16"]
    assert w.H == g["lm_shape"]["heads"] and w.D == g["lm_shape"]["head_dim"] and w.nb == g["lm_shape"]["nb"]


@pytest.mark.parametrize("seed,T,p", [(0, 1, 0.5), (1, 37, 0.7), (2, 130, 0.5), (3, 64, 0.0), (4, 64, 1.0)])
def test_compaction_matches_loop(seed, T, p):
    w = small("qk", 2, 3, T, 8, dtype="bf16", keep_p=p, seed=seed)
    x = make_inputs(w)
    keep = x["keep_q"].numpy()
    xb = x["q"].view(torch.int16).numpy()  # bit patterns
    cnt = oracle.qk_count(keep)
    Tc = max(1, int(cnt.max()) + 5)
    for pad in (oracle.Q_PAD, oracle.K_PAD):
        xc, idx = oracle.qk_compact(xb, keep, Tc, pad)
        for b in range(2):
            for h in range(3):
                kept = [t for t in range(T) if keep[b, t, h]]
                assert cnt[b, h] == len(kept)
                assert list(idx[b, h, :len(kept)]) == kept
                assert (idx[b, h, len(kept):] == pad).all()
                for r, t in enumerate(kept):
                    assert (xc[b, h, r] == xb[b, t, h]).all()
                assert (xc[b, h, len(kept):] == 0).all()


def _bucket_scalar(xrow, Rh, nb):
    half = nb // 2
    c = []
    for j in range(half):
        acc = 0.0
        for d in range(len(xrow)):
            acc = acc + float(xrow[d]) * float(Rh[d][j])
        c.append(acc)
    full = c + [-t for t in c]
    best = 0
    for j in range(1, nb):
        if full[j] > full[best]:
            best = j
    return best


def test_hash_bucket_matches_scalar_loop_bitexact():
    w = small("hash", 1, 2, 40, 64, dtype="bf16", nb=16, seed=5)
    x = make_inputs(w)
    q = x["q"].double().numpy()
    R = x["R"].double().numpy()
    bq = oracle.hash_bucket(q, R, 16)
    for h in range(2):
        for t in range(40):
            assert bq[0, h, t] == _bucket_scalar(q[0, t, h], R[h], 16)


def test_hash_bucket_hand_example():
    # D = 4, nb = 4. x = e_0 picks row 0 of R: c = [0.5, -1] -> [c; -c] =
    # [0.5, -1, -0.5, 1] -> bucket 3. x = 2 e_1 with R row 1 = [0.25, 0.125]:
    # c = [0.5, 0.25] -> bucket 0.
    R = np.zeros((1, 4, 2))
    R[0, 0] = [0.5, -1.0]
    R[0, 1] = [0.25, 0.125]
    x = np.zeros((1, 2, 1, 4))
    x[0, 0, 0, 0] = 1.0
    x[0, 1, 0, 1] = 2.0
    assert list(oracle.hash_bucket(x, R, 4)[0, 0]) == [3, 0]


def test_hash_bucket_symmetries():
    w = small("hash", 2, 3, 200, 64, dtype="bf16", nb=16, seed=6)
    x = make_inputs(w)
    q = x["q"].double().numpy()
    R = x["R"].double().numpy()
    b = oracle.hash_bucket(q, R, 16)
    # negation maps bucket v to v + nb/2 (mod nb); power-of-two scaling keeps it
    assert (oracle.hash_bucket(-q, R, 16) == (b + 8) % 16).all()
    assert (oracle.hash_bucket(q * 8.0, R, 16) == b).all()
    assert (oracle.hash_bucket(q, R * 0.25, 16) == b).all()
    # zero rotations: all ties -> first index
    assert (oracle.hash_bucket(q, np.zeros_like(R), 16) == 0).all()
    assert b.min() >= 0 and b.max() < 16


def test_hash_sort_matches_python_sorted():
    rng = np.random.default_rng(3)
    bucket = rng.integers(0, 6, size=(2, 3, 77)).astype(np.int32)
    perm, bs, off = oracle.hash_sort(bucket, 6)
    for b in range(2):
        for h in range(3):
            ref = sorted(range(77), key=lambda t: (bucket[b, h, t], t))
            assert list(perm[b, h]) == ref
            assert list(bs[b, h]) == [bucket[b, h, t] for t in ref]
            hist = [int((bucket[b, h] == v).sum()) for v in range(6)]
            assert list(off[b, h]) == [sum(hist[:v]) for v in range(7)]


def test_hash_sort_hand_example():
    bucket = np.array([3, 0, 3, 0, 1], dtype=np.int32).reshape(1, 1, 5)
    perm, bs, off = oracle.hash_sort(bucket, 4)
    assert list(perm[0, 0]) == [1, 3, 4, 0, 2]
    assert list(bs[0, 0]) == [0, 0, 1, 3, 3]
    assert list(off[0, 0]) == [0, 2, 3, 3, 5]


def test_hash_segments_hand_example():
    """Buckets of sizes 2, 1, 0, 2 (nb = 4) with align 2: bucket 0 at row 0,
    bucket 1 at row 2 (one pad), bucket 2 empty, bucket 3 at row 4."""
    bucket = np.array([3, 0, 3, 0, 1], dtype=np.int32).reshape(1, 1, 5)
    perm, _, off = oracle.hash_sort(bucket, 4)
    idx, bkt, seg = oracle.hash_segments(perm, off, 4, 2, -1, 8)
    assert list(idx[0, 0]) == [1, 3, 4, -1, 0, 2, -1, -1]
    assert list(bkt[0, 0]) == [0, 0, 1, 1, 3, 3, 4, 4]
    assert list(seg[0, 0]) == [0, 2, 4, 4, 6]


@pytest.mark.parametrize("align", [1, 16, 64, 128])
def test_hash_segments_invariants(align):
    """Removing the pad rows gives back the sorted order; every bucket starts
    at a multiple of align and fits the segment_rows bound; buckets never
    decrease along the rows; no tile of align rows holds two buckets."""
    rng = np.random.default_rng(align)
    nb, T = 8, 300
    bucket = rng.integers(0, nb, size=(2, 2, T)).astype(np.int32)
    bucket[1, 1] = 5  # one bucket holds everything
    perm, bs, off = oracle.hash_sort(bucket, nb)
    Tseg = oracle.segment_rows(T, nb, align)
    assert Tseg % 128 == 0 and Tseg >= T + nb * (align - 1)
    idx, bkt, seg = oracle.hash_segments(perm, off, nb, align, 1_000_000_000, Tseg)
    for b in range(2):
        for h in range(2):
            real = idx[b, h] != 1_000_000_000
            assert list(idx[b, h][real]) == list(perm[b, h])
            assert list(bkt[b, h][real]) == list(bs[b, h])
            assert (seg[b, h] % align == 0).all()
            assert (np.diff(bkt[b, h]) >= 0).all()
            tiles = bkt[b, h].reshape(-1, align) if Tseg % align == 0 else None
            if tiles is not None:
                assert (tiles.min(axis=1) == tiles.max(axis=1)).all()
            n = np.diff(off[b, h])
            assert list(np.diff(seg[b, h])) == [-(-int(c) // align) * align for c in n]


def test_gather_rows():
    x = np.arange(2 * 5 * 3 * 4, dtype=np.int16).reshape(2, 5, 3, 4)
    perm = np.array([[[4, 0, -1], [1, 1, 1000000000], [2, 3, 4]]] * 2, dtype=np.int32)
    g = oracle.gather_rows(x, perm)
    assert (g[1, 0, 0] == x[1, 4, 0]).all() and (g[1, 0, 2] == 0).all()
    assert (g[0, 1, 2] == 0).all() and (g[0, 2, 1] == x[0, 3, 2]).all()


@pytest.mark.parametrize("strict,noncausal", [(False, False), (True, False), (False, True)])
@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
def test_visible_pairs_brute_force(mode, strict, noncausal):
    omode = "hash" if mode == "hash_keep" else mode
    w = small(omode, 2, 2, 45, 16, keep_p=0.6, nb=4, seed=7)
    x = make_inputs(w)
    kq, kk = x["keep_q"].numpy(), x["keep_k"].numpy()
    bq = bk = None
    if omode == "hash":
        R = x["R"].double().numpy()
        bq = oracle.hash_bucket(x["q"].double().numpy(), R, 4)
        bk = oracle.hash_bucket(x["k"].double().numpy(), R, 4)
    keeps = (kq, kk) if mode in ("qk", "hash_keep") else (None, None)
    got = oracle.visible_pairs(omode, 45, 2, 2, *keeps, bq, bk, strict=strict, noncausal=noncausal)
    for b in range(2):
        for h in range(2):
            n = 0
            for i in range(45):
                for j in range(45 if noncausal else (i if strict else i + 1)):
                    if mode in ("qk", "hash_keep") and not (kq[b, i, h] and kk[b, j, h]):
                        continue
                    if omode == "hash" and bq[b, h, i] != bk[b, h, j]:
                        continue
                    n += 1
            assert got[b, h] == n
    if mode == "dense":
        assert (got == (45 * 45 if noncausal else 45 * 44 // 2 if strict else 45 * 46 // 2)).all()
    if mode == "qk" and noncausal:  # every kept query sees every kept key
        assert (got == (kq != 0).sum(axis=1) * (kk != 0).sum(axis=1)).all()


@pytest.mark.parametrize("T,Tk", [(45, 70), (70, 45), (1, 9), (9, 1)])
@pytest.mark.parametrize("strict,noncausal", [(False, False), (True, False), (False, True)])
@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
def test_visible_pairs_separate_lengths_brute_force(mode, strict, noncausal, T, Tk):
    omode = "hash" if mode == "hash_keep" else mode
    w = small(omode, 2, 2, T, 16, keep_p=0.6, nb=4, seed=8, Tk=Tk)
    x = make_inputs(w)
    kq, kk = x["keep_q"].numpy(), x["keep_k"].numpy()
    bq = bk = None
    if omode == "hash":
        R = x["R"].double().numpy()
        bq = oracle.hash_bucket(x["q"].double().numpy(), R, 4)
        bk = oracle.hash_bucket(x["k"].double().numpy(), R, 4)
    keeps = (kq, kk) if mode in ("qk", "hash_keep") else (None, None)
    got = oracle.visible_pairs(omode, T, 2, 2, *keeps, bq, bk, strict=strict, noncausal=noncausal, Tk=Tk)
    for b in range(2):
        for h in range(2):
            n = 0
            for i in range(T):
                for j in range(Tk):
                    if not noncausal and (j >= i if strict else j > i):
                        continue
                    if mode in ("qk", "hash_keep") and not (kq[b, i, h] and kk[b, j, h]):
                        continue
                    if omode == "hash" and bq[b, h, i] != bk[b, h, j]:
                        continue
                    n += 1
            assert got[b, h] == n
    if mode == "dense" and not strict and not noncausal:
        assert (got == sum(min(i + 1, Tk) for i in range(T))).all()
