"""Pins of the oracle's attention forward/backward (CPU only).

Each test checks the oracle against something other than itself: pure-Python
brute force, torch's scaled_dot_product_attention, closed forms, invariants or
central finite differences. Negative controls plant a mistake in a copy of the
oracle and require the pins to catch it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import scfa_oracle as so
from io_aware_attention_head_amd.inputs import make_inputs, small


def _np64(t):
    return t.to(torch.float64).numpy()


def _omode(mode):
    """Oracle mode of a test mode ("hash_keep": hash with keep masks)."""
    return "hash" if mode == "hash_keep" else mode


def _keeps(mode, kq, kk):
    """Keep masks the oracle gets: QK and hash_keep only."""
    return (kq, kk) if mode in ("qk", "hash_keep") else (None, None)


def _case(mode, T, H=2, D=16, seed=0, keep_p=0.6, nb=4, B=1, Tk=0):
    w = small(_omode(mode), B, H, T, D, dtype="bf16", keep_p=keep_p, nb=nb, seed=seed, Tk=Tk)
    x = make_inputs(w)
    q, k, v = _np64(x["q"]), _np64(x["k"]), _np64(x["v"])
    kq, kk = x["keep_q"].numpy(), x["keep_k"].numpy()
    bq = bk = None
    if _omode(mode) == "hash":
        bq = oracle.hash_bucket(q, x["R"].double().numpy(), nb)
        bk = oracle.hash_bucket(k, x["R"].double().numpy(), nb)
    return w, x, q, k, v, kq, kk, bq, bk


def _brute_fwd(mode, q, k, v, kq, kk, bq, bk, strict=False, noncausal=False):
    """Pairwise enumeration with Python scalars and math.exp (strict: keys
    j < i only; noncausal: every key j)."""
    B, T, H, D = q.shape
    Tk = k.shape[1]
    tau = 1.0 / math.sqrt(D)
    O = np.zeros_like(q)
    L = np.full((B, H, T), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                vis = []
                for j in range(Tk if noncausal else min(Tk, i if strict else i + 1)):
                    if mode in ("qk", "hash_keep") and not (kq[b, i, h] and kk[b, j, h]):
                        continue
                    if mode in ("hash", "hash_keep") and bq[b, h, i] != bk[b, h, j]:
                        continue
                    vis.append(j)
                if not vis:
                    continue
                s = [tau * sum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D)) for j in vis]
                m = max(s)
                lse = m + math.log(sum(math.exp(x - m) for x in s))
                L[b, h, i] = lse
                for jj, j in enumerate(vis):
                    w = math.exp(s[jj] - lse)
                    O[b, i, h] += w * v[b, j, h]
    return O, L


@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
@pytest.mark.parametrize("T,seed", [(1, 0), (7, 1), (33, 2), (64, 3)])
def test_fwd_matches_pairwise_brute_force(mode, T, seed):
    _, _, q, k, v, kq, kk, bq, bk = _case(mode, T, seed=seed)
    O, L = oracle.attention_fwd(_omode(mode), q, k, v, *_keeps(mode, kq, kk), bq, bk)
    Ob, Lb = _brute_fwd(mode, q, k, v, kq, kk, bq, bk)
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], atol=1e-12, rtol=0)


def test_fwd_brute_force_full_head_dim():
    _, _, q, k, v, kq, kk, bq, bk = _case("hash", 24, H=1, D=64, seed=9, nb=2)
    O, L = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    Ob, Lb = _brute_fwd("hash", q, k, v, kq, kk, bq, bk)
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)


def _sdpa_causal(q, k, v):
    # (B,T,H,D) -> (B,H,T,D); float64 on CPU.
    qt, kt, vt = (torch.from_numpy(a).permute(0, 2, 1, 3).contiguous() for a in (q, k, v))
    return qt, kt, vt


@pytest.mark.parametrize("mode", ["dense", "qk"])
def test_dense_and_all_keep_equal_causal_sdpa(mode):
    _, _, q, k, v, kq, kk, _, _ = _case(mode, 96, H=3, D=64, seed=4, keep_p=1.0)
    assert kq.all() and kk.all()
    O, _ = oracle.attention_fwd(mode, q, k, v, kq, kk)
    qt, kt, vt = _sdpa_causal(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(O, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)


def test_bwd_dense_equals_sdpa_autograd():
    _, x, q, k, v, kq, kk, _, _ = _case("dense", 80, H=2, D=64, seed=5)
    dO = _np64(x["dO"])
    dQ, dK, dV = oracle.attention_bwd("dense", q, k, v, dO)
    qt, kt, vt = (t.requires_grad_(True) for t in _sdpa_causal(q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    g = torch.autograd.grad((out * torch.from_numpy(dO).permute(0, 2, 1, 3)).sum(), (qt, kt, vt))
    for mine, ref in zip((dQ, dK, dV), g):
        np.testing.assert_allclose(mine, ref.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)


def test_single_bucket_equals_causal():
    # R = 0 makes every projection +-0, so the first-index tie-break puts every
    # token in bucket 0 and hash-sparse attention is plain causal attention.
    _, x, q, k, v, *_ = _case("hash", 50, H=2, D=64, seed=6)
    R0 = np.zeros((2, 64, 8))
    bq = oracle.hash_bucket(q, R0, 16)
    bk = oracle.hash_bucket(k, R0, 16)
    assert (bq == 0).all() and (bk == 0).all()
    O, L = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    Od, Ld = oracle.attention_fwd("dense", q, k, v)
    np.testing.assert_allclose(O, Od, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L, Ld, atol=1e-13, rtol=0)


def test_bucket_relabelling_invariance():
    _, _, q, k, v, kq, kk, bq, bk = _case("hash", 64, H=2, D=16, seed=7, nb=8)
    sigma = np.random.default_rng(0).permutation(8)
    O, L = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    O2, L2 = oracle.attention_fwd("hash", q, k, v, bkt_q=sigma[bq], bkt_k=sigma[bk])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)


def test_sorted_domain_and_within_bucket_permutation_invariance():
    """Attention over rows sorted by (bucket, position), each row carrying its
    position and bucket, scattered back to original order, equals the
    original-order result; so does any within-bucket or global reordering."""
    _, _, q, k, v, _, _, bq, bk = _case("hash", 64, H=2, D=16, seed=8, nb=4)
    O, L = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    qp, _, _ = oracle.hash_sort(bq, 4)
    kp, _, _ = oracle.hash_sort(bk, 4)
    rng = np.random.default_rng(1)
    for h in range(2):
        orders = [(qp[0, h], kp[0, h])]
        # within-bucket shuffles of the sorted order
        qs, ks = qp[0, h].copy(), kp[0, h].copy()
        for arr, bb in ((qs, bq[0, h]), (ks, bk[0, h])):
            for val in np.unique(bb):
                sel = np.flatnonzero(bb[arr] == val)
                arr[sel] = arr[sel][rng.permutation(len(sel))]
        orders.append((qs, ks))
        orders.append((rng.permutation(64), rng.permutation(64)))
        for qo, ko in orders:
            Or, Lr = oracle.attention_rows(q[0, qo, h], k[0, ko, h], v[0, ko, h], qo, ko, bq[0, h, qo], bk[0, h, ko])
            back = np.zeros_like(Or)
            back[qo] = Or
            lb = np.zeros_like(Lr)
            lb[qo] = Lr
            np.testing.assert_allclose(back, O[0, :, h], atol=1e-13, rtol=0)
            np.testing.assert_array_equal(np.isinf(lb), np.isinf(L[0, h]))


def test_compacted_domain_equals_original_order():
    _, x, q, k, v, kq, kk, _, _ = _case("qk", 64, H=2, D=16, seed=10, keep_p=0.5)
    O, L = oracle.attention_fwd("qk", q, k, v, kq, kk)
    Tc = 64
    qc, qi = oracle.qk_compact(q, kq, Tc, oracle.Q_PAD)
    kc, ki = oracle.qk_compact(k, kk, Tc, oracle.K_PAD)
    vc, _ = oracle.qk_compact(v, kk, Tc, oracle.K_PAD)
    for h in range(2):
        Or, Lr = oracle.attention_rows(qc[0, h], kc[0, h], vc[0, h], qi[0, h], ki[0, h])
        real = qi[0, h] >= 0
        np.testing.assert_allclose(Or[real], O[0, qi[0, h][real], h], atol=1e-13, rtol=0)
        assert np.isinf(Lr[~real]).all()
        dropped = kq[0, :, h] == 0
        assert (O[0, dropped, h] == 0).all() and np.isinf(L[0, h, dropped]).all()


def test_closed_forms():
    _, x, q, k, v, kq, kk, _, _ = _case("qk", 40, H=2, D=16, seed=11, keep_p=0.6)
    B, T, H, D = q.shape
    # Q = 0: uniform weights -> mean of visible values, LSE = ln n.
    O, L = oracle.attention_fwd("qk", np.zeros_like(q), k, v, kq, kk)
    for h in range(H):
        for i in range(T):
            vis = [j for j in range(i + 1) if kq[0, i, h] and kk[0, j, h]]
            if vis:
                np.testing.assert_allclose(O[0, i, h], v[0, vis, h].mean(axis=0), atol=1e-13)
                assert abs(L[0, h, i] - math.log(len(vis))) < 1e-13
            else:
                assert (O[0, i, h] == 0).all() and L[0, h, i] == -math.inf
    # V constant -> O = c on rows with a visible key.
    c = np.broadcast_to(np.arange(D, dtype=np.float64) - 3.5, v.shape)
    O, L = oracle.attention_fwd("qk", q, k, c, kq, kk)
    fin = np.isfinite(L).transpose(0, 2, 1)
    np.testing.assert_allclose(O[fin], c[fin], atol=1e-13)
    # Key shift by a constant vector: O unchanged, LSE shifts by tau q.c.
    shift = np.linspace(-1, 1, D)
    O1, L1 = oracle.attention_fwd("qk", q, k, v, kq, kk)
    O2, L2 = oracle.attention_fwd("qk", q, k + shift, v, kq, kk)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    fin = np.isfinite(L1)
    expect = L1 + (q @ shift / math.sqrt(D)).transpose(0, 2, 1)
    np.testing.assert_allclose(L2[fin], expect[fin], atol=1e-12)


def test_single_visible_key_closed_form():
    # Only key j = 0 kept: every kept query sees exactly that key.
    _, _, q, k, v, kq, _, _, _ = _case("qk", 20, H=1, D=16, seed=12)
    kk = np.zeros_like(kq)
    kk[0, 0, 0] = 1
    O, L = oracle.attention_fwd("qk", q, k, v, kq, kk)
    for i in range(20):
        if kq[0, i, 0]:
            np.testing.assert_allclose(O[0, i, 0], v[0, 0, 0], atol=1e-14)
            assert abs(L[0, 0, i] - q[0, i, 0] @ k[0, 0, 0] / 4.0) < 1e-13


def test_hand_worked_qk_example():
    """T = 4, Q = 0: hand-derived from the uniform-softmax closed form.
    keep_q = [1,1,0,1], keep_k = [0,1,1,1]; query 0 sees no kept key at or
    before it, query 2 is dropped, query 1 sees key 1, query 3 sees keys 1..3."""
    v = np.array([[1, 2], [3, -1], [5, 7], [-2, 4]], dtype=np.float64).reshape(1, 4, 1, 2)
    q = np.zeros_like(v)
    k = np.ones_like(v)
    kq = np.array([1, 1, 0, 1], dtype=np.uint8).reshape(1, 4, 1)
    kk = np.array([0, 1, 1, 1], dtype=np.uint8).reshape(1, 4, 1)
    O, L = oracle.attention_fwd("qk", q, k, v, kq, kk)
    np.testing.assert_allclose(O[0, :, 0], [[0, 0], [3, -1], [0, 0], [2, 10 / 3]], atol=1e-15)
    assert L[0, 0, 0] == -math.inf and L[0, 0, 2] == -math.inf
    assert L[0, 0, 1] == 0.0 and abs(L[0, 0, 3] - math.log(3)) < 1e-15


def _loss(mode, q, k, v, dO, kq, kk, bq, bk):
    O, _ = oracle.attention_fwd(_omode(mode), q, k, v, *_keeps(mode, kq, kk), bq, bk)
    return float((O * dO).sum())


@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
def test_bwd_central_finite_differences(mode):
    _, x, q, k, v, kq, kk, bq, bk = _case(mode, 10, H=1, D=4, seed=13, keep_p=0.6, nb=2)
    dO = _np64(x["dO"])
    grads = oracle.attention_bwd(_omode(mode), q, k, v, dO, *_keeps(mode, kq, kk), bq, bk)
    eps = 1e-6
    for which, g in zip(range(3), grads):
        args = [q.copy(), k.copy(), v.copy()]
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            a = [t.copy() for t in args]
            a[which][idx] += eps
            lp = _loss(mode, a[0], a[1], a[2], dO, kq, kk, bq, bk)
            a[which][idx] -= 2 * eps
            lm = _loss(mode, a[0], a[1], a[2], dO, kq, kk, bq, bk)
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(num - g).max() <= 1e-6 * scale, (which, np.abs(num - g).max())


def test_gradient_identities():
    _, x, q, k, v, kq, kk, _, _ = _case("qk", 48, H=2, D=16, seed=14, keep_p=0.6)
    dO = _np64(x["dO"])
    dQ, dK, dV = oracle.attention_bwd("qk", q, k, v, dO, kq, kk)
    _, L = oracle.attention_fwd("qk", q, k, v, kq, kk)
    for h in range(2):
        # rows of dS sum to zero -> sum_j dK_j = 0
        np.testing.assert_allclose(dK[0, :, h].sum(axis=0), 0, atol=1e-12)
        has = np.isfinite(L[0, h])
        np.testing.assert_allclose(dV[0, :, h].sum(axis=0), dO[0, has, h].sum(axis=0), atol=1e-12)
        # zero gradients at dropped / stranded tokens
        assert (dQ[0, ~has, h] == 0).all()
        assert (dK[0, kk[0, :, h] == 0, h] == 0).all() and (dV[0, kk[0, :, h] == 0, h] == 0).all()


# ---- negative controls: plant a mistake in a copy of the oracle ----------

def test_negative_control_strict_mask_is_caught(monkeypatch):
    _, _, q, k, v, kq, kk, bq, bk = _case("qk", 33, seed=15)
    orig = so._vis_rows

    def strict(mode, rows, T, kq_, kk_, bq_, bk_, strict_=False, noncausal_=False):
        vis = orig(mode, rows, T, kq_, kk_, bq_, bk_, strict_, noncausal_)
        return vis & (np.arange(T)[None, :] < rows[:, None])  # '>' planted where '>=' is asked for

    monkeypatch.setattr(so, "_vis_rows", strict)
    O, _ = so.attention_fwd("qk", q, k, v, kq, kk)
    Ob, _ = _brute_fwd("qk", q, k, v, kq, kk, None, None)
    assert np.abs(O - Ob).max() > 1e-3


def test_negative_control_missing_scale_is_caught():
    _, _, q, k, v, kq, kk, bq, bk = _case("dense", 33, seed=16)
    O, _ = oracle.attention_fwd("dense", q, k, v, scale=1.0)
    Ob, _ = _brute_fwd("dense", q, k, v, kq, kk, None, None)
    assert np.abs(O - Ob).max() > 1e-3


def test_negative_control_flipped_keep_bit_changes_row():
    _, _, q, k, v, kq, kk, _, _ = _case("qk", 30, H=1, seed=17, keep_p=0.99)
    kq[:] = 1
    kk[:] = 1
    O, _ = oracle.attention_fwd("qk", q, k, v, kq, kk)
    kk2 = kk.copy()
    kk2[0, 3, 0] = 0
    O2, _ = oracle.attention_fwd("qk", q, k, v, kq, kk2)
    assert np.abs(O2[0, 3:, 0] - O[0, 3:, 0]).max(axis=1).min() > 0
    np.testing.assert_array_equal(O2[0, :3, 0], O[0, :3, 0])


def test_hash_with_keep_all_kept_equals_hash():
    """Hashing combined with within-bucket dropping, nothing dropped: plain
    hash-sparse attention, to the bit."""
    _, _, q, k, v, kq, kk, bq, bk = _case("hash", 60, H=2, D=16, seed=21, nb=8)
    ones = np.ones_like(kq)
    O1, L1 = oracle.attention_fwd("hash", q, k, v, ones, ones, bq, bk)
    O2, L2 = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_hash_with_keep_single_bucket_equals_qk():
    """One bucket (R = 0) with keep masks: QK-drop attention (the QK path is
    pinned on its own against brute force and SDPA)."""
    _, _, q, k, v, kq, kk, _, _ = _case("qk", 70, H=2, D=16, seed=22, keep_p=0.5)
    R0 = np.zeros((2, 16, 4))
    bq, bk = oracle.hash_bucket(q, R0, 8), oracle.hash_bucket(k, R0, 8)
    O1, L1 = oracle.attention_fwd("hash", q, k, v, kq, kk, bq, bk)
    O2, L2 = oracle.attention_fwd("qk", q, k, v, kq, kk)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    g1 = oracle.attention_bwd("hash", q, k, v, q, kq, kk, bq, bk)
    g2 = oracle.attention_bwd("qk", q, k, v, q, kq, kk)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def test_hash_with_keep_dropped_rows_and_gradients_are_zero():
    _, x, q, k, v, kq, kk, bq, bk = _case("hash_keep", 48, H=2, D=16, seed=23, keep_p=0.5, nb=4)
    O, L = oracle.attention_fwd("hash", q, k, v, kq, kk, bq, bk)
    dropped_q = kq.transpose(0, 2, 1) == 0  # (B, H, T)
    assert np.isneginf(L[dropped_q]).all()
    assert (O.transpose(0, 2, 1, 3)[dropped_q] == 0).all()
    dQ, dK, dV = oracle.attention_bwd("hash", q, k, v, _np64(x["dO"]), kq, kk, bq, bk)
    dropped_k = kk == 0  # (B, T, H)
    assert (dK[dropped_k] == 0).all() and (dV[dropped_k] == 0).all()
    assert (dQ[kq == 0] == 0).all()


@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
@pytest.mark.parametrize("T,seed", [(1, 30), (9, 31), (40, 32)])
def test_strict_matches_pairwise_brute_force(mode, T, seed):
    """The explainer's '>' variant of the causal test (a key strictly before
    the query) against pairwise enumeration over j < i."""
    _, _, q, k, v, kq, kk, bq, bk = _case(mode, T, seed=seed)
    O, L = oracle.attention_fwd(_omode(mode), q, k, v, *_keeps(mode, kq, kk), bq, bk, strict=True)
    Ob, Lb = _brute_fwd(mode, q, k, v, kq, kk, bq, bk, strict=True)
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], atol=1e-12, rtol=0)
    assert np.isneginf(L[:, :, 0]).all() and (O[:, 0] == 0).all()  # the first token sees nothing


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_strict_equals_inclusive_on_shifted_sequence(mode):
    """Query i strictly after key j is query i - 1 of the sequence whose
    queries start one token later: strict(q, k, v)[1:] = causal(q[1:], k[:-1],
    v[:-1]) with the keep masks / buckets shifted alike (forward and the
    query gradient; keys and values of the last token get nothing)."""
    _, x, q, k, v, kq, kk, bq, bk = _case(mode, 57, H=2, D=16, seed=33)
    keeps = _keeps(mode, kq, kk)
    O, L = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk, strict=True)
    sk = (None, None) if keeps[0] is None else (kq[:, 1:], kk[:, :-1])
    sb = (None, None) if bq is None else (bq[:, :, 1:], bk[:, :, :-1])
    O2, L2 = oracle.attention_fwd(mode, q[:, 1:], k[:, :-1], v[:, :-1], *sk, *sb)
    np.testing.assert_allclose(O[:, 1:], O2, atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(L[:, :, 1:]), np.isinf(L2))
    fin = np.isfinite(L2)
    np.testing.assert_allclose(L[:, :, 1:][fin], L2[fin], atol=1e-13, rtol=0)
    dO = _np64(x["dO"])
    dQ, dK, dV = oracle.attention_bwd(mode, q, k, v, dO, *keeps, bq, bk, strict=True)
    dQ2, dK2, dV2 = oracle.attention_bwd(mode, q[:, 1:], k[:, :-1], v[:, :-1], dO[:, 1:], *sk, *sb)
    np.testing.assert_allclose(dQ[:, 1:], dQ2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dK[:, :-1], dK2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dV[:, :-1], dV2, atol=1e-12, rtol=0)
    assert (dQ[:, 0] == 0).all() and (dK[:, -1] == 0).all() and (dV[:, -1] == 0).all()


def test_strict_bwd_central_finite_differences():
    _, x, q, k, v, kq, kk, bq, bk = _case("qk", 10, H=1, D=4, seed=34, keep_p=0.7)
    dO = _np64(x["dO"])
    grads = oracle.attention_bwd("qk", q, k, v, dO, kq, kk, strict=True)
    eps = 1e-6
    loss = lambda a: float((oracle.attention_fwd("qk", a[0], a[1], a[2], kq, kk, strict=True)[0] * dO).sum())  # noqa: E731
    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            a = [q.copy(), k.copy(), v.copy()]
            a[which][idx] += eps
            lp = loss(a)
            a[which][idx] -= 2 * eps
            num[idx] = (lp - loss(a)) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(num).max())


@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
@pytest.mark.parametrize("T,seed", [(1, 40), (9, 41), (40, 42)])
def test_noncausal_matches_pairwise_brute_force(mode, T, seed):
    """Bidirectional attention (no position test) against pairwise
    enumeration over every key."""
    _, _, q, k, v, kq, kk, bq, bk = _case(mode, T, seed=seed)
    O, L = oracle.attention_fwd(_omode(mode), q, k, v, *_keeps(mode, kq, kk), bq, bk, noncausal=True)
    Ob, Lb = _brute_fwd(mode, q, k, v, kq, kk, bq, bk, noncausal=True)
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], atol=1e-12, rtol=0)


def test_noncausal_dense_equals_library_attention():
    """Dense bidirectional attention is plain softmax(tau Q K^T) V: torch's
    scaled_dot_product_attention without a mask, in float64 on the CPU."""
    _, x, q, k, v, _, _, _, _ = _case("dense", 70, H=3, D=16, seed=43)
    O, L = oracle.attention_fwd("dense", q, k, v, noncausal=True)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)  # noqa: E731  (B, H, T, D)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=False)
    np.testing.assert_allclose(O, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    s = torch.einsum("bhid,bhjd->bhij", t(q), t(k)) / math.sqrt(16)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_noncausal_is_permutation_equivariant(mode):
    """Without a position test, reordering the tokens (q, k, v, keep bits and
    buckets alike) reorders O, LSE and every gradient the same way; the
    causal result has no such symmetry."""
    _, x, q, k, v, kq, kk, bq, bk = _case(mode, 37, H=2, D=16, seed=44)
    keeps = _keeps(mode, kq, kk)
    dO = _np64(x["dO"])
    perm = np.random.default_rng(45).permutation(37)
    pk = (None, None) if keeps[0] is None else (kq[:, perm], kk[:, perm])
    pb = (None, None) if bq is None else (bq[:, :, perm], bk[:, :, perm])
    O, L = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk, noncausal=True)
    O2, L2 = oracle.attention_fwd(mode, q[:, perm], k[:, perm], v[:, perm], *pk, *pb, noncausal=True)
    np.testing.assert_allclose(O2, O[:, perm], atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(L2), np.isinf(L[:, :, perm]))
    fin = np.isfinite(L2)
    np.testing.assert_allclose(L2[fin], L[:, :, perm][fin], atol=1e-13, rtol=0)
    g = oracle.attention_bwd(mode, q, k, v, dO, *keeps, bq, bk, noncausal=True)
    g2 = oracle.attention_bwd(mode, q[:, perm], k[:, perm], v[:, perm], dO[:, perm], *pk, *pb, noncausal=True)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(b, a[:, perm], atol=1e-12, rtol=0)
    Oc, _ = oracle.attention_fwd(mode, q[:, perm], k[:, perm], v[:, perm], *pk, *pb)
    Oc0, _ = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk)
    assert np.abs(Oc - Oc0[:, perm]).max() > 1e-3


def test_noncausal_bwd_central_finite_differences():
    _, x, q, k, v, kq, kk, bq, bk = _case("hash_keep", 10, H=1, D=4, seed=46, keep_p=0.8, nb=2)
    dO = _np64(x["dO"])
    grads = oracle.attention_bwd("hash", q, k, v, dO, kq, kk, bq, bk, noncausal=True)
    eps = 1e-6
    loss = lambda a: float((oracle.attention_fwd("hash", a[0], a[1], a[2], kq, kk, bq, bk,  # noqa: E731
                                                 noncausal=True)[0] * dO).sum())
    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            a = [q.copy(), k.copy(), v.copy()]
            a[which][idx] += eps
            lp = loss(a)
            a[which][idx] -= 2 * eps
            num[idx] = (lp - loss(a)) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(num).max())


@pytest.mark.parametrize("mode", ["dense", "qk", "hash", "hash_keep"])
@pytest.mark.parametrize("T,Tk,seed", [(9, 23, 50), (23, 9, 51), (1, 5, 52), (5, 1, 53)])
@pytest.mark.parametrize("variant", ["causal", "strict", "noncausal"])
def test_separate_lengths_match_pairwise_brute_force(mode, T, Tk, seed, variant):
    """T_Q != T_KV: queries at 0..T-1, keys at 0..Tk-1, against pairwise
    enumeration."""
    _, _, q, k, v, kq, kk, bq, bk = _case(mode, T, seed=seed, Tk=Tk)
    assert q.shape[1] == T and k.shape[1] == Tk and v.shape[1] == Tk
    flags = {"strict": variant == "strict", "noncausal": variant == "noncausal"}
    O, L = oracle.attention_fwd(_omode(mode), q, k, v, *_keeps(mode, kq, kk), bq, bk, **flags)
    Ob, Lb = _brute_fwd(mode, q, k, v, kq, kk, bq, bk, **flags)
    np.testing.assert_allclose(O, Ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_longer_keys_reduce_to_the_square_case(mode):
    """Tk > Tq, causal: the keys after the last query are never visible, so
    the result equals the square case on the first Tq keys, and those keys
    get no gradient."""
    _, x, q, k, v, kq, kk, bq, bk = _case(mode, 31, H=2, D=16, seed=54, Tk=50)
    keeps = _keeps(mode, kq, kk)
    sk = (None, None) if keeps[0] is None else (kq, kk[:, :31])
    sb = (None, None) if bq is None else (bq, bk[:, :, :31])
    O, L = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk)
    O2, L2 = oracle.attention_fwd(mode, q, k[:, :31], v[:, :31], *sk, *sb)
    np.testing.assert_allclose(O, O2, atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(L), np.isinf(L2))
    np.testing.assert_allclose(L[np.isfinite(L)], L2[np.isfinite(L2)], atol=1e-13, rtol=0)
    dO = _np64(x["dO"])
    dQ, dK, dV = oracle.attention_bwd(mode, q, k, v, dO, *keeps, bq, bk)
    dQ2, dK2, dV2 = oracle.attention_bwd(mode, q, k[:, :31], v[:, :31], dO, *sk, *sb)
    np.testing.assert_allclose(dQ, dQ2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dK[:, :31], dK2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dV[:, :31], dV2, atol=1e-13, rtol=0)
    assert (dK[:, 31:] == 0).all() and (dV[:, 31:] == 0).all()


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_longer_queries_split_into_square_and_bidirectional(mode):
    """Tq > Tk, causal: the first Tk queries give the square case; every
    later query sees every key, as in the non-causal result."""
    _, x, q, k, v, kq, kk, bq, bk = _case(mode, 50, H=2, D=16, seed=55, Tk=31)
    keeps = _keeps(mode, kq, kk)
    O, L = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk)
    sk = (None, None) if keeps[0] is None else (kq[:, :31], kk)
    sb = (None, None) if bq is None else (bq[:, :, :31], bk)
    O2, L2 = oracle.attention_fwd(mode, q[:, :31], k, v, *sk, *sb)
    np.testing.assert_allclose(O[:, :31], O2, atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(L[:, :, :31]), np.isinf(L2))
    np.testing.assert_allclose(L[:, :, :31][np.isfinite(L2)], L2[np.isfinite(L2)], atol=1e-13, rtol=0)
    On, Ln = oracle.attention_fwd(mode, q, k, v, *keeps, bq, bk, noncausal=True)
    np.testing.assert_allclose(O[:, 31:], On[:, 31:], atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(L[:, :, 31:]), np.isinf(Ln[:, :, 31:]))
    fin = np.isfinite(Ln[:, :, 31:])
    np.testing.assert_allclose(L[:, :, 31:][fin], Ln[:, :, 31:][fin], atol=1e-13, rtol=0)


def test_separate_lengths_bwd_central_finite_differences():
    _, x, q, k, v, kq, kk, bq, bk = _case("qk", 7, H=1, D=4, seed=56, keep_p=0.8, Tk=11)
    dO = _np64(x["dO"])
    assert dO.shape == q.shape
    grads = oracle.attention_bwd("qk", q, k, v, dO, kq, kk, strict=True)
    assert grads[1].shape == k.shape and grads[2].shape == v.shape
    eps = 1e-6
    loss = lambda a: float((oracle.attention_fwd("qk", a[0], a[1], a[2], kq, kk, strict=True)[0] * dO).sum())  # noqa: E731
    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            a = [q.copy(), k.copy(), v.copy()]
            a[which][idx] += eps
            lp = loss(a)
            a[which][idx] -= 2 * eps
            num[idx] = (lp - loss(a)) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(num).max())
