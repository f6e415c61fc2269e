"""GPU parity of the non-causal variant (SCFA_NONCAUSAL: no position test,
bidirectional attention over the kept / same-bucket tokens, which the
explainer lists as untested) against the float64 oracle, through the C ABI:
forward outputs, range tables, pair counts and gradients in every mode,
hashing combined with dropping, and the benchmark shape through a captured
Plan."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs, small
from gpu_util import TOL_GRAD, announce, check_fwd, f64, need_gpu, oracle_buckets, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    small("dense", 1, 2, 333, seed=121, grad=True),
    small("qk", 2, 3, 777, keep_p=0.6, seed=122, grad=True),
    small("qk", 1, 2, 513, dtype="f32", keep_p=0.5, seed=123),
    small("hash", 2, 3, 1000, nb=16, seed=124, grad=True),
    small("hash", 1, 2, 300, nb=2, seed=125, grad=True),
]


def _inputs(w, skew=False):
    """Seeded inputs; skew=True also drops most queries of head 0 and most
    keys of head 1 (QK), so that whole query / key tiles of those heads are
    pads."""
    x = make_inputs(w)
    if skew:
        x["keep_q"][:, 90:, 0] = 0
        x["keep_k"][:, 150:, 1] = 0
    return x


def _prepare(w, g, drop=False):
    if w.mode == "hash":
        keeps = dict(keep_q=g["keep_q"], keep_k=g["keep_k"]) if drop else {}
        return scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb, noncausal=True, **keeps)
    if w.mode == "qk":
        return scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"], noncausal=True)
    return scfa.prepare_dense(g["q"], g["k"], g["v"], noncausal=True)


def _oracle_args(w, x, drop=False):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    if w.mode == "hash":
        bq, bk = oracle_buckets(w, x)
        if drop:
            return (q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), bq, bk)
        return (q, k, v, None, None, bq, bk)
    if w.mode == "qk":
        return (q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), None, None)
    return (q, k, v, None, None, None, None)


def _check_forward(w, x, drop=False):
    g = to_dev(x)
    pre = _prepare(w, g, drop)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    torch.cuda.synchronize()
    a = _oracle_args(w, x, drop)
    Or, Lr = oracle.attention_fwd(w.mode, *a, noncausal=True)
    err, lerr = check_fwd(w, O, lse, Or, Lr)
    print(f"{w.name}: max-abs {err:.2e}  lse {lerr:.2e}")
    if w.mode == "dense":  # every query sees every key: no empty row
        assert torch.isfinite(lse).all()
    if not drop:
        # tables: the oracle's rules without the position test
        qi, ki = pre.q_idx.cpu().numpy(), pre.k_idx.cpu().numpy()
        qb = pre.q_bkt.cpu().numpy() if pre.q_bkt is not None else None
        kb = pre.k_bkt.cpu().numpy() if pre.k_bkt is not None else None
        omode = "hash" if w.mode == "hash" else "qk"
        ref = oracle.range_tables(omode, qi[:, :, :pre.Tq], ki[:, :, :pre.Tk],
                                  qb[:, :, :pre.Tq] if qb is not None else None,
                                  kb[:, :, :pre.Tk] if kb is not None else None, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N,
                                  noncausal=True)
        assert np.array_equal(tab.fwd.cpu().numpy()[:, :, :ref["fwd"].shape[2]], ref["fwd"])
        assert np.array_equal(tab.bwd.cpu().numpy()[:, :, :ref["bwd"].shape[2]], ref["bwd"])
        assert np.array_equal(tab.tiles.cpu().numpy(), ref["tiles"])
    pairs = scfa.count_visible(pre).cpu().numpy()
    exp = oracle.visible_pairs(w.mode, w.T, w.B, w.H, a[3], a[4], a[5], a[6], noncausal=True)
    assert np.array_equal(pairs, exp)
    return g, pre, tab, O, lse, a


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_noncausal_forward_tables_and_pairs(w):
    need_gpu()
    announce(f"noncausal fwd {w.name}")
    _check_forward(w, _inputs(w))


def test_noncausal_qk_pad_tiles():
    """Heads whose kept queries / keys fill only a few tiles: the all-pad
    query tiles must process nothing and the all-pad key tiles must be
    skipped (the position test alone no longer rules them out)."""
    need_gpu()
    w = small("qk", 2, 3, 1200, keep_p=0.8, seed=126, grad=True)
    announce("noncausal qk pad tiles")
    x = _inputs(w, skew=True)
    g, pre, tab, O, lse, a = _check_forward(w, x)
    assert pre.Tq >= 3 * scfa.SCFA_TILE_M  # head 0 holds at most 90 kept queries: whole pad tiles
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    ref = oracle.attention_bwd("qk", a[0], a[1], a[2], f64(x["dO"]), *a[3:], noncausal=True)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        rel = float(np.linalg.norm(f64(got) - r) / np.linalg.norm(r))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"


@pytest.mark.parametrize("w", [c for c in CASES if c.grad], ids=lambda w: w.name)
def test_noncausal_backward(w):
    need_gpu()
    announce(f"noncausal bwd {w.name}")
    x = _inputs(w)
    g = to_dev(x)
    pre = _prepare(w, g)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    a = _oracle_args(w, x)
    ref = oracle.attention_bwd(w.mode, a[0], a[1], a[2], f64(x["dO"]), *a[3:], noncausal=True)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        rel = float(np.linalg.norm(f64(got) - r) / np.linalg.norm(r))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"


def test_noncausal_hash_with_drop():
    """Hashing combined with dropping, without the position test: forward,
    pair count and gradients."""
    need_gpu()
    w = small("hash", 2, 3, 900, nb=8, keep_p=0.6, seed=127, grad=True)
    announce("noncausal hash+drop")
    x = _inputs(w)
    g, pre, tab, O, lse, a = _check_forward(w, x, drop=True)
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    ref = oracle.attention_bwd("hash", a[0], a[1], a[2], f64(x["dO"]), *a[3:], noncausal=True)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        rel = float(np.linalg.norm(f64(got) - r) / np.linalg.norm(r))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"


def test_noncausal_rejects_strict_together():
    need_gpu()
    w = CASES[0]
    g = to_dev(make_inputs(w))
    pre = scfa.prepare_dense(g["q"], g["k"], g["v"], noncausal=True)
    tab = scfa.build_tables(pre)
    with pytest.raises(scfa.ScfaError):
        scfa.scfa_qk_sparse_fwd(g["q"], g["k"], g["v"], pre.q_idx, pre.k_idx, tab.qstats, tab.kstats, tab.fwd,
                                w.T, torch.empty_like(g["q"], dtype=torch.float32),
                                torch.empty(w.B, w.H, w.T, device=g["q"].device), 0.125,
                                flags=scfa.SCFA_STRICT | scfa.SCFA_NONCAUSAL)


def test_noncausal_plan_full_size_graph():
    """The benchmark shape (B=2, H=12, T=16384, nb=16) without the position
    test through a graph-captured Plan: sampled rows of every head against
    the oracle, the pair count and bit-equal replays."""
    need_gpu()
    w = WORKLOADS["hash_bf16_t16384_nb16"]
    announce("noncausal plan full size")
    x = make_inputs(w)
    g = to_dev(x)
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb, noncausal=True)
    plan.run(g)
    torch.cuda.synchronize()
    O_ref, l_ref = plan.O.clone(), plan.lse.clone()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(w.T, 160, replace=False), [0, 1, w.T - 1]]))
    bq, bk = oracle_buckets(w, x)
    Or, Lr = oracle.attention_fwd("hash", f64(x["q"]), f64(x["k"]), f64(x["v"]), bkt_q=bq, bkt_k=bk, rows=rows,
                                  noncausal=True)
    check_fwd(w, plan.O, plan.lse, Or, Lr, rows=rows)
    ref = oracle.visible_pairs("hash", w.T, w.B, w.H, bkt_q=bq, bkt_k=bk, noncausal=True)
    assert np.array_equal(plan.count_visible().cpu().numpy(), ref)
    graph = plan.capture(g)
    for _ in range(2):
        plan.O.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.O, O_ref) and torch.equal(plan.lse, l_ref)
