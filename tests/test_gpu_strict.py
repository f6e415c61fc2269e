"""GPU parity of the strict causal variant (SCFA_STRICT: a key is visible only
strictly before its query, the explainer's '>' form of the causal test)
against the float64 oracle, through the C ABI: forward outputs, range tables,
pair counts and gradients in every mode."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs, small
from gpu_util import TOL_GRAD, announce, check_fwd, f64, need_gpu, oracle_buckets, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    small("dense", 1, 2, 333, seed=111, grad=True),
    small("qk", 2, 3, 777, keep_p=0.6, seed=112, grad=True),
    small("qk", 1, 2, 513, dtype="f32", keep_p=0.5, seed=113),
    small("hash", 2, 3, 1000, nb=16, seed=114, grad=True),
    small("hash", 1, 2, 300, nb=2, seed=115, grad=True),
]


def _prepare(w, g):
    if w.mode == "hash":
        return scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb, strict=True)
    if w.mode == "qk":
        return scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"], strict=True)
    return scfa.prepare_dense(g["q"], g["k"], g["v"], strict=True)


def _oracle_args(w, x):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    if w.mode == "hash":
        bq, bk = oracle_buckets(w, x)
        return (q, k, v, None, None, bq, bk)
    if w.mode == "qk":
        return (q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), None, None)
    return (q, k, v, None, None, None, None)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_strict_forward_tables_and_pairs(w):
    need_gpu()
    announce(f"strict fwd {w.name}")
    x = make_inputs(w)
    g = to_dev(x)
    pre = _prepare(w, g)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    torch.cuda.synchronize()
    a = _oracle_args(w, x)
    Or, Lr = oracle.attention_fwd(w.mode, *a, strict=True)
    err, lerr = check_fwd(w, O, lse, Or, Lr)
    print(f"{w.name}: max-abs {err:.2e}  lse {lerr:.2e}")
    # the first token sees nothing
    assert torch.isneginf(lse[:, :, 0]).all() and (O[:, 0] == 0).all()
    # tables: the oracle's rules with the strict causal extremum test
    qi, ki = pre.q_idx.cpu().numpy(), pre.k_idx.cpu().numpy()
    qb = pre.q_bkt.cpu().numpy() if pre.q_bkt is not None else None
    kb = pre.k_bkt.cpu().numpy() if pre.k_bkt is not None else None
    omode = "hash" if w.mode == "hash" else "qk"
    ref = oracle.range_tables(omode, qi[:, :, :pre.Tq], ki[:, :, :pre.Tk], qb[:, :, :pre.Tq] if qb is not None else None,
                              kb[:, :, :pre.Tk] if kb is not None else None, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N,
                              strict=True)
    nQt, nKt = tab.fwd.shape[2], tab.bwd.shape[2]
    assert np.array_equal(tab.fwd.cpu().numpy()[:, :, :ref["fwd"].shape[2]], ref["fwd"])
    assert np.array_equal(tab.bwd.cpu().numpy()[:, :, :ref["bwd"].shape[2]], ref["bwd"])
    assert np.array_equal(tab.tiles.cpu().numpy(), ref["tiles"])
    pairs = scfa.count_visible(pre).cpu().numpy()
    exp = oracle.visible_pairs(w.mode, w.T, w.B, w.H, a[3], a[4], a[5], a[6], strict=True)
    assert np.array_equal(pairs, exp)


@pytest.mark.parametrize("w", [c for c in CASES if c.grad], ids=lambda w: w.name)
def test_strict_backward(w):
    need_gpu()
    announce(f"strict bwd {w.name}")
    x = make_inputs(w)
    g = to_dev(x)
    pre = _prepare(w, g)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    a = _oracle_args(w, x)
    ref = oracle.attention_bwd(w.mode, a[0], a[1], a[2], f64(x["dO"]), *a[3:], strict=True)
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        gn = f64(got)
        rel = float(np.linalg.norm(gn - r) / np.linalg.norm(r))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"
    # the first query and the last key take no part
    assert (f64(grads[0])[:, 0] == 0).all()
    assert (f64(grads[1])[:, -1] == 0).all() and (f64(grads[2])[:, -1] == 0).all()


def test_strict_plan_full_size_graph():
    """The benchmark workload, strict, through a graph-captured Plan: sampled
    rows of every head against the oracle, the pair count and bit-equal
    replays."""
    need_gpu()
    w = WORKLOADS["hash_bf16_t16384_nb16"]
    announce("strict plan full size")
    x = make_inputs(w)
    g = to_dev(x)
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb, strict=True)
    plan.run(g)
    torch.cuda.synchronize()
    O_ref, l_ref = plan.O.clone(), plan.lse.clone()
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([rng.choice(w.T, 160, replace=False), [0, 1, w.T - 1]]))
    bq, bk = oracle_buckets(w, x)
    Or, Lr = oracle.attention_fwd("hash", f64(x["q"]), f64(x["k"]), f64(x["v"]), bkt_q=bq, bkt_k=bk, rows=rows,
                                  strict=True)
    check_fwd(w, plan.O, plan.lse, Or, Lr, rows=rows)
    ref = oracle.visible_pairs("hash", w.T, w.B, w.H, bkt_q=bq, bkt_k=bk, strict=True)
    assert np.array_equal(plan.count_visible().cpu().numpy(), ref)
    graph = plan.capture(g)
    for _ in range(2):
        plan.O.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.O, O_ref) and torch.equal(plan.lse, l_ref)
