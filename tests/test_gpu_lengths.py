"""GPU parity of separate query and key lengths (T_Q != T_KV: queries at
positions 0..T_Q-1, keys and values at 0..T_KV-1, the explainer's decision
tensors of two lengths) against the float64 oracle, through the C ABI:
forward outputs, range tables, pair counts and gradients in every mode, with
the causal, strict and non-causal position tests, and Plans (one-side hash
launches, graph replay) at larger shapes."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import make_inputs, small
from gpu_util import TOL_GRAD, announce, check_fwd, f64, need_gpu, oracle_buckets, to_dev

pytestmark = pytest.mark.gpu

# (workload, variant): T is the query length, Tk the key/value length
CASES = [
    (small("dense", 1, 2, 333, seed=131, grad=True, Tk=517), "causal"),
    (small("dense", 1, 2, 517, seed=132, grad=True, Tk=333), "causal"),
    (small("qk", 2, 3, 777, keep_p=0.6, seed=133, grad=True, Tk=401), "causal"),
    (small("qk", 2, 3, 401, keep_p=0.6, seed=134, grad=True, Tk=777), "strict"),
    (small("qk", 1, 2, 300, dtype="f32", keep_p=0.5, seed=135, Tk=700), "causal"),
    (small("hash", 2, 3, 1000, nb=16, seed=136, grad=True, Tk=1500), "causal"),
    (small("hash", 2, 3, 1500, nb=8, seed=137, grad=True, Tk=1000), "noncausal"),
    (small("hash", 1, 2, 200, nb=4, dtype="f32", seed=138, Tk=900), "strict"),
    # extremes: one query against many keys, many queries against one key
    (small("dense", 1, 2, 1, seed=140, Tk=257), "causal"),
    (small("qk", 1, 2, 257, keep_p=0.7, seed=141, Tk=1), "causal"),
    (small("hash", 1, 2, 3, nb=4, seed=142, Tk=700), "noncausal"),
    (small("hash", 1, 2, 700, nb=4, seed=143, Tk=1), "causal"),
]


def _flags(variant):
    return {"strict": variant == "strict", "noncausal": variant == "noncausal"}


def _prepare(w, g, variant):
    f = _flags(variant)
    if w.mode == "hash":
        return scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb, **f)
    if w.mode == "qk":
        return scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"], **f)
    return scfa.prepare_dense(g["q"], g["k"], g["v"], **f)


def _oracle_args(w, x):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    if w.mode == "hash":
        bq, bk = oracle_buckets(w, x)
        return (q, k, v, None, None, bq, bk)
    if w.mode == "qk":
        return (q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), None, None)
    return (q, k, v, None, None, None, None)


def _ids(c):
    return f"{c[0].name}-{c[1]}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_lengths_forward_tables_and_pairs(case):
    w, variant = case
    need_gpu()
    announce(f"lengths fwd {w.name} {variant}")
    x = make_inputs(w)
    assert x["k"].shape[1] == w.T_kv != w.T
    g = to_dev(x)
    pre = _prepare(w, g, variant)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    torch.cuda.synchronize()
    assert O.shape == (w.B, w.T, w.H, w.D) and lse.shape == (w.B, w.H, w.T)
    a = _oracle_args(w, x)
    Or, Lr = oracle.attention_fwd(w.mode, *a, **_flags(variant))
    err, lerr = check_fwd(w, O, lse, Or, Lr)
    print(f"{w.name} {variant}: max-abs {err:.2e}  lse {lerr:.2e}")
    qi, ki = pre.q_idx.cpu().numpy(), pre.k_idx.cpu().numpy()
    qb = pre.q_bkt.cpu().numpy()[:, :, :pre.Tq] if pre.q_bkt is not None else None
    kb = pre.k_bkt.cpu().numpy()[:, :, :pre.Tk] if pre.k_bkt is not None else None
    omode = "hash" if w.mode == "hash" else "qk"
    ref = oracle.range_tables(omode, qi[:, :, :pre.Tq], ki[:, :, :pre.Tk], qb, kb, scfa.SCFA_TILE_M, scfa.SCFA_TILE_N,
                              **_flags(variant))
    assert np.array_equal(tab.fwd.cpu().numpy()[:, :, :ref["fwd"].shape[2]], ref["fwd"])
    assert np.array_equal(tab.bwd.cpu().numpy()[:, :, :ref["bwd"].shape[2]], ref["bwd"])
    assert np.array_equal(tab.tiles.cpu().numpy(), ref["tiles"])
    pairs = scfa.count_visible(pre).cpu().numpy()
    exp = oracle.visible_pairs(w.mode, w.T, w.B, w.H, a[3], a[4], a[5], a[6], Tk=w.T_kv, **_flags(variant))
    assert np.array_equal(pairs, exp)


@pytest.mark.parametrize("case", [c for c in CASES if c[0].grad], ids=_ids)
def test_lengths_backward(case):
    w, variant = case
    need_gpu()
    announce(f"lengths bwd {w.name} {variant}")
    x = make_inputs(w)
    g = to_dev(x)
    pre = _prepare(w, g, variant)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    assert grads[0].shape == (w.B, w.T, w.H, w.D)
    assert grads[1].shape == grads[2].shape == (w.B, w.T_kv, w.H, w.D)
    a = _oracle_args(w, x)
    ref = oracle.attention_bwd(w.mode, a[0], a[1], a[2], f64(x["dO"]), *a[3:], **_flags(variant))
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        rel = float(np.linalg.norm(f64(got) - r) / np.linalg.norm(r))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"
    if w.T_kv > w.T and variant == "causal":  # keys after the last query take no part
        assert (f64(grads[1])[:, w.T:] == 0).all() and (f64(grads[2])[:, w.T:] == 0).all()


@pytest.mark.parametrize("mode,T,Tk", [("hash", 8192, 16384), ("hash", 16384, 4096), ("qk", 4096, 8192)])
def test_lengths_plan_graph(mode, T, Tk):
    """Plans with T_kv != T (hash: the one-side bucket and layout launches and
    the statistics built with the tables) at larger shapes: sampled rows of
    every head against the oracle, the pair count, bit-equal graph replays
    and, for QK, the backward of the first head against the oracle."""
    need_gpu()
    w = small(mode, 2, 4, T, nb=16, keep_p=0.5, seed=139, grad=(mode == "qk"), Tk=Tk)
    announce(f"lengths plan {mode} T={T} Tk={Tk}")
    x = make_inputs(w)
    g = to_dev(x)
    plan = scfa.Plan(mode, w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb, T_kv=Tk)
    plan.run(g)
    torch.cuda.synchronize()
    assert int(plan.dev_err.item()) == 0
    O_ref, l_ref = plan.O.clone(), plan.lse.clone()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(T, 96, replace=False), [0, T - 1, min(T, Tk) - 1]]))
    a = _oracle_args(w, x)
    Or, Lr = oracle.attention_fwd(mode, *a, rows=rows)
    check_fwd(w, plan.O, plan.lse, Or, Lr, rows=rows)
    ref = oracle.visible_pairs(mode, T, w.B, w.H, a[3], a[4], a[5], a[6], Tk=Tk)
    assert np.array_equal(plan.count_visible().cpu().numpy(), ref)
    graph = plan.capture(g)
    for _ in range(2):
        plan.O.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.O, O_ref) and torch.equal(plan.lse, l_ref)
    if mode == "qk":
        plan.run(g)
        grads = plan.backward(g["dO"])
        torch.cuda.synchronize()
        refg = oracle.attention_bwd(mode, a[0], a[1], a[2], f64(x["dO"]), *a[3:], heads=[(0, 0)])
        for name, got, r in zip(("dQ", "dK", "dV"), grads, refg):
            gn, rn = f64(got)[0, :, 0], r[0, :, 0]
            rel = float(np.linalg.norm(gn - rn) / np.linalg.norm(rn))
            assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"
