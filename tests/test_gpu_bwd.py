"""GPU parity of the backward (dQ, dK, dV) against the float64 oracle, through
the C ABI: relative Frobenius error per tensor <= 2e-2, zero rows where the
method defines zero gradients, gradient identities at full size."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs, small
from gpu_util import TOL_GRAD, announce, f64, need_gpu, oracle_buckets, run_pipeline

pytestmark = pytest.mark.gpu


def _oracle_bwd(w, x, heads=None, buckets=None):
    q, k, v, dO = (f64(x[n]) for n in ("q", "k", "v", "dO"))
    if w.mode == "hash":
        bq, bk = buckets if buckets is not None else oracle_buckets(w, x)
        return oracle.attention_bwd("hash", q, k, v, dO, bkt_q=bq, bkt_k=bk, heads=heads)
    if w.mode == "qk":
        return oracle.attention_bwd("qk", q, k, v, dO, x["keep_q"].numpy(), x["keep_k"].numpy(), heads=heads)
    return oracle.attention_bwd("dense", q, k, v, dO, heads=heads)


def _run(w, x):
    g, pre, tab, O, lse = run_pipeline(w, x)
    grads = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    return g, pre, tab, O, lse, grads


def _check(grads, ref, heads=None):
    out = []
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        gn = f64(got)
        assert np.isfinite(gn).all(), f"{name} not finite"
        if heads is not None:
            gs = np.stack([gn[b, :, h] for b, h in heads])
            rs = np.stack([r[b, :, h] for b, h in heads])
        else:
            gs, rs = gn, r
        den = np.linalg.norm(rs)
        rel = float(np.linalg.norm(gs - rs) / den) if den > 0 else float(np.abs(gs).max())
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"
        out.append(rel)
    return out


SMALL = [
    small("hash", 2, 3, 1000, nb=16, seed=71, grad=True),
    small("hash", 1, 2, 300, nb=4, seed=72, grad=True),
    small("qk", 2, 3, 777, keep_p=0.6, seed=73, grad=True),
    small("qk", 1, 4, 2048, keep_p=0.5, seed=74, grad=True),
    small("dense", 1, 2, 700, seed=75, grad=True),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_bwd_small(w):
    need_gpu()
    announce(f"bwd {w.name}")
    x = make_inputs(w)
    _, pre, tab, O, lse, grads = _run(w, x)
    rels = _check(grads, _oracle_bwd(w, x))
    print(f"{w.name}: rel dQ {rels[0]:.2e} dK {rels[1]:.2e} dV {rels[2]:.2e}")
    if w.mode == "qk":
        kq, kk = x["keep_q"].numpy(), x["keep_k"].numpy()
        dQ, dK, dV = (f64(t) for t in grads)
        assert (dQ[kq == 0] == 0).all()
        assert (dK[kk == 0] == 0).all() and (dV[kk == 0] == 0).all()


@pytest.mark.parametrize("case", ["all_keys_dropped", "T1", "one_each"])
def test_bwd_edge_cases(case):
    need_gpu()
    announce(f"bwd edge {case}")
    T = 1 if case == "T1" else 300
    w = small("qk", 1, 2, T, keep_p=0.7, seed=76, grad=True)
    x = make_inputs(w)
    if case == "all_keys_dropped":
        x["keep_k"].zero_()
    elif case == "one_each":
        x["keep_q"].zero_()
        x["keep_k"].zero_()
        x["keep_q"][:, 200] = 1
        x["keep_k"][:, 10] = 1
    _, pre, tab, O, lse, grads = _run(w, x)
    ref = _oracle_bwd(w, x)
    if case == "all_keys_dropped":
        for t in grads:
            assert (t == 0).all()
    else:
        _check(grads, ref)


def test_bwd_hash_single_bucket_equals_dense():
    need_gpu()
    announce("bwd single bucket vs dense")
    w = small("hash", 1, 2, 500, nb=16, seed=77, grad=True)
    x = make_inputs(w)
    x["R"].zero_()
    _, _, _, _, _, gh = _run(w, x)
    wd = small("dense", 1, 2, 500, seed=77, grad=True)
    _, _, _, _, _, gd = _run(wd, x)
    ref = _oracle_bwd(wd, x)
    _check(gh, ref)
    _check(gd, ref)


@pytest.mark.parametrize("case", ["T1", "T2", "last_bucket_only", "skewed", "nb64_short"])
def test_bwd_hash_edge_cases(case):
    """Hash-mode gradients against the oracle where buckets and tiles are
    degenerate: one and two tokens, every token in the last bucket, most
    tokens in two buckets, and nb = 64 buckets over 300 tokens (most buckets
    hold a handful of tokens or none, so tiles are mostly pad rows)."""
    need_gpu()
    announce(f"bwd hash edge {case}")
    T = {"T1": 1, "T2": 2, "nb64_short": 300}.get(case, 900)
    nb = 64 if case == "nb64_short" else 16
    w = small("hash", 1, 3, T, nb=nb, seed=81, grad=True)
    x = make_inputs(w)
    if case == "last_bucket_only":
        x["R"].zero_()
        x["R"][:, :, nb // 2 - 1] = 1.0
        x["q"] = (-x["q"].float().abs() - 0.01).to(torch.bfloat16)
        x["k"] = (-x["k"].float().abs() - 0.01).to(torch.bfloat16)
    elif case == "skewed":
        x["R"][:, :, 0] += 3.0
    _, pre, tab, O, lse, grads = _run(w, x)
    buckets = oracle_buckets(w, x)
    if case == "last_bucket_only":
        assert (buckets[0] == nb - 1).all() and (buckets[1] == nb - 1).all()
    rels = _check(grads, _oracle_bwd(w, x, buckets=buckets))
    print(f"{case}: rel dQ {rels[0]:.2e} dK {rels[1]:.2e} dV {rels[2]:.2e}")


def test_bwd_deterministic_and_fp32_unsupported():
    need_gpu()
    announce("bwd determinism")
    w = small("hash", 1, 4, 2000, nb=16, seed=78, grad=True)
    x = make_inputs(w)
    g, pre, tab, O, lse, g1 = _run(w, x)
    g1 = tuple(t.clone() for t in g1)
    g2 = scfa.backward(pre, tab, O, lse, g["dO"])
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    wf = small("hash", 1, 1, 200, dtype="f32", nb=4, seed=79, grad=True)
    xf = make_inputs(wf)
    gf, pref, tabf, Of, lsef = run_pipeline(wf, xf)
    with pytest.raises(scfa.ScfaError):
        scfa.backward(pref, tabf, Of, lsef, gf["dO"])


@pytest.mark.parametrize("mode", ["hash", "qk"])
def test_plan_backward_matches_call(mode):
    """A plan's backward (backward table, launch order, kernels) equals one
    backward call on the tables it built, bit for bit, and rewrites every
    gradient row when called again; before its first backward the plan's
    tables are refused."""
    need_gpu()
    announce(f"plan backward {mode}")
    w = small(mode, 2, 3, 1500, nb=16, keep_p=0.6, seed=80, grad=True)
    g = {k: v.to("cuda:0") for k, v in make_inputs(w).items()}
    plan = scfa.Plan(mode, w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb)
    plan.run(g)
    with pytest.raises(scfa.ScfaError):
        scfa.backward(plan.prepared(), plan.tab, plan.O, plan.lse, g["dO"])
    first = tuple(t.clone() for t in plan.backward(g["dO"]))
    ref = scfa.backward(plan.prepared(), plan.tab, plan.O, plan.lse, g["dO"])
    torch.cuda.synchronize()
    for a, b in zip(first, ref):
        assert torch.equal(a, b)
    for t in plan._grads:
        t.fill_(float("nan"))
    got = plan.backward(g["dO"])
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["hash", "qk", "dense"])
def test_plan_backward_graph_replay(mode):
    """A plan's backward captured as one HIP graph (as the benchmark times
    it): three replays, each into gradients first filled with NaN and with
    an eager backward in between, equal the eager backward bit for bit."""
    need_gpu()
    announce(f"plan backward graph {mode}")
    w = small("qk" if mode == "dense" else mode, 1, 3, 1300, nb=8, keep_p=0.6, seed=81, grad=True)
    g = {k: v.to("cuda:0") for k, v in make_inputs(w).items()}
    plan = scfa.Plan(mode, w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb)
    plan.run(g)
    plan.backward(g["dO"])
    torch.cuda.synchronize()
    ref = [t.clone() for t in plan._grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.backward(g["dO"])
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.backward(g["dO"])
    for _ in range(3):
        for t in plan._grads:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(plan._grads, ref):
            assert torch.equal(a, b)
        plan.backward(g["dO"])
        torch.cuda.synchronize()
        for a, b in zip(plan._grads, ref):
            assert torch.equal(a, b)


def _check_tiles(grads, ref, pre, heads):
    """Per-tile check of the gradients: dQ over each 128-query tile and dK, dV
    over each 64-key tile of the kernels' layout (rows of q_idx / k_idx), so
    that one wrong tile cannot hide in a whole-tensor norm. Bound per tile:
    ||g - r||_F <= TOL_GRAD * ||r||_F + 1e-3 * (RMS tile norm of the head),
    the absolute floor covering tiles whose reference nearly cancels.
    Returns the largest ratio error / bound."""
    worst = 0.0
    for name, got, r, idx, rows in zip(("dQ", "dK", "dV"), grads, ref, (pre.q_idx, pre.k_idx, pre.k_idx),
                                       (scfa.SCFA_TILE_M, scfa.SCFA_TILE_N, scfa.SCFA_TILE_N)):
        gn = f64(got)
        ix = idx.cpu().numpy()
        T = gn.shape[1]
        for b, h in heads:
            lay = ix[b, h]
            nt = len(lay) // rows
            errs, norms = [], []
            for t in range(nt):
                pos = lay[t * rows:(t + 1) * rows]
                pos = pos[(pos >= 0) & (pos < T)]
                if len(pos) == 0:
                    continue
                errs.append(np.linalg.norm(gn[b, pos, h] - r[b, pos, h]))
                norms.append(np.linalg.norm(r[b, pos, h]))
            errs, norms = np.array(errs), np.array(norms)
            floor = 1e-3 * np.sqrt((norms ** 2).mean())
            ratio = errs / (TOL_GRAD * norms + floor)
            bad = np.flatnonzero(ratio > 1)
            assert len(bad) == 0, (f"{name} head {(b, h)}: {len(bad)} tiles over the bound, worst rel "
                                   f"{(errs[bad] / np.maximum(norms[bad], 1e-300)).max():.3e}")
            worst = max(worst, float(ratio.max()))
    return worst


_FULL = [("train_hash_bf16_t16384_nb16", (0, 1, 2, 3)), ("train_hash_bf16_t16384_nb16", (4, 5, 6, 7)),
         ("train_hash_bf16_t16384_nb16", (8, 9, 10, 11)), ("train_qk_bf16_t8192_keep0.5", tuple(range(12)))]


@pytest.mark.parametrize("name,hs", _FULL, ids=[f"{n}-h{h[0]}-{h[-1]}" for n, h in _FULL])
def test_bwd_full_size(name, hs):
    """Training-step workloads at full size, every head against the oracle
    (split over several tests to bound each one's oracle time): relative
    Frobenius error of each head's dQ, dK, dV, a per-tile bound over the
    kernels' query and key tiles, and gradient identities on every head."""
    need_gpu()
    w = WORKLOADS[name]
    announce(f"full-size bwd {name} heads {hs}")
    x = make_inputs(w)
    g, pre, tab, O, lse, grads = _run(w, x)
    heads = [(0, h) for h in hs]
    buckets = oracle_buckets(w, x) if w.mode == "hash" else None
    ref = _oracle_bwd(w, x, heads=heads, buckets=buckets)
    worst = [0.0, 0.0, 0.0]
    for hd in heads:
        rels = _check(grads, ref, heads=[hd])
        worst = [max(a, b) for a, b in zip(worst, rels)]
    ratio = _check_tiles(grads, ref, pre, heads)
    print(f"{name} heads {hs}: worst per-head rel dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}; "
          f"worst tile error / bound {ratio:.2f}")
    dQ, dK, dV = (f64(t) for t in grads)
    dO = f64(x["dO"])
    L = lse.cpu().numpy()
    for b in range(w.B):
        for h in range(w.H):
            # rows of dS sum to zero -> sum_j dK_j = 0; sum_j dV_j = sum of dO over rows with a visible key
            scale = np.abs(dK[b, :, h]).sum(axis=0).max() + 1e-9
            assert np.abs(dK[b, :, h].sum(axis=0)).max() <= 2e-2 * scale
            has = np.isfinite(L[b, h])
            ref_v = dO[b, has, h].sum(axis=0)
            assert np.abs(dV[b, :, h].sum(axis=0) - ref_v).max() <= 2e-2 * (np.abs(ref_v).max() + 1)
            assert (dQ[b, ~has, h] == 0).all()


def test_bwd_long_ranges():
    """One bucket (R = 0) at T = 33000: every key tile's query range spans
    258 query tiles and every query tile's key range up to 516 key tiles, so
    both backward kernels read the tile statistics from global memory (more
    than their LDS copy holds) and the forward does too (more than 512 key
    tiles); one head against the oracle."""
    need_gpu()
    w = small("hash", 1, 1, 33000, nb=2, seed=76, grad=True)
    announce("bwd long ranges hash nb=2 T=33000")
    x = make_inputs(w)
    x["R"].zero_()  # a single bucket: causal attention over all 33000 tokens
    g, pre, tab, O, lse, grads = _run(w, x)
    assert tab.fwd.shape[2] > 256 and tab.kstats.shape[2] > 512
    heads = [(0, 0)]
    ref = _oracle_bwd(w, x, heads=heads)
    rels = _check(grads, ref, heads=heads)
    print(f"long ranges: rel dQ {rels[0]:.2e} dK {rels[1]:.2e} dV {rels[2]:.2e}")
