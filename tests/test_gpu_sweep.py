"""GPU parity at the extreme points of the runtime sweeps (bench.py --sweep:
the explainer's "Experimental Results" figures of hash-sparse runtime
against nb and T, and of QK-sparse runtime against the drop rate and T).
Each point runs through the same Plan the sweep times, with the sweep's
seed and shapes reduced to B=1, H=2: sampled rows of both heads against the
oracle (forward), one head's gradients against the oracle (backward)."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import make_inputs, small
from gpu_util import TOL_GRAD, announce, check_fwd, f64, need_gpu, oracle_buckets, oracle_fwd, to_dev

pytestmark = pytest.mark.gpu

# (mode, nb, keep, T): most and fewest buckets and the highest drop rate at
# the longest sweep length, and the shortest length of each sweep
POINTS = [("hash", 64, None, 16384), ("hash", 2, None, 16384), ("qk", 16, 0.3, 16384), ("hash", 64, None, 1024),
          ("qk", 16, 0.7, 1024), ("qk", 16, 0.3, 1024)]


@pytest.mark.parametrize("mode,nb,keep,T", POINTS,
                         ids=[f"{m}-nb{nb}-keep{kp}-T{T}" for m, nb, kp, T in POINTS])
def test_sweep_extreme_point(mode, nb, keep, T):
    need_gpu()
    announce(f"sweep point {mode} nb={nb} keep={keep} T={T}")
    w = small(mode, 1, 2, T, nb=nb, keep_p=keep if keep is not None else 0.7, seed=91, grad=True)
    x = make_inputs(w)
    g = to_dev(x)
    plan = scfa.Plan(mode, 1, 2, T, 64, torch.bfloat16, nb=nb)
    plan.run(g)
    plan.backward(g["dO"])
    torch.cuda.synchronize()
    assert int(plan.dev_err.item()) == 0
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(T, min(T, 128), replace=False), [0, T - 1]]))
    buckets = oracle_buckets(w, x) if mode == "hash" else None
    Or, Lr = oracle_fwd(w, x, rows=rows, buckets=buckets)
    err, lerr = check_fwd(w, plan.O, plan.lse, Or, Lr, rows=rows)
    if mode == "hash":
        ref_pairs = oracle.visible_pairs("hash", T, 1, 2, bkt_q=buckets[0], bkt_k=buckets[1])
    else:
        ref_pairs = oracle.visible_pairs("qk", T, 1, 2, x["keep_q"].numpy(), x["keep_k"].numpy())
    assert np.array_equal(plan.count_visible().cpu().numpy(), ref_pairs)
    q, k, v, dO = (f64(x[n]) for n in ("q", "k", "v", "dO"))
    heads = [(0, 1)]
    if mode == "hash":
        ref = oracle.attention_bwd("hash", q, k, v, dO, bkt_q=buckets[0], bkt_k=buckets[1], heads=heads)
    else:
        ref = oracle.attention_bwd("qk", q, k, v, dO, x["keep_q"].numpy(), x["keep_k"].numpy(), heads=heads)
    rels = []
    for name, got, r in zip(("dQ", "dK", "dV"), plan._grads, ref):
        gs, rs = f64(got)[0, :, 1], r[0, :, 1]
        rel = float(np.linalg.norm(gs - rs) / np.linalg.norm(rs))
        assert rel <= TOL_GRAD, f"{name} relative Frobenius error {rel:.3e}"
        rels.append(rel)
    print(f"sweep {mode} nb={nb} keep={keep} T={T}: fwd max-abs {err:.2e} lse {lerr:.2e}; "
          f"bwd rel {rels[0]:.2e} {rels[1]:.2e} {rels[2]:.2e}")
