"""GPU parity on a seeded random sample of small configurations against the
float64 oracle, through the C ABI: every mode (dense, QK-drop, hash,
hash + drop), every position test (causal, strict, non-causal), one or two
sequence lengths, ragged lengths around the tile sizes, bf16 and fp32
inputs. Each case checks the forward outputs on every row, the gradients
(bf16 cases), and the same path through a Plan."""
import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import make_inputs, small
from gpu_util import TOL_GRAD, announce, check_fwd, f64, need_gpu, oracle_buckets, to_dev

pytestmark = pytest.mark.gpu

_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 191, 255, 257, 300, 383, 511, 640]


def _cases(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = ["dense", "qk", "hash", "hash_drop"][i % 4]
        variant = ["causal", "strict", "noncausal"][int(rng.integers(0, 3))]
        T = int(rng.choice(_LENGTHS))
        Tk = int(rng.choice(_LENGTHS)) if rng.random() < 0.4 else T
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        nb = int(rng.choice([2, 4, 8, 16, 32]))
        keep = float(rng.choice([0.3, 0.5, 0.7, 0.9]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        out.append((mode, variant, B, H, T, Tk, nb, keep, dtype, 500 + i))
    return out


CASES = _cases()


def _long_cases(n=8, seed=4048):
    """Longer sequences (ranges beyond one 64-tile window of the tile tests),
    one or two heads."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = ["dense", "qk", "hash", "hash_drop"][i % 4]
        variant = ["causal", "strict", "noncausal"][int(rng.integers(0, 3))]
        T = int(rng.integers(4100, 6000))
        Tk = int(rng.integers(4100, 6000)) if rng.random() < 0.4 else T
        nb = int(rng.choice([2, 4]))  # few buckets: long ranges
        keep = float(rng.choice([0.7, 0.9]))
        out.append((mode, variant, 1, int(rng.integers(1, 3)), T, Tk, nb, keep, "bf16", 700 + i))
    return out


CASES = CASES + _long_cases()


def _ids(c):
    mode, variant, B, H, T, Tk, nb, keep, dtype, seed = c
    return f"{mode}-{variant}-B{B}H{H}T{T}Tk{Tk}-nb{nb}-p{keep}-{dtype}-s{seed}"


def _flags(variant):
    return {"strict": variant == "strict", "noncausal": variant == "noncausal"}


def _oracle(mode, w, x, variant, grad):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    f = _flags(variant)
    if mode in ("hash", "hash_drop"):
        bq, bk = oracle_buckets(w, x)
        kq, kk = (x["keep_q"].numpy(), x["keep_k"].numpy()) if mode == "hash_drop" else (None, None)
        args = ("hash", q, k, v, kq, kk, bq, bk)
    elif mode == "qk":
        args = ("qk", q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), None, None)
    else:
        args = ("dense", q, k, v, None, None, None, None)
    fwd = oracle.attention_fwd(*args, **f)
    bwd = oracle.attention_bwd(*args[:4], f64(x["dO"]), *args[4:], **f) if grad else None
    return fwd, bwd


def _prepare(mode, w, g, variant):
    f = _flags(variant)
    if mode == "hash":
        return scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb, **f)
    if mode == "hash_drop":
        return scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb, keep_q=g["keep_q"], keep_k=g["keep_k"], **f)
    if mode == "qk":
        return scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"], **f)
    return scfa.prepare_dense(g["q"], g["k"], g["v"], **f)


def _check_grads(grads, ref, what):
    for name, got, r in zip(("dQ", "dK", "dV"), grads, ref):
        gn = f64(got)
        assert np.isfinite(gn).all(), f"{what} {name} not finite"
        den = np.linalg.norm(r)
        rel = float(np.linalg.norm(gn - r) / den) if den > 0 else float(np.abs(gn).max())
        assert rel <= TOL_GRAD, f"{what} {name} relative Frobenius error {rel:.3e}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_random_config(case):
    mode, variant, B, H, T, Tk, nb, keep, dtype, seed = case
    need_gpu()
    announce(f"random {_ids(case)}")
    grad = dtype == "bf16"
    w = small("hash" if mode == "hash_drop" else mode, B, H, T, nb=nb, keep_p=keep, dtype=dtype, seed=seed, grad=grad,
              Tk=Tk)
    x = make_inputs(w)
    g = to_dev(x)
    (Or, Lr), ref = _oracle(mode, w, x, variant, grad)

    # the functional path: preprocessing, tables, forward, backward
    pre = _prepare(mode, w, g, variant)
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab)
    grads = scfa.backward(pre, tab, O, lse, g["dO"]) if grad else None
    torch.cuda.synchronize()
    check_fwd(w, O, lse, Or, Lr)
    if grad:
        _check_grads(grads, ref, "call")

    # the same configuration through a Plan (its own launches and tables)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    plan = scfa.Plan(mode, B, H, T, w.D, dt, nb=nb, T_kv=Tk, **_flags(variant))
    plan.run(g)
    pgrads = plan.backward(g["dO"]) if grad else None
    torch.cuda.synchronize()
    assert int(plan.dev_err.item()) == 0
    check_fwd(w, plan.O, plan.lse, Or, Lr)
    if grad:
        _check_grads(pgrads, ref, "plan")
