"""Shared helpers of the GPU parity tests: run the HIP pipeline through the
C ABI and compute the oracle's expected values on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import io_aware_attention_head_amd.scfa as scfa
from io_aware_attention_head_amd.inputs import make_inputs

# Tolerances: forward max-abs over all of O (1e-2 for bf16 inputs, 1e-4 for
# fp32 inputs), LSE absolute 1e-3 on finite entries and -inf exactly where the
# oracle has -inf, gradients relative Frobenius 2e-2 per tensor.
TOL_O = {"bf16": 1e-2, "f32": 1e-4}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    scfa.lib()  # fail loudly when the library is missing


def dev():
    return torch.device("cuda:0")


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: dict) -> dict:
    return {k: v.to(dev()) for k, v in x.items()}


def np_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a bf16/fp32 tensor as an integer numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def run_pipeline(w, x: dict, out_dtype=torch.float32):
    g = to_dev(x)
    if w.mode == "hash":
        pre = scfa.prepare_hash(g["q"], g["k"], g["v"], g["R"], w.nb)
    elif w.mode == "qk":
        pre = scfa.prepare_qk(g["q"], g["k"], g["v"], g["keep_q"], g["keep_k"])
    else:
        pre = scfa.prepare_dense(g["q"], g["k"], g["v"])
    tab = scfa.build_tables(pre)
    O, lse = scfa.forward(pre, tab, out_dtype)
    torch.cuda.synchronize()
    return g, pre, tab, O, lse


def oracle_buckets(w, x):
    R = x["R"].double().numpy()
    return oracle.hash_bucket(f64(x["q"]), R, w.nb), oracle.hash_bucket(f64(x["k"]), R, w.nb)


def oracle_fwd(w, x, heads=None, rows=None, buckets=None):
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    if w.mode == "hash":
        bq, bk = buckets if buckets is not None else oracle_buckets(w, x)
        return oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk, heads=heads, rows=rows)
    if w.mode == "qk":
        return oracle.attention_fwd("qk", q, k, v, x["keep_q"].numpy(), x["keep_k"].numpy(), heads=heads, rows=rows)
    return oracle.attention_fwd("dense", q, k, v, heads=heads, rows=rows)


def check_fwd(w, O, lse, Or, Lr, heads=None, rows=None):
    """Compare GPU O/LSE with the oracle on the selected heads/rows."""
    Og, Lg = f64(O), f64(lse)
    B, T, H, D = Og.shape
    hs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    rr = np.arange(T) if rows is None else np.asarray(rows)
    worst = 0.0
    lworst = 0.0
    for b, h in hs:
        go, ro = Og[b, rr, h], Or[b, rr, h]
        assert np.isfinite(go).all(), f"non-finite output in head {(b, h)}"
        worst = max(worst, float(np.abs(go - ro).max()))
        gl, rl = Lg[b, h, rr], Lr[b, h, rr]
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"LSE -inf pattern differs in head {(b, h)}"
        assert not np.isnan(gl).any() and not np.isposinf(gl).any()
        fin = np.isfinite(rl)
        if fin.any():
            lworst = max(lworst, float(np.abs(gl[fin] - rl[fin]).max()))
    tol = TOL_O[w.dtype]
    assert worst <= tol, f"forward max-abs error {worst:.3e} > {tol}"
    assert lworst <= TOL_LSE, f"LSE max-abs error {lworst:.3e} > {TOL_LSE}"
    return worst, lworst
