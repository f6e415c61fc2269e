"""Seeded synthetic inputs for sparse causal flash attention.

This module only draws random numbers; it holds none of the attention
arithmetic. Both the HIP path's tests/benchmark and the CPU oracle's tests
take their inputs from here, so the two sides always see the same values.

Shapes follow the explainer of arXiv 2306.01160 ("Faster Causal Attention Over
Large Sequences Through Sparse Flash Attention"): Q, K, V are (B, T, H, D)
("3.2 Big-Picture Architecture", item 2), keep decisions are (B, T, H)
("QK-Sparse Attention: Compaction and Index-Guided Tiling"), and the language
model workloads use 12 heads of 64 dimensions ("System Integration: The
Training Loop").

Recipe (fixed draw order from one seeded CPU ``torch.Generator``):
Q, K, V ~ N(0,1); keep_q, keep_k = U[0,1) < p; R ~ N(0,1) of shape
(H, D, nb/2); dO ~ N(0,1). All draws are float32; bf16 configurations round
Q, K, V and dO to bf16 (round-to-nearest-even) after drawing. R stays float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

MODES = ("dense", "qk", "hash")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str          # "dense" | "qk" | "hash"
    B: int
    H: int
    T: int
    D: int = 64
    dtype: str = "bf16"  # "bf16" | "f32"
    keep_p: float = 1.0  # probability that a token is KEPT (qk mode)
    nb: int = 16         # number of LSH buckets (hash mode)
    seed: int = 0
    grad: bool = False   # also draw dO and run the backward
    Tk: int = 0          # key/value length when it differs from T (0: T)

    @property
    def T_kv(self) -> int:
        return self.Tk if self.Tk else self.T


# The five workloads: a small fp32 QK case, a dense-causal sanity case, QK-drop
# at T=8192 (two keep rates), hash-sparse at T=16384, and a training step
# (forward + backward) in both sparse modes.
WORKLOADS = {
    "qk_f32_t256": Workload("qk_f32_t256", "qk", 1, 2, 256, dtype="f32", keep_p=0.7, seed=1),
    "dense_bf16_t2048": Workload("dense_bf16_t2048", "dense", 4, 12, 2048, seed=2),
    "qk_bf16_t8192_keep0.7": Workload("qk_bf16_t8192_keep0.7", "qk", 2, 12, 8192, keep_p=0.7, seed=3),
    "qk_bf16_t8192_keep0.5": Workload("qk_bf16_t8192_keep0.5", "qk", 2, 12, 8192, keep_p=0.5, seed=4),
    "hash_bf16_t16384_nb16": Workload("hash_bf16_t16384_nb16", "hash", 2, 12, 16384, nb=16, seed=5),
    "train_hash_bf16_t16384_nb16": Workload("train_hash_bf16_t16384_nb16", "hash", 1, 12, 16384, nb=16,
                                            seed=6, grad=True),
    "train_qk_bf16_t8192_keep0.5": Workload("train_qk_bf16_t8192_keep0.5", "qk", 1, 12, 8192, keep_p=0.5,
                                            seed=7, grad=True),
}


def _torch_dtype(name: str) -> torch.dtype:
    if name == "bf16":
        return torch.bfloat16
    if name == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {name!r}")


def make_inputs(w: Workload, keep_override: Optional[float] = None) -> dict:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict of CPU tensors: q (B,T,H,D), k, v (B,Tk,H,D) in the
    workload dtype; keep_q (B,T,H), keep_k (B,Tk,H) uint8 (1 = kept); R
    (H,D,nb/2) float32; dO (B,T,H,D) in the workload dtype. In dense mode the
    keep masks are all ones. Tk is the workload's key length (T unless set).
    """
    if w.mode not in MODES:
        raise ValueError(f"unknown mode {w.mode!r}")
    if w.nb % 2:
        raise ValueError("nb must be even")
    g = torch.Generator().manual_seed(w.seed)
    shape = (w.B, w.T, w.H, w.D)
    kshape = (w.B, w.T_kv, w.H, w.D)
    q = torch.randn(shape, generator=g)
    k = torch.randn(kshape, generator=g)
    v = torch.randn(kshape, generator=g)
    p = w.keep_p if keep_override is None else keep_override
    keep_q = (torch.rand((w.B, w.T, w.H), generator=g) < p).to(torch.uint8)
    keep_k = (torch.rand((w.B, w.T_kv, w.H), generator=g) < p).to(torch.uint8)
    R = torch.randn((w.H, w.D, w.nb // 2), generator=g)
    dO = torch.randn(shape, generator=g)
    if w.mode == "dense":
        keep_q.fill_(1)
        keep_k.fill_(1)
    dt = _torch_dtype(w.dtype)
    return {
        "q": q.to(dt), "k": k.to(dt), "v": v.to(dt),
        "keep_q": keep_q, "keep_k": keep_k, "R": R, "dO": dO.to(dt),
    }


def small(mode: str, B: int, H: int, T: int, D: int = 64, dtype: str = "bf16", keep_p: float = 0.7,
          nb: int = 16, seed: int = 0, grad: bool = False, Tk: int = 0) -> Workload:
    """A named ad-hoc workload for tests (edge cases, ragged shapes); Tk: a
    key/value length other than T."""
    tk = f"Tk{Tk}" if Tk and Tk != T else ""
    return Workload(f"{mode}_{dtype}_B{B}H{H}T{T}{tk}D{D}_s{seed}", mode, B, H, T, D, dtype, keep_p, nb, seed, grad,
                    Tk if Tk != T else 0)
