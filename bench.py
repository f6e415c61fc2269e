#!/usr/bin/env python
"""Benchmark of the sparse causal flash attention hot path on one MI355X.

One step = the whole hash-sparse forward path over one batch of resident
synthetic inputs: LSH buckets of Q and K, stable sort by bucket into the
bucket-aligned layout, tile range tables, attention forward (the gather into
sorted order fused into its loads, output scattered back to original
positions). Workload: B=2, H=12, T=16384, D=64, nb=16, bf16 inputs,
N(0,1) values (the language-model shapes of the explainer of arXiv
2306.01160: 12 heads of 64 dimensions, 16 buckets).

Prints ONE JSON line. `value` = visible-pair TFLOP/s of the whole step
(4*D FLOPs per visible (query, key) pair / step time). Extra keys give the
forward kernel alone (TFLOP/s, fraction of the bf16 MFMA peak), its speedup
over the same kernel run dense-causal on the same shape, per-stage times and
achieved GB/s of the preprocessing, the roofline of the forward kernel, and
the CPU oracle timed on a bounded sample.

Before anything is timed, the timed workloads are checked against the CPU
oracle: the hash step's output on every row of two heads, the QK-drop steps'
on sampled rows of every head; a miss ends the run without a figure. The
QK-drop forward at T=8192 (keep 0.7 and 0.5) and both training steps
(forward + backward, hash at T=16384 and QK-drop at T=8192) are reported
beside the hash line, each against its dense-causal twin.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FWD_SOURCE = os.path.join(ROOT, "io_aware_attention_head_amd", "csrc", "scfa_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_hash_bf16_t16384_nb16.json")


def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hash_bf16_t16384_nb16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (HBM counter calibration) and exit")
    ap.add_argument("--fwd-only", action="store_true", help="only launch the forward kernel in the timed loop "
                                                            "(for counter collection)")
    ap.add_argument("--bwd-only", action="store_true", help="only launch the backward of the hash training "
                                                            "workload in a timed loop (for counter collection)")
    ap.add_argument("--no-train", action="store_true", help="skip the backward (training) figures")
    ap.add_argument("--no-qk", action="store_true", help="skip the QK-drop T=8192 figures")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: the isolated sweeps of the explainer's runtime figures "
                         "(hash nb x T, QK keep x T; forward and forward+backward against dense causal), one JSON "
                         "line per point")
    return ap.parse_args()


def _copy_calibration():
    import torch
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}))


def _cores():
    return len(os.sched_getaffinity(0))


def _oracle_hash_heads(w, x, nh):
    """The float64 oracle, untuned, on the first `nh` heads (b = 0) of a hash
    workload: LSH bucket + stable sort of those heads' queries and keys and
    the explicit masked-softmax forward over all of their rows."""
    import oracle
    sl = slice(0, nh)
    q = x["q"][0:1, :, sl].double().numpy()
    k = x["k"][0:1, :, sl].double().numpy()
    v = x["v"][0:1, :, sl].double().numpy()
    R = x["R"][sl].double().numpy()
    bq = oracle.hash_bucket(q, R, w.nb)
    bk = oracle.hash_bucket(k, R, w.nb)
    oracle.hash_sort(bq, w.nb)
    oracle.hash_sort(bk, w.nb)
    O, lse = oracle.attention_fwd("hash", q, k, v, bkt_q=bq, bkt_k=bk)
    return O, lse, bq, bk


def _compare(O_gpu, lse_gpu, O_ref, lse_ref, tol_o, tol_lse=1e-3):
    """Element-wise comparison of the GPU output with the oracle's (same
    rows and heads): O max-abs, LSE max-abs on finite entries, the -inf
    pattern of the LSE."""
    import numpy as np
    Og = O_gpu.double().cpu().numpy()
    Lg = lse_gpu.double().cpu().numpy()
    o_err = float(np.abs(Og - O_ref).max())
    same_inf = bool(np.array_equal(np.isneginf(Lg), np.isneginf(lse_ref)))
    fin = np.isfinite(lse_ref)
    l_err = float(np.abs(Lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    ok = bool(np.isfinite(Og).all()) and o_err <= tol_o and l_err <= tol_lse and same_inf
    return {"max_abs_O": o_err, "max_abs_lse": l_err, "lse_neg_inf_pattern_equal": same_inf, "tol_O": tol_o,
            "tol_lse": tol_lse, "ok": ok}


def _sampled_parity(mode, x_cpu, O, lse, nrows=24, seed=0, R=None, nb=16):
    """O and LSE of heads (0, 0) and (0, H-1) on `nrows` sampled rows (and
    the first and last) against the oracle; R overrides the workload's
    rotation in hash mode."""
    import numpy as np
    import torch
    import oracle
    B, T, H, D = x_cpu["q"].shape
    rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(T, nrows, replace=False), [0, T - 1]]))
    hs = sorted({0, H - 1})
    q, k, v = (x_cpu[n][0:1, :, hs].double().numpy() for n in ("q", "k", "v"))
    kw = {}
    if mode == "hash":
        Rh = (x_cpu["R"] if R is None else R.cpu())[hs].double().numpy()
        kw = {"bkt_q": oracle.hash_bucket(q, Rh, nb), "bkt_k": oracle.hash_bucket(k, Rh, nb)}
    elif mode == "qk":
        kw = {"keep_q": x_cpu["keep_q"][0:1, :, hs].numpy(), "keep_k": x_cpu["keep_k"][0:1, :, hs].numpy()}
    Or, Lr = oracle.attention_fwd(mode, q, k, v, rows=rows, **kw)
    ri = torch.from_numpy(rows).to(O.device)
    hi = torch.tensor(hs, device=O.device)
    par = _compare(O[0:1][:, ri][:, :, hi], lse[0:1][:, hi][:, :, ri], Or[:, rows], Lr[:, :, rows], 1e-2)
    par["sample"] = f"{len(rows)} sampled rows of heads {[(0, h) for h in hs]}"
    return par


def _hash_parity_and_cpu_baseline(w, x_cpu, plan, nh=2, runs=3):
    """Oracle leg of the hash line, run before anything is timed: the oracle
    on `nh` heads (b=0, all rows) once (warm-up), compared element by element
    with the plan's output; then `runs` more timed runs whose median is the
    CPU baseline (BLAS threads = the cores available to this process)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    n = _cores()
    with threadpool_limits(n):
        O, lse, bq, bk = _oracle_hash_heads(w, x_cpu, nh)
        par = _compare(plan.O[0:1, :, :nh], plan.lse[0:1, :nh], O, lse, 1e-2)
        par["sample"] = f"every row of heads (b=0, h=0..{nh - 1}) of {w.name}"
        if not par["ok"]:
            return par, None
        times = []
        for _ in range(runs):
            t0 = time.perf_counter()
            _oracle_hash_heads(w, x_cpu, nh)
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    pairs = int(oracle.visible_pairs("hash", w.T, 1, nh, bkt_q=bq, bkt_k=bk).sum())
    cpu = {"value": 4 * w.D * pairs / dt / 1e12, "unit": "visible-pair TFLOP/s", "cores": n, "kind": "oracle",
           "seconds_median": round(dt, 3), "seconds_runs": [round(t, 3) for t in times], "runs": runs,
           "sample": f"{nh} of {w.B * w.H} heads (b=0, h=0..{nh - 1}) of {w.name}: float64 LSH bucket + stable "
                     f"sort of their queries and keys, explicit masked-softmax forward over all {w.T} rows "
                     f"({pairs} visible pairs); one warm-up run (the parity check), median of {runs}"}
    return par, cpu


def _one_thread_baselines():
    """The oracle at one BLAS thread on the small workloads: the fp32 QK-drop
    case T=256 (count, compaction and forward; median of 9) and the dense
    causal bf16 case T=2048 on 8 of its 48 heads (forward; median of 3)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs
    out = {}
    w1 = WORKLOADS["qk_f32_t256"]
    x1 = make_inputs(w1)
    q, k, v = (x1[n].double().numpy() for n in ("q", "k", "v"))
    kq, kk = x1["keep_q"].numpy(), x1["keep_k"].numpy()
    pairs1 = int(oracle.visible_pairs("qk", w1.T, w1.B, w1.H, kq, kk).sum())
    with threadpool_limits(1):
        ts = []
        for _ in range(10):
            t0 = time.perf_counter()
            oracle.qk_count(kq)
            oracle.qk_count(kk)
            oracle.attention_fwd("qk", q, k, v, kq, kk)
            ts.append(time.perf_counter() - t0)
    dt = float(np.median(ts[1:]))
    out[w1.name] = {"value": 4 * w1.D * pairs1 / dt / 1e12, "unit": "visible-pair TFLOP/s", "cores": 1,
                    "seconds_median": round(dt, 5), "runs": 9, "sample": "whole workload (B=1, H=2, T=256): keep "
                                                                         "counts and forward"}
    w2 = WORKLOADS["dense_bf16_t2048"]
    x2 = make_inputs(w2)
    nh = 8
    q, k, v = (x2[n][0:1, :, :nh].double().numpy() for n in ("q", "k", "v"))
    pairs2 = nh * w2.T * (w2.T + 1) // 2
    with threadpool_limits(1):
        ts = []
        for _ in range(4):
            t0 = time.perf_counter()
            oracle.attention_fwd("dense", q, k, v)
            ts.append(time.perf_counter() - t0)
    dt = float(np.median(ts[1:]))
    out[w2.name] = {"value": 4 * w2.D * pairs2 / dt / 1e12, "unit": "visible-pair TFLOP/s", "cores": 1,
                    "seconds_median": round(dt, 4), "runs": 3,
                    "sample": f"{nh} of {w2.B * w2.H} heads (b=0, h=0..{nh - 1}), forward over all {w2.T} rows"}
    return out


def _grad_identities(plan, dO):
    """Properties of the gradients that hold at any size, checked on the GPU
    before the backward is timed: every gradient finite; per head the key
    gradients sum to zero (the rows of dS sum to zero) and the value
    gradients sum to the upstream gradients of the rows that see a key; rows
    without a visible key get dQ = 0."""
    import torch
    dQ, dK, dV = plan._grads
    ok = all(bool(torch.isfinite(t).all().item()) for t in (dQ, dK, dV))
    has = torch.isfinite(plan.lse).permute(0, 2, 1)  # (B, T, H)
    sk = dK.double().sum(dim=1)
    ok &= bool((sk.abs() <= 2e-2 * dK.double().abs().sum(dim=1).amax(dim=-1, keepdim=True) + 1e-9).all().item())
    ref_v = (dO.double() * has[..., None]).sum(dim=1)
    ok &= bool(((dV.double().sum(dim=1) - ref_v).abs() <= 2e-2 * (ref_v.abs().amax(dim=-1, keepdim=True) + 1)).all()
               .item())
    ok &= bool((dQ[~has] == 0).all().item())
    return ok


def _backward_graph(plan, dO, name, mode):
    """One HIP graph of plan.backward(dO) (backward table, dQ, dK/dV), checked
    bit for bit against the eager call over three replays with eager work in
    between; the backward allocates nothing after its first call and records
    no memset."""
    import torch
    plan.backward(dO)
    torch.cuda.synchronize()
    ref = [t.clone() for t in plan._grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.backward(dO)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.backward(dO)
    for _ in range(3):
        for t in plan._grads:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(plan._grads, ref)):
            raise SystemExit(f"{name} ({mode}): the backward graph replay differs from the eager backward")
        plan.backward(dO)  # eager work between the replays
        torch.cuda.synchronize()
    return graph


def _train_one(name, K):
    """Forward + backward of one training workload and of its dense-causal
    twin (same kernels, positions 0..T-1): the recomputation backward
    (backward table, dQ (with Delta) and dK/dV kernels) timed after a forward
    with HIP events as replays of one HIP graph (checked against the eager
    call; the eager-launch time is reported beside it), the forward kernel
    timed on its own."""
    import torch
    import io_aware_attention_head_amd.scfa as scfa
    from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs

    wt = WORKLOADS[name]
    xt = {k: v.to("cuda:0") for k, v in make_inputs(wt).items()}
    res = {"workload": wt.name, "mode": wt.mode, "B": wt.B, "H": wt.H, "T": wt.T, "D": wt.D}
    if wt.mode == "hash":
        res["nb"] = wt.nb
    else:
        res["keep"] = wt.keep_p
    for mode in (wt.mode, "dense"):
        plan = scfa.Plan(mode, wt.B, wt.H, wt.T, wt.D, torch.bfloat16, nb=wt.nb)
        plan.run(xt)
        for _ in range(2):
            plan.backward(xt["dO"])
        torch.cuda.synchronize()
        if not _grad_identities(plan, xt["dO"]):
            raise SystemExit(f"{name} ({mode}): gradient identities fail; nothing timed")
        pairs = int(plan.count_visible().sum().item())
        ms_eager = _time_ms(lambda: plan.backward(xt["dO"]), K)
        graph = _backward_graph(plan, xt["dO"], name, mode)
        ms = _time_ms(graph.replay, K)
        fms = _time_ms(plan.forward, K)
        tf = 10 * wt.D * pairs / (ms * 1e-3) / 1e12
        tfb = 14 * wt.D * pairs / ((ms + fms) * 1e-3) / 1e12
        key = "sparse" if mode == wt.mode else "dense"
        res[key] = {"bwd_ms": round(ms, 5), "bwd_ms_eager_launches": round(ms_eager, 5), "bwd_tflops": round(tf, 2),
                    "pct_bf16_peak_bwd": round(100 * tf / PEAK_BF16_TFLOPS, 2), "visible_pairs": pairs,
                    "fwd_kernel_ms": round(fms, 5), "fwd_bwd_ms": round(ms + fms, 5),
                    "fwd_bwd_tflops": round(tfb, 2), "pct_bf16_peak_fwd_bwd": round(100 * tfb / PEAK_BF16_TFLOPS, 2)}
        del plan
        torch.cuda.empty_cache()
    res["speedup_vs_dense_causal_bwd"] = round(res["dense"]["bwd_ms"] / res["sparse"]["bwd_ms"], 3)
    res["speedup_vs_dense_causal_fwd_bwd"] = round(res["dense"]["fwd_bwd_ms"] / res["sparse"]["fwd_bwd_ms"], 3)
    res["checked"] = "gradient identities on every head (finite; sum dK = 0; sum dV = sum dO over rows with a key)"
    return res


def _train_figures(K):
    """Both training steps: hash-sparse (B=1, H=12, T=16384, nb=16) and
    QK-drop (B=1, H=12, T=8192, keep 0.5), forward + backward, each against
    its dense-causal twin (4 D + 10 D FLOPs per visible pair)."""
    out = {name: _train_one(name, K) for name in ("train_hash_bf16_t16384_nb16", "train_qk_bf16_t8192_keep0.5")}
    out["flop_convention"] = ("10*D per visible pair for the backward (dV, dP, dQ, dK products and the recomputed "
                              "scores); 14*D for forward+backward")
    return out


def _qk_figures(K, warmup):
    """QK-drop forward at B=2, H=12, T=8192 (keep 0.7 and 0.5): parity on
    sampled rows of every head against the oracle first, then the whole step
    (keep counts, compaction into index arrays, tables, launch order,
    forward) as a graph replay and the forward kernel on its own (HIP events
    around each launch in the step's order), against the same kernel run
    dense-causal on the same shape."""
    import numpy as np
    import torch
    import oracle
    import io_aware_attention_head_amd.scfa as scfa
    from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs

    out = {}
    dense_ms = None
    rng = np.random.default_rng(17)
    for name in ("qk_bf16_t8192_keep0.7", "qk_bf16_t8192_keep0.5"):
        w = WORKLOADS[name]
        x_cpu = make_inputs(w)
        x = {k: v.to("cuda:0") for k, v in x_cpu.items()}
        plan = scfa.Plan("qk", w.B, w.H, w.T, w.D, torch.bfloat16)
        plan.run(x)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([rng.choice(w.T, 48, replace=False), [0, w.T - 1]]))
        kq, kk = x_cpu["keep_q"].numpy(), x_cpu["keep_k"].numpy()
        Or, Lr = oracle.attention_fwd("qk", *(x_cpu[n].double().numpy() for n in ("q", "k", "v")), kq, kk, rows=rows)
        ri = torch.from_numpy(rows).to(plan.O.device)
        par = _compare(plan.O[:, ri], plan.lse[:, :, ri], Or[:, rows], Lr[:, :, rows], 1e-2)
        par["sample"] = f"{len(rows)} sampled rows of every head"
        if not par["ok"] or int(plan.dev_err.item()) != 0:
            raise SystemExit(f"{name}: parity against the oracle fails ({par}); nothing timed")
        pairs = int(plan.count_visible().sum().item())
        ref_pairs = int(oracle.visible_pairs("qk", w.T, w.B, w.H, kq, kk).sum())
        if pairs != ref_pairs:
            raise SystemExit(f"{name}: visible pairs {pairs} != oracle {ref_pairs}; nothing timed")
        tiles = int(plan.tab.tiles.sum().item())
        # per-stage times (eager): compaction, tables + launch order, forward
        stages = {"compact": lambda: plan.compact(x["q"], x["k"], x["keep_q"], x["keep_k"]), "tables": plan.tables,
                  "forward": plan.forward}
        ev = {s: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
              for s in stages}
        torch.cuda.synchronize()
        for i in range(K):
            for s, fn in stages.items():
                ev[s][i][0].record()
                fn()
                ev[s][i][1].record()
        torch.cuda.synchronize()
        stage_ms = {s: sum(a.elapsed_time(b) for a, b in ev[s]) / K for s in stages}
        graph = plan.capture(x)
        for _ in range(max(1, warmup)):
            graph.replay()
        step_ms = _time_ms(graph.replay, K)
        if dense_ms is None:
            dense = scfa.Plan("dense", w.B, w.H, w.T, w.D, torch.bfloat16)
            dense.run(x)
            torch.cuda.synchronize()
            dpar = _sampled_parity("dense", x_cpu, dense.O, dense.lse, seed=2)
            if not dpar["ok"]:
                raise SystemExit(f"dense-causal twin: parity against the oracle fails ({dpar}); nothing timed")
            dense_pairs = int(dense.count_visible().sum().item())
            dense_tiles = int(dense.tab.tiles.sum().item())
            dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            for a, b in dev_ev:
                a.record()
                dense.forward()
                b.record()
            torch.cuda.synchronize()
            dense_ms = sum(a.elapsed_time(b) for a, b in dev_ev) / K
            out["dense_causal_twin"] = {"B": w.B, "H": w.H, "T": w.T, "fwd_kernel_ms": round(dense_ms, 5),
                                        "fwd_kernel_tflops": round(4 * w.D * dense_pairs / (dense_ms * 1e-3) / 1e12, 2),
                                        "tiles_processed": dense_tiles, "parity": dpar}
            del dense
        fwd_ms = stage_ms["forward"]
        tf = 4 * w.D * pairs / (fwd_ms * 1e-3) / 1e12
        out[name] = {"keep": w.keep_p, "B": w.B, "H": w.H, "T": w.T, "D": w.D, "visible_pairs": pairs,
                     "step_ms": round(step_ms, 5), "step_tflops": round(4 * w.D * pairs / (step_ms * 1e-3) / 1e12, 2),
                     "fwd_kernel_ms": round(fwd_ms, 5), "fwd_kernel_tflops": round(tf, 2),
                     "pct_bf16_peak_fwd": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                     "speedup_vs_dense_causal_fwd": round(dense_ms / fwd_ms, 3),
                     "stage_ms": {s: round(v, 5) for s, v in stage_ms.items()}, "tiles_processed": tiles,
                     "tiles_skipped_frac_vs_dense_causal": round(1 - tiles / out["dense_causal_twin"]["tiles_processed"],
                                                                 4),
                     "parity": par}
        del plan, graph, x
        torch.cuda.empty_cache()
    return out


class _ClockSampler:
    """Shader clock as the driver reports it (the active level of the
    amdgpu sysfs pp_dpm_sclk file), sampled every 5 ms on a host thread
    while the GPU work runs. None when no such file is readable."""

    def __init__(self):
        import glob
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = False
        self._t = None

    def _read(self):
        vals = []
        for f in self.files:
            try:
                for line in open(f):
                    if "*" in line:
                        vals.append(float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]))
            except (OSError, ValueError, IndexError):
                pass
        return vals

    def _loop(self):
        while not self._stop:
            v = self._read()
            if v:
                self.samples.append(max(v))
            time.sleep(0.005)

    def __enter__(self):
        import threading
        if self.files:
            self._t = threading.Thread(target=self._loop, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop = True
        if self._t is not None:
            self._t.join()

    def result(self):
        if not self.samples:
            return {"mhz_median": None, "source": "no readable pp_dpm_sclk in sysfs"}
        import statistics
        return {"mhz_median": statistics.median(self.samples), "mhz_min": min(self.samples),
                "mhz_max": max(self.samples), "samples": len(self.samples),
                "source": "amdgpu sysfs pp_dpm_sclk, active DPM level, sampled every 5 ms over the GPU work of this run"}


def _stress_figures(w, x, x_cpu, K, dense_fwd_ms):
    """Skewed buckets (reported, not targeted): the benchmark workload with
    rotation column 0 biased by +3, which pulls most tokens into buckets 0
    and nb/2; the pages warn that such imbalance erodes the gain."""
    import torch
    import io_aware_attention_head_amd.scfa as scfa

    xs = dict(x)
    R = x["R"].clone()
    R[:, :, 0] += 3.0
    xs["R"] = R
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, torch.bfloat16, nb=w.nb)
    plan.run(xs)
    torch.cuda.synchronize()
    sizes = torch.stack([torch.bincount(b.flatten(), minlength=w.nb) for b in (plan.bq, plan.bk)]).float()
    frac = (sizes.max(dim=1).values / sizes.sum(dim=1)).max().item()
    pairs = int(plan.count_visible().sum().item())
    par = _sampled_parity("hash", x_cpu, plan.O, plan.lse, seed=3, R=R, nb=w.nb)
    if not par["ok"]:
        raise SystemExit(f"skewed buckets: parity against the oracle fails ({par}); nothing timed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        plan.run(xs)
    b.record()
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / K
    a.record()
    for _ in range(K):
        plan.forward()
    b.record()
    torch.cuda.synchronize()
    fms = a.elapsed_time(b) / K
    return {"rotation": "R[:, :, 0] += 3", "largest_bucket_frac": round(frac, 4), "visible_pairs": pairs,
            "step_ms_eager_launches": round(step_ms, 5), "fwd_kernel_ms": round(fms, 5),
            "fwd_kernel_tflops": round(4 * w.D * pairs / (fms * 1e-3) / 1e12, 2),
            "speedup_vs_dense_causal_fwd": round(dense_fwd_ms / fms, 3), "parity": par}


def _time_ms(fn, K):
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def _sweep(K):
    """Isolated runtime sweeps in the manner of the explainer's figures
    ("Experimental Results": hash-sparse runtime against nb and T, QK-sparse
    against the drop rate and T) at B=1, H=12, D=64, bf16: for each point the
    preprocessing + forward (eager launches), the forward kernel, the
    backward, and the same kernels run dense-causal on the same shape. One
    JSON line per point; the dense twin is timed once per T."""
    import torch
    import io_aware_attention_head_amd.scfa as scfa
    from io_aware_attention_head_amd.inputs import make_inputs, small

    dense = {}
    for T in (1024, 2048, 4096, 8192, 16384):
        wd = small("dense", 1, 12, T, seed=90, grad=True)
        xd = {k: v.to("cuda:0") for k, v in make_inputs(wd).items()}
        pd = scfa.Plan("dense", 1, 12, T, 64, torch.bfloat16)
        pd.run(xd)
        dense[T] = {"fwd_ms": _time_ms(pd.forward, K), "bwd_ms": _time_ms(lambda: pd.backward(xd["dO"]), K)}
        del pd, xd
        torch.cuda.empty_cache()
    points = [("hash", nb, None, T) for nb in (2, 4, 8, 16, 32, 64) for T in (1024, 2048, 4096, 8192, 16384)]
    points += [("qk", 16, keep, T) for keep in (0.7, 0.5, 0.3) for T in (1024, 2048, 4096, 8192, 16384)]
    for mode, nb, keep, T in points:
        w = small(mode, 1, 12, T, nb=nb, keep_p=keep if keep is not None else 0.7, seed=91, grad=True)
        x = {k: v.to("cuda:0") for k, v in make_inputs(w).items()}
        pl = scfa.Plan(mode, 1, 12, T, 64, torch.bfloat16, nb=nb)
        pl.run(x)
        pairs = int(pl.count_visible().sum().item())
        step = _time_ms(lambda: pl.run(x), K)
        fwd = _time_ms(pl.forward, K)
        bwd = _time_ms(lambda: pl.backward(x["dO"]), K)
        d = dense[T]
        rec = {"sweep": "hash_nb_T" if mode == "hash" else "qk_keep_T", "mode": mode, "T": T, "B": 1, "H": 12,
               "D": 64, "visible_pairs": pairs, "prep_fwd_ms_eager": round(step, 4), "fwd_kernel_ms": round(fwd, 4),
               "bwd_ms": round(bwd, 4), "fwd_tflops": round(4 * 64 * pairs / (fwd * 1e-3) / 1e12, 1),
               "dense_fwd_ms": round(d["fwd_ms"], 4), "dense_bwd_ms": round(d["bwd_ms"], 4),
               "speedup_fwd": round(d["fwd_ms"] / fwd, 3), "speedup_fwd_bwd": round((d["fwd_ms"] + d["bwd_ms"]) /
                                                                                 (fwd + bwd), 3),
               "speedup_prep_fwd": round(d["fwd_ms"] / step, 3)}
        rec["nb" if mode == "hash" else "keep"] = nb if mode == "hash" else keep
        print(json.dumps(rec), flush=True)
        del pl, x
        torch.cuda.empty_cache()


def _bwd_only(K):
    """The backward of the hash training workload in a timed loop (for
    counter collection): backward table, dQ (with Delta) and dK/dV kernels."""
    import torch
    import io_aware_attention_head_amd.scfa as scfa
    from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs

    wt = WORKLOADS["train_hash_bf16_t16384_nb16"]
    xt = {k: v.to("cuda:0") for k, v in make_inputs(wt).items()}
    plan = scfa.Plan("hash", wt.B, wt.H, wt.T, wt.D, torch.bfloat16, nb=wt.nb)
    plan.run(xt)
    plan.backward(xt["dO"])
    torch.cuda.synchronize()
    if not _grad_identities(plan, xt["dO"]):
        raise SystemExit("gradient identities fail; nothing timed")
    ms = _time_ms(lambda: plan.backward(xt["dO"]), K)
    print(json.dumps({"workload": wt.name, "bwd_ms": round(ms, 5), "steps": K}), flush=True)


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); the hot path "
              f"needs no communication and shards per head; no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        _copy_calibration()
        return
    if args.sweep:
        _sweep(args.steps)
        return
    if args.bwd_only:
        _bwd_only(args.steps)
        return
    import io_aware_attention_head_amd.scfa as scfa
    from io_aware_attention_head_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if w.mode != "hash" or w.grad:
        raise SystemExit("bench.py times the hash-sparse forward workload")
    dev = torch.device("cuda:0")
    x_cpu = make_inputs(w)
    x = {k: v.to(dev) for k, v in x_cpu.items()}
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    plan = scfa.Plan("hash", w.B, w.H, w.T, w.D, dtype, nb=w.nb)
    dense = scfa.Plan("dense", w.B, w.H, w.T, w.D, dtype)

    # warm-up (also builds the operands the dense twin uses)
    for _ in range(max(1, args.warmup)):
        plan.run(x)
        dense.run(x)
    torch.cuda.synchronize()
    pairs = int(plan.count_visible().sum().item())
    dense_pairs = int(dense.count_visible().sum().item())
    tiles = int(plan.tab.tiles.sum().item())
    dense_tiles = int(dense.tab.tiles.sum().item())
    assert int(plan.dev_err.item()) == 0, "device error flag set"
    assert torch.isfinite(plan.O).all().item(), "non-finite output"
    assert pairs > 0

    # ---- parity against the oracle before anything is timed ----------------
    parity, cpu, dense_parity = None, None, None
    if not args.no_cpu_baseline:
        parity, cpu = _hash_parity_and_cpu_baseline(w, x_cpu, plan)
        dense_parity = _sampled_parity("dense", x_cpu, dense.O, dense.lse, seed=1)
        if not (parity["ok"] and dense_parity["ok"]):
            print(json.dumps({"error": "parity against the oracle fails; nothing timed", "parity": parity,
                              "dense_causal_parity": dense_parity}), flush=True)
            sys.exit(1)

    stages = ["bucket", "sort", "tables", "forward"]
    fns = {"bucket": lambda: plan.bucket(x["q"], x["k"], x["R"]), "sort": plan.sort, "tables": plan.tables,
           "forward": plan.forward}
    if args.fwd_only:
        stages = ["forward"]
    K = args.steps
    ev = {s: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for s in stages}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # ---- per-stage times, eager launches ---------------------------------------
    clock = _ClockSampler().__enter__()  # sampled over all the GPU work from here on
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        for s in stages:
            ev[s][i][0].record()
            fns[s]()
            ev[s][i][1].record()
    end.record()
    torch.cuda.synchronize()
    ms_step_eager = start.elapsed_time(end) / K
    stage_ms = {s: sum(a.elapsed_time(b) for a, b in ev[s]) / K for s in stages}
    O_eager = plan.O.clone()

    # ---- timed region: the step as one HIP graph replay ------------------------
    graph = None
    if not args.fwd_only:
        graph = plan.capture(x)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.O, O_eager), "graph replay differs from the eager step"
        for _ in range(max(1, args.warmup)):
            graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        if graph is not None:
            graph.replay()
        else:
            plan.forward()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    if graph is not None:
        assert torch.equal(plan.O, O_eager), "timed replays differ from the eager step"

    # ---- dense-causal twin: same kernel, same shape, positions 0..T-1 ------
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in dev_ev:
        a.record()
        dense.forward()
        b.record()
    torch.cuda.synchronize()
    dense_fwd_ms = sum(a.elapsed_time(b) for a, b in dev_ev) / K
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dense_graph = dense.capture(x) if graph is not None else None
    torch.cuda.synchronize()
    d0.record()
    for _ in range(K):
        if dense_graph is not None:
            dense_graph.replay()
        else:
            dense.tables()
            dense.forward()
    d1.record()
    torch.cuda.synchronize()
    dense_step_ms = d0.elapsed_time(d1) / K

    fwd_ms = stage_ms["forward"]
    flops = 4 * w.D * pairs
    fwd_tflops = flops / (fwd_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    nQt, nKt = plan.tab.fwd.shape[2], plan.tab.bwd.shape[2]
    esz = 2 if dtype == torch.bfloat16 else 4
    out_esz = 4
    BHT = w.B * w.H * w.T
    # algorithmic bytes: each stage reads its inputs once and writes its outputs once
    alg_bytes = {
        "bucket": 2 * BHT * w.D * esz + 2 * BHT * 4,
        "sort": 2 * (BHT * 4 + 2 * BHT * 4),
        "forward": 3 * BHT * w.D * esz + BHT * w.D * out_esz + BHT * 4,
    }
    prep_gbs = {s: alg_bytes[s] / (stage_ms[s] * 1e-3) / 1e9 for s in ("bucket", "sort") if s in stage_ms}

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE))
            if t.get("fwd_source_sha256_16") == _src_hash(FWD_SOURCE):
                traffic = t.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": "visible-pair TFLOP/s + % bf16 MFMA peak + speedup vs dense causal, T=8k/16k",
        "value": round(step_tflops, 3),
        "unit": "visible-pair TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dtype == torch.bfloat16 else "f32",
        "data": "synthetic: seeded N(0,1) Q/K/V and rotations (no dataset needed)",
        "config": {"workload": w.name, "mode": "hash", "B": w.B, "H": w.H, "T": w.T, "D": w.D, "nb": w.nb,
                   "seed": w.seed, "out_dtype": "f32", "tile_m": scfa.SCFA_TILE_M, "tile_n": scfa.SCFA_TILE_N,
                   "parallelism": "single GPU"},
        "step": "LSH bucket + stable sort + bucket-aligned layout + range tables + attention forward with the gather "
                "fused into its loads (inputs resident in HBM), launched as one HIP graph",
        "parity": parity if parity is not None else "not checked (--no-cpu-baseline)",
        "dense_causal_parity": dense_parity,
        "ms_per_step_eager_launches": round(ms_step_eager, 5),
        "visible_pairs": pairs,
        "fwd_kernel_ms": round(fwd_ms, 5),
        "fwd_kernel_tflops": round(fwd_tflops, 2),
        "pct_bf16_peak_fwd": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "dense_causal_fwd_ms": round(dense_fwd_ms, 5),
        "dense_causal_fwd_tflops": round(4 * w.D * dense_pairs / (dense_fwd_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense_causal_fwd": round(dense_fwd_ms / fwd_ms, 3),
        "dense_causal_step_ms": round(dense_step_ms, 5),
        "speedup_vs_dense_causal_step": round(dense_step_ms / ms_step, 3),
        "stage_ms": {s: round(v, 5) for s, v in stage_ms.items()},
        "preproc_gbs": {s: round(v, 1) for s, v in prep_gbs.items()},
        "tiles_processed": tiles,
        "dense_causal_tiles_processed": dense_tiles,
        "tiles_skipped_frac": round(1 - tiles / dense_tiles, 4),
        "tiles_skipped_denominator": "tiles the same kernel processes dense-causal on this shape",
        "tiles_skipped_frac_vs_layout_rectangle": round(1 - tiles / (nQt * nKt * w.B * w.H), 4),
        "visible_density": round(pairs / (tiles * scfa.SCFA_TILE_M * scfa.SCFA_TILE_N), 4),
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "k_fwd<hash,bf16>", "alg_flops_per_launch": flops,
                     "alg_bytes_per_launch": alg_bytes["forward"]},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "torch": torch.__version__, "hip": torch.version.hip},
        "wall_s_timed": round(wall, 3),
    }
    del graph, dense_graph, dense
    torch.cuda.empty_cache()
    if not args.fwd_only:
        if not args.no_qk:
            out["qk"] = _qk_figures(K, args.warmup)
        if not args.no_train:
            out["train"] = _train_figures(K)
        out["stress_skewed_buckets"] = _stress_figures(w, x, x_cpu, K, dense_fwd_ms)
    torch.cuda.synchronize()
    clock.__exit__()
    clk = clock.result()
    if clk.get("mhz_median"):
        # 4096 bf16 FLOPs per clock per compute unit (dense MFMA)
        clk["peak_bf16_tflops_at_median_clock"] = round(props.multi_processor_count * clk["mhz_median"] * 4096 / 1e6,
                                                        1)
    out["clock"] = clk
    if cpu is not None:
        cpu["one_thread"] = _one_thread_baselines()
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
