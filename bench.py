"""Benchmark of the fused linear log-prob on one MI355X.

One step is one pass of the whole path over one batch: active-row compaction, the vocab
tile kernel with its fused softmax-statistics epilogue, the fixed-order merge (the
forward), then the chunked backward of L = -sum_t mask_t adv_t logp_t.  The headline step
is rlk_linear_logp_fwd_bwd, which does all of it in one call: each token block's forward
keeps its logits (16-bit codes, relative to the column maximum) in the workspace, so the backward
forms dL/dz from them instead of running the logits GEMM again.  The same step as two calls
(rlk_linear_logp_fwd, then rlk_linear_logp_bwd, which recomputes the logits) is timed beside
it.  The default workload is the Qwen3-8B LM-head shape with N=16384 tokens in 64 packed
sequences (~60% active), T=0.7 and targets sampled from the oracle softmax (stored under
tests/golden), with per-sequence advantages ~N(0,1) for the backward.  Inputs are seeded
synthetic data, resident in HBM before the timed region.

Prints one JSON line.  `value` is active tokens per second for the whole step; the
forward alone, the two-call step, and the roofline of the forward tile kernel (the GEMM
kernel of both forms, timed with HIP events on the stream it runs on) are reported beside
it, and the float64 CPU oracle is timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "active tokens/sec + % bf16 MFMA peak, fused linear logp fwd (and fwd+bwd)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOADS = {
    # name: (config id, use stored sampled targets)
    "tiny-fp32-N64-H256-V1000": (1, False),
    "qwen3-8b-head-N16384-T0.7": (3, True),
    "qwen3-8b-head-N4096-fwdbwd": (5, False),
    "qwen3-8b-head-N2048": (2, False),
    "large-hidden-head-N8192-H7168": (4, False),
}
DEFAULT_WORKLOAD = "qwen3-8b-head-N16384-T0.7"
# Sources of the forward tile kernel: a stored traffic measurement is used only while these
# are byte-identical to what was profiled.
FWD_TILE_SOURCES = [f"linear_selected_token_amd/csrc/{f}"
                    for f in ("fwd.hip", "common.hpp", "mainloop.hpp", "kernels.hpp")]
LOGITS_SOURCES = [f"linear_selected_token_amd/csrc/{f}"
                  for f in ("logits.hip", "common.hpp", "kernels.hpp")]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    p.add_argument("--mode", default="fwdbwd",
                   choices=["fwd", "fwdbwd", "entropy", "ppo", "kl", "logits", "gemm-reference"],
                   help="fwdbwd: forward and backward (the headline: one fused call, and the "
                        "two calls beside it); fwd: forward "
                        "only; entropy: a step with an entropy bonus (the entropy forward and "
                        "its backward); ppo: forward, clipped policy-gradient loss with a KL "
                        "penalty, backward, plus the dlogp diagnostics; kl: full-vocabulary KL "
                        "to a teacher head of the same shape, forward and backward; gemm-reference: "
                        "the vendor library's plain bf16 GEMM of the forward's shape (it writes "
                        "the logits), as a reference point for the tile kernel; logits: log-prob from existing "
                        "bf16 logits of the same shape (an HBM-bound path, reported against "
                        "HBM bandwidth)")
    p.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample (0 disables it)")
    p.add_argument("--configs", type=int, default=1,
                   help="with the default workload and mode, also time the other workloads "
                        "(configs 1, 2, 4, 5) and add them under 'configs' (0 skips them)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB (to scale "
                        "the profiler's HBM byte counters) and exit")
    return p.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size: reads and writes `mib` MiB once."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def make_workload(name):
    import workloads as wl
    cfg, sampled = WORKLOADS[name]
    w = wl.make(cfg)
    if sampled:
        t = np.load(os.path.join(ROOT, "tests", "golden", "cfg3_sampled_targets.npy"))
        w = wl.with_targets(w, t)
    return w


def cpu_baseline(w, mode, target_s):
    """Time the float64 oracle on a bounded sample of active tokens of the same workload."""
    import oracle
    import workloads as wl
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    act = np.nonzero(w.mask)[0]
    W64 = wl.as_f64(w.W)
    h64 = wl.as_f64(w.h[act])
    m = np.ones(act.size, dtype=np.uint8)
    y = w.targets[act]
    adv = w.adv[act]
    res = {}

    def run(n):
        t0 = time.perf_counter()
        res["logp"], _ = oracle.linear_logp(h64[:n], W64, y[:n], m[:n], w.T)
        if mode == "entropy":
            oracle.entropy(h64[:n], W64, m[:n], w.T)
            oracle.linear_logp_entropy_grads(h64[:n], W64, y[:n], m[:n], w.T, adv[:n],
                                             np.full(n, 0.01))
        elif mode != "fwd":
            oracle.linear_logp_grads(h64[:n], W64, y[:n], m[:n], w.T, adv[:n])
        return time.perf_counter() - t0

    # one calibration run (its fixed costs make the per-token estimate an overestimate, so
    # the sample stays within about target_s seconds), then the timed sample
    k = min(act.size, 128)
    per = run(k) / k
    n = int(min(act.size, max(k, target_s / max(per, 1e-9))))
    n = max(16, (n // 16) * 16)
    dt = run(n)
    what = {"fwd": "forward",
            "entropy": "forward + entropy + gradients with an entropy bonus"}.get(
        mode, "forward + dL/dh + dL/dW")
    # the oracle's work is its BLAS calls, so the threads it used are the BLAS pool's, at most
    # the CPUs this process may run on
    out = {"value": n / dt, "unit": "active tokens/s", "cores": int(min(blas, affinity)),
           "kind": "oracle", "blas_threads": int(blas), "cpus_in_affinity": int(affinity),
           "sample": f"first {n} active tokens of the same workload scored as one batch "
                     f"({what}, float64, numpy/OpenBLAS), {dt:.1f} s"}
    return out, act[:n], res["logp"]


def sample_parity(logp_gpu, rows, oracle_logp):
    """max |dlogp| of the measured run's logp against the oracle's on the CPU sample, and the
    dlogp diagnostics of the same comparison computed by the library on the GPU."""
    import torch
    import linear_selected_token_amd as rlk
    dev = logp_gpu.device
    idx = torch.from_numpy(np.asarray(rows)).to(dev)
    a = logp_gpu[idx].contiguous()
    b = torch.from_numpy(np.asarray(oracle_logp, dtype=np.float32)).to(dev)
    m = torch.ones(a.numel(), dtype=torch.uint8, device=dev)
    diag, worst = rlk.rlk_dlogp_diagnostics(a, b, m, 0.2)
    d = dict(zip(rlk.DIAG_FIELDS, [float(x) for x in diag.cpu().tolist()]))
    err = float(np.max(np.abs(a.double().cpu().numpy() - np.asarray(oracle_logp))))
    return {"sample_tokens": int(a.numel()), "max_abs_dlogp_vs_oracle": err,
            "diagnostics": {k: (int(v) if k == "active" else float(f"{v:.4g}")) for k, v in d.items()},
            "worst_sample_row": int(rows[int(worst.item())]) if int(worst.item()) >= 0 else None}


def traffic_for(kernel_src_files, name):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/<name>.traffic.md), or
    None once the kernel's sources differ from the ones that were profiled."""
    path = os.path.join(ROOT, "profiles", f"{name}.traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep and k.strip() in ("source_sha256", "bytes_per_launch"):
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in kernel_src_files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("source_sha256") != h.hexdigest() or "bytes_per_launch" not in rec:
        return None
    return int(rec["bytes_per_launch"])


def upload(w, dev):
    import torch

    def mat(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    return (mat(w.h), mat(w.W), torch.from_numpy(w.targets).to(dev),
            torch.from_numpy(w.mask).to(dev), torch.from_numpy(w.adv).to(dev))


def bench_logits(args, w):
    """Log-prob from existing logits: bf16 logits [N, V] of the workload's shape, drawn on the
    device from a seeded generator (synthetic), resident before the timed region."""
    import torch
    import linear_selected_token_amd as rlk
    dev = torch.device("cuda", 0)
    N, V, T, Na = w.N, w.V, w.T, w.n_active
    g = torch.Generator(device=dev)
    g.manual_seed(1003)
    logits = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, N, 1024):
        logits[r0:r0 + 1024] = (torch.randn((min(1024, N - r0), V), generator=g, device=dev)
                                * 3.0).to(torch.bfloat16)
    targets = torch.from_numpy(w.targets).to(dev)
    mask = torch.from_numpy(w.mask).to(dev)
    ws = torch.empty(rlk.logits_workspace_bytes(N, V), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        rlk.rlk_logp_from_logits(logits, targets, mask, T, workspace=ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        rlk.rlk_logp_from_logits(logits, targets, mask, T, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # active logits rows once; mask, index and target reads; logp and lse written
    nbytes = Na * V * 2 + N + 4 * N + 4 * Na + 8 * N
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "active tokens/sec, log-prob from existing bf16 logits",
        "value": round(Na / (ms * 1e-3), 1), "unit": "active tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0, 3^2) logits rounded to bf16",
        "config": {"workload": args.workload, "mode": "logits", "N": N, "V": V, "T": T,
                   "n_active": Na, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "logits_logp_kernel<bf16>",
                     "timed": "the whole call per step (compaction + the kernel)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(LOGITS_SOURCES, "logits_logp_kernel"),
                     "algorithmic_bytes_per_step": nbytes},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_entropy(args, w):
    """A training step with an entropy bonus: the forward that also returns each token's
    entropy and the gradients of L = -sum_t mask_t (adv_t logp_t + c_t H_t) (c_t = 0.01), timed
    whole on the caller's stream.  The headline is the fused call
    (rlk_linear_logp_fwd_bwd_entropy); the two calls (the entropy forward, then the
    entropy-bonus backward) are timed beside it, their logp and entropy checked bit for bit
    against it, and so are the entropy forward alone and the plain forward (the entropy's
    overhead)."""
    import torch
    import linear_selected_token_amd as rlk
    dev = torch.device("cuda", 0)
    N, H, V, T, Na = w.N, w.H, w.V, w.T, w.n_active
    h, W, targets, mask, adv = upload(w, dev)
    dt = 0 if w.dtype == "bf16" else 1
    coef = torch.full((N,), 0.01, dtype=torch.float32, device=dev)
    ws_e = torch.empty(rlk.fwd_entropy_workspace_bytes(N, H, V, dt), dtype=torch.uint8,
                       device=dev)
    ws_p = torch.empty(rlk.fwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(rlk.bwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    res = {}

    def step():
        lp, lse, ent = rlk.rlk_linear_logp_fwd_entropy(h, W, targets, mask, T, workspace=ws_e)
        rlk.rlk_linear_logp_bwd_entropy(h, W, targets, mask, T, adv, coef, lse, ent,
                                        workspace=ws_b, dh=dh, dW=dW)
        res["two"] = (lp, ent)

    two_ms = timed(step)
    fwd_ms = timed(lambda: rlk.rlk_linear_logp_fwd_entropy(h, W, targets, mask, T,
                                                           workspace=ws_e))
    plain_ms = timed(lambda: rlk.rlk_linear_logp_fwd(h, W, targets, mask, T, workspace=ws_p))
    del ws_b
    ws_f = torch.empty(rlk.fwd_bwd_entropy_workspace_bytes(N, H, V, dt), dtype=torch.uint8,
                       device=dev)

    def fused_step():
        lp, _, ent, _, _ = rlk.rlk_linear_logp_fwd_bwd_entropy(h, W, targets, mask, T, adv, coef,
                                                               workspace=ws_f, dh=dh, dW=dW)
        res["fused"] = (lp, ent)

    ms = timed(fused_step)
    for a, b in zip(res["fused"], res["two"]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "fused and two-call differ"
    flop = 6.0 * Na * H * V   # forward, dL/dh, dL/dW, as executed by the fused call
    tf = flop / (ms * 1e-3) / 1e12
    out = {
        "metric": "active tokens/sec, fused linear logp fwd+bwd with an entropy bonus",
        "value": round(Na / (ms * 1e-3), 1), "unit": "active tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded h~N(0,1), W~N(0,1/H) rounded to bf16, packed "
                "prompt/response sequences",
        "config": {"workload": args.workload, "mode": "entropy", "N": N, "H": H, "V": V,
                   "T": T, "n_active": Na, "ent_coef": 0.01, "parallelism": "none (1 GPU)"},
        "timed": "rlk_linear_logp_fwd_bwd_entropy per step, on the current stream",
        "two_calls": {"ms": round(two_ms, 4), "active_tokens_per_s": round(Na / (two_ms * 1e-3), 1),
                      "calls": "rlk_linear_logp_fwd_entropy, rlk_linear_logp_bwd_entropy"},
        "workspace_bytes": ws_f.numel(),
        "fwd_entropy_ms": round(fwd_ms, 4),
        "plain_fwd_ms": round(plain_ms, 4),
        "entropy_fwd_overhead_frac": round(fwd_ms / plain_ms - 1.0, 4),
        # the whole step's executed flops over its time: a lower bound of every kernel's rate
        "roofline": {"bound": "mfma", "kernel": "whole step (fused entropy forward + "
                     "entropy-bonus gradients; 6 Na H V flops)", "achieved": round(tf, 2),
                     "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": flop,
                     "avg_launch_ms": round(ms, 4)},
    }
    if args.cpu_baseline_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, "entropy", args.cpu_baseline_seconds)[0]
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_ppo(args, w):
    """A PPO/GRPO-style step: the forward, the clipped policy-gradient loss with a KL penalty
    on the fresh log-prob (old and reference log-probs are seeded perturbations of it, made
    before the timed region), and the backward driven by the loss's -dloss/dlogp.  The headline
    runs it as one call (rlk_linear_ppo_fwd_bwd); the chain of three calls is timed beside it
    (their per-token outputs must agree bit for bit), and the loss fragment and the dlogp
    diagnostics alone."""
    import torch
    import linear_selected_token_amd as rlk
    dev = torch.device("cuda", 0)
    N, H, V, T, Na = w.N, w.H, w.V, w.T, w.n_active
    h, W, targets, mask, adv = upload(w, dev)
    dt = 0 if w.dtype == "bf16" else 1
    ws_f = torch.empty(rlk.fwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(rlk.bwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    logp0, _ = rlk.rlk_linear_logp_fwd(h, W, targets, mask, T, workspace=ws_f)
    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    old = logp0 + 0.05 * torch.randn(N, generator=g, device=dev)
    ref = logp0 + 0.05 * torch.randn(N, generator=g, device=dev)
    scale = 1.0 / max(Na, 1)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    res = {}

    def step():
        logp, lse = rlk.rlk_linear_logp_fwd(h, W, targets, mask, T, workspace=ws_f)
        loss, badv, _, _ = rlk.rlk_ratio_kl_loss(logp, old, ref, adv, mask, 0.2, 0.28, 0.01,
                                                 scale)
        rlk.rlk_linear_logp_bwd(h, W, targets, mask, T, badv, lse, workspace=ws_b, dh=dh, dW=dW)
        res["chain"] = (logp, loss, badv)

    chain_ms = timed(step)
    del ws_b
    ws_p = torch.empty(rlk.ppo_fwd_bwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)

    def fused_step():
        out = rlk.rlk_linear_ppo_fwd_bwd(h, W, targets, mask, T, old, ref, adv, 0.2, 0.28, 0.01,
                                         scale, workspace=ws_p, dh=dh, dW=dW)
        res["fused"] = (out[0], out[2], out[3])

    ms = timed(fused_step)
    for a, b in zip(res["fused"], res["chain"]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "fused and chained PPO differ"
    loss_ms = timed(lambda: rlk.rlk_ratio_kl_loss(logp0, old, ref, adv, mask, 0.2, 0.28, 0.01,
                                                  scale))
    diag_ms = timed(lambda: rlk.rlk_dlogp_diagnostics(logp0, old, mask, 0.2))
    flop = 6.0 * Na * H * V
    tf = flop / (ms * 1e-3) / 1e12
    loss_bytes = N * (4 * 4 + 1 + 4 * 2) + 32 * ((N + 1023) // 1024)
    out = {
        "metric": "active tokens/sec, fused linear logp fwd + clipped PG/KL loss + bwd",
        "value": round(Na / (ms * 1e-3), 1), "unit": "active tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded h~N(0,1), W~N(0,1/H) rounded to bf16, packed "
                "prompt/response sequences; old/ref log-probs = logp + N(0, 0.05^2)",
        "config": {"workload": args.workload, "mode": "ppo", "N": N, "H": H, "V": V, "T": T,
                   "n_active": Na, "eps_lo": 0.2, "eps_hi": 0.28, "beta": 0.01,
                   "parallelism": "none (1 GPU)"},
        "timed": "rlk_linear_ppo_fwd_bwd per step (forward, loss fragment per token block, "
                 "gradients), on the current stream",
        "chain_of_calls": {"ms": round(chain_ms, 4),
                           "active_tokens_per_s": round(Na / (chain_ms * 1e-3), 1),
                           "calls": "rlk_linear_logp_fwd, rlk_ratio_kl_loss, rlk_linear_logp_bwd"},
        "workspace_bytes": ws_p.numel(),
        "loss_fragment": {"ms": round(loss_ms, 5), "bytes": loss_bytes,
                          "gbs": round(loss_bytes / (loss_ms * 1e-3) / 1e9, 1)},
        "diagnostics_ms": round(diag_ms, 5),
        "roofline": {"bound": "mfma", "kernel": "whole step (forward + loss fragment + "
                     "backward; 6 Na H V flops)", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": flop,
                     "avg_launch_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_kl(args, w):
    """Distillation step: forward and reverse full-vocabulary KL between the workload's student
    head and a teacher head of the same shape (seeded N(0,1) hidden states, N(0,1/H) weights,
    drawn on the device, bf16), then the backward of the forward KL into the student."""
    import torch
    import linear_selected_token_amd as rlk
    dev = torch.device("cuda", 0)
    N, H, V, T, Na = w.N, w.H, w.V, w.T, w.n_active
    h, W, _, mask, _ = upload(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1011)
    ht = torch.randn((N, H), generator=g, device=dev).to(torch.bfloat16)
    Wt = torch.empty((V, H), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, V, 8192):
        r1 = min(V, r0 + 8192)
        Wt[r0:r1] = (torch.randn((r1 - r0, H), generator=g, device=dev) / H ** 0.5).to(
            torch.bfloat16)
    coef = torch.full((N,), 1.0 / max(Na, 1), dtype=torch.float32, device=dev)
    import ctypes
    nb = ctypes.c_size_t(0)
    rlk.lib().rlk_linear_kl_fwd_workspace_size(N, H, H, V, 0, ctypes.byref(nb))
    ws_f = torch.empty(int(nb.value), dtype=torch.uint8, device=dev)
    rlk.lib().rlk_linear_kl_bwd_workspace_size(N, H, H, V, 0, ctypes.byref(nb))
    ws_b = torch.empty(int(nb.value), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def fwd():
        return rlk.rlk_linear_kl_fwd(h, W, ht, Wt, mask, T, workspace=ws_f)

    def step():
        _, kr, ls, lt = fwd()
        rlk.rlk_linear_kl_bwd(h, W, ht, Wt, mask, T, coef, None, ls, lt, kr, workspace=ws_b)

    ms = timed(step)
    fwd_ms = timed(fwd)
    flop = 12.0 * Na * H * V   # 2 heads forward + 2 heads recomputed + dL/dh + dL/dW
    tf = flop / (ms * 1e-3) / 1e12
    out = {
        "metric": "active tokens/sec, full-vocabulary KL to a teacher head, fwd + bwd",
        "value": round(Na / (ms * 1e-3), 1), "unit": "active tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: the workload's student head; teacher h~N(0,1), W~N(0,1/H) drawn "
                "on the device, bf16",
        "config": {"workload": args.workload, "mode": "kl", "N": N, "H_s": H, "H_t": H, "V": V,
                   "T": T, "n_active": Na, "parallelism": "none (1 GPU)"},
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(4.0 * Na * H * V / (fwd_ms * 1e-3) / 1e12, 2),
        "workspace_bytes": {"fwd": int(ws_f.numel()), "bwd": int(ws_b.numel())},
        "roofline": {"bound": "mfma", "kernel": "whole step (the two-head tile kernel over the "
                     "vocabulary, again per chunk for dL/dz, dL/dh, dL/dW)", "achieved": round(tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flop_per_launch": flop, "avg_launch_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_gemm_reference(args, w):
    """The library GEMM (torch.matmul, hipBLASLt on ROCm) of the tile kernel's shape: the
    active tokens' h [Na, H] times W^T [H, V] into bf16 logits [Na, V].  It does none of the
    softmax work and writes the logits the fused path never forms; a reference point for
    what the matrix cores sustain on this shape."""
    import torch
    dev = torch.device("cuda", 0)
    N, H, V, Na = w.N, w.H, w.V, w.n_active
    h, W, _, mask, _ = upload(w, dev)
    ha = h[torch.from_numpy(np.nonzero(w.mask)[0]).to(dev)].contiguous()
    out = torch.empty((Na, V), dtype=h.dtype, device=dev)
    Wt = W.t()

    for _ in range(args.warmup):
        torch.matmul(ha, Wt, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        torch.matmul(ha, Wt, out=out)
        e1.record()
    torch.cuda.synchronize()
    ts = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms = float(np.mean(ts))
    flop = 2.0 * Na * H * V
    tf = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TFLOP/s, library bf16 GEMM of the forward tile kernel's shape (reference)",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "step_ms_min": round(float(np.min(ts)), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "mode": "gemm-reference", "M": Na, "K": H,
                   "N": V, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "library GEMM (torch.matmul)",
                     "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flop_per_launch": flop, "avg_launch_ms": round(ms, 4)},
        "cpu_baseline": None}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the path has no "
                                   "multi-GPU mode (run with --gpus 1)"}))
        sys.exit(2)
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    import torch
    import linear_selected_token_amd as rlk

    dev = torch.device("cuda", 0)
    w = make_workload(args.workload)
    if args.mode == "logits":
        bench_logits(args, w)
        return
    if args.mode == "entropy":
        bench_entropy(args, w)
        return
    if args.mode == "ppo":
        bench_ppo(args, w)
        return
    if args.mode == "kl":
        bench_kl(args, w)
        return
    if args.mode == "gemm-reference":
        bench_gemm_reference(args, w)
        return
    m = measure(w, dev, args.steps, args.warmup, args.mode == "fwdbwd")
    N, H, V, T, Na = w.N, w.H, w.V, w.T, w.n_active
    head = m["fused"] if "fused" in m else m
    out = {
        "metric": METRIC,
        "value": round(Na / (head["ms"] * 1e-3), 1),
        "unit": "active tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "step_ms_median": head["step_ms_median"],
        "step_ms_min": head["step_ms_min"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded h~N(0,1), W~N(0,1/H) rounded to bf16, packed "
                "prompt/response sequences",
        "config": {"workload": args.workload, "mode": args.mode, "N": N, "H": H, "V": V,
                   "T": T, "n_active": Na, "parallelism": "none (1 GPU)"},
        "timed": ("rlk_linear_logp_fwd_bwd per step (forward and backward in one call), on the "
                  "current stream" if "fused" in m else
                  "rlk_linear_logp_fwd per step, on the current stream"),
        "fwd": m["fwd"],
        "roofline": m["roofline"],
    }
    if "fused" in m:
        out["fwd_bwd_tflops_executed"] = m["fused"]["tflops_executed"]
        out["fwd_bwd_mfma_frac"] = m["fused"]["mfma_frac"]
        out["fwd_bwd_frac_over_8NaHV"] = m["fused"]["frac_over_8NaHV"]
        out["bwd_added_ms"] = m["fused"]["bwd_added_ms"]
        if "one_block" in m["fused"]:
            # not the headline: the default workspace (under 1e9 bytes) is
            out["fused_one_block_workspace"] = m["fused"]["one_block"]
        out["two_calls"] = m["two_calls"]
    if "workspace_bytes" in m:
        out["workspace_bytes"] = m["workspace_bytes"]
    logp = m.pop("_logp")
    del m
    if args.cpu_baseline_seconds > 0:
        out["cpu_baseline"], rows, olp = cpu_baseline(w, args.mode, args.cpu_baseline_seconds)
        out["gpu_over_cpu_baseline"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
        out["parity"] = sample_parity(logp, rows, olp)
    else:
        out["cpu_baseline"] = None
    del logp
    if args.configs and args.workload == DEFAULT_WORKLOAD and args.mode == "fwdbwd":
        out["configs"] = bench_configs(args, dev)
    print(json.dumps(out), flush=True)


def measure(w, dev, steps, warmup, do_bwd):
    """Time the public entry points on one workload.

    A step is rlk_linear_logp_fwd (compaction, tile kernel, merge) and, if do_bwd,
    rlk_linear_logp_bwd, enqueued on the current stream; HIP events bracket the forward and
    the backward of every step and the whole timed region.  With do_bwd the fused call
    rlk_linear_logp_fwd_bwd is timed the same way in a loop of its own (its logp must carry
    the forward's bits).  The tile kernel alone is timed in a further loop that calls the
    forward's three stages as separate entry points, with events on the stream the tile
    kernel runs on (the roofline's launch duration)."""
    import torch
    import linear_selected_token_amd as rlk
    N, H, V, T, Na = w.N, w.H, w.V, w.T, w.n_active
    dt = 0 if w.dtype == "bf16" else 1
    h, W, targets, mask, adv = upload(w, dev)
    fws = torch.empty(rlk.fwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
    ws_bytes = {"fwd": fws.numel()}
    if do_bwd:
        bws = torch.empty(rlk.bwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device=dev)
        dh = torch.empty((N, H), dtype=torch.float32, device=dev)
        dW = torch.empty((V, H), dtype=torch.float32, device=dev)
        ws_bytes["bwd"] = bws.numel()
    res = {}

    def step(ev):
        ev[0].record()
        logp, lse = rlk.rlk_linear_logp_fwd(h, W, targets, mask, T, workspace=fws)
        ev[1].record()
        if do_bwd:
            rlk.rlk_linear_logp_bwd(h, W, targets, mask, T, adv, lse, workspace=bws, dh=dh, dW=dW)
        ev[2].record()
        res["logp"] = logp

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    for _ in range(warmup):
        step(events(3))
    torch.cuda.synchronize()
    evs = [events(3) for _ in range(steps)]
    t0, t1 = events(2)
    torch.cuda.synchronize()
    t0.record()
    for ev in evs:
        step(ev)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if do_bwd else 0.0

    # the tile kernel alone: the forward's stages as separate calls
    bufs = rlk.ForwardBuffers(N, V, dev)

    def stages(ev):
        rlk.rlk_compact_active(mask, bufs.idx, bufs.n_active, bufs.target_logit, bufs.logp,
                               bufs.lse)
        ev[0].record()
        rlk.rlk_linear_logp_partials(h, W, targets, bufs.idx, bufs.n_active, T, bufs.part_max,
                                     bufs.part_sum, bufs.target_logit)
        ev[1].record()
        rlk.rlk_linear_logp_merge(bufs.part_max, bufs.part_sum, bufs.target_logit, bufs.idx,
                                  bufs.n_active, N, V, bufs.logp, bufs.lse)

    for _ in range(warmup):
        stages(events(2))
    tevs = [events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    for ev in tevs:
        stages(ev)
    torch.cuda.synchronize()
    tile_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in tevs]))
    assert torch.equal(bufs.logp[:N], res["logp"]), "stage calls and rlk_linear_logp_fwd differ"
    del bufs

    fused = None
    if do_bwd:
        # the fused call: forward and backward in one, no second logits GEMM
        del bws
        xws = torch.empty(rlk.fwd_bwd_workspace_bytes(N, H, V, dt), dtype=torch.uint8,
                          device=dev)
        ws_bytes["fwd_bwd"] = xws.numel()

        def fstep(ev):
            ev[0].record()
            logp, _, _, _ = rlk.rlk_linear_logp_fwd_bwd(h, W, targets, mask, T, adv,
                                                        workspace=xws, dh=dh, dW=dW)
            ev[1].record()
            res["flogp"] = logp

        for _ in range(warmup):
            fstep(events(2))
        torch.cuda.synchronize()
        fevs = [events(2) for _ in range(steps)]
        f0, f1 = events(2)
        torch.cuda.synchronize()
        f0.record()
        for ev in fevs:
            fstep(ev)
        f1.record()
        torch.cuda.synchronize()
        fms = f0.elapsed_time(f1) / steps
        fstep_ms = [e[0].elapsed_time(e[1]) for e in fevs]
        assert torch.equal(res["flogp"], res["logp"]), "fused and two-call logp differ"
        del xws
        fused = {"ms": fms, "step_ms_median": round(float(np.median(fstep_ms)), 4),
                 "step_ms_min": round(float(np.min(fstep_ms)), 4)}
        # the same call with a workspace that holds every active token in one block
        nb = rlk.fwd_bwd_workspace_bytes_for_block(N, H, V, dt, Na)
        if nb > ws_bytes["fwd_bwd"]:
            xws = torch.empty(nb, dtype=torch.uint8, device=dev)
            for _ in range(warmup):
                fstep(events(2))
            torch.cuda.synchronize()
            f0, f1 = events(2)
            f0.record()
            for ev in fevs:
                fstep(ev)
            f1.record()
            torch.cuda.synchronize()
            assert torch.equal(res["flogp"], res["logp"]), "one-block and two-call logp differ"
            oms = f0.elapsed_time(f1) / steps
            fused["one_block"] = {"ms": round(oms, 4),
                                  "active_tokens_per_s": round(Na / (oms * 1e-3), 1),
                                  "workspace_bytes": nb}
            del xws

    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    fwd_flop = 2.0 * Na * H * V
    bwd_flop = 6.0 * Na * H * V   # recompute + dL/dh + dL/dW, as executed
    tile_tflops = fwd_flop / (tile_ms * 1e-3) / 1e12
    srcs = FWD_TILE_SOURCES
    roofline = {"bound": "mfma", "kernel": f"fwd_tiles_kernel<{'bf16' if bf16 else 'fp32'}>",
                "achieved": round(tile_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tile_tflops / peak, 4),
                "traffic": traffic_for(srcs, "fwd_tiles_kernel") if bf16 and w.spec.seed == 1003
                else None,
                "algorithmic_flop_per_launch": fwd_flop, "avg_launch_ms": round(tile_ms, 4)}
    m = {"ms": ms, "step_ms_median": round(float(np.median(step_ms)), 4),
         "step_ms_min": round(float(np.min(step_ms)), 4),
         "fwd": {"ms": round(fwd_ms, 4), "active_tokens_per_s": round(Na / (fwd_ms * 1e-3), 1),
                 "tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
                 "mfma_frac": round(fwd_flop / (fwd_ms * 1e-3) / 1e12 / peak, 4)},
         "roofline": roofline, "workspace_bytes": ws_bytes, "_logp": res["logp"]}
    if do_bwd:
        # the two calls: 8 H V flops per active token (the backward runs the logits GEMM again)
        m["two_calls"] = {
            "ms": round(ms, 4), "active_tokens_per_s": round(Na / (ms * 1e-3), 1),
            "step_ms_median": m["step_ms_median"], "step_ms_min": m["step_ms_min"],
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "bwd_tflops_executed": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_mfma_frac": round(bwd_flop / (bwd_ms * 1e-3) / 1e12 / peak, 4),
            "tflops_executed": round((fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round((fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12 / peak, 4)}
        # the fused call: 6 H V flops per active token (forward, dL/dh, dL/dW)
        fflop = 6.0 * Na * H * V
        fused["tflops_executed"] = round(fflop / (fused["ms"] * 1e-3) / 1e12, 2)
        fused["mfma_frac"] = round(fflop / (fused["ms"] * 1e-3) / 1e12 / peak, 4)
        # the same job counted as the recompute formulation's 8 H V flops per active token (what
        # the two calls execute): a rate for comparing the two forms, not flops executed here
        fused["frac_over_8NaHV"] = round(fwd_flop * 4 / (fused["ms"] * 1e-3) / 1e12 / peak, 4)
        # what the backward adds to a forward alone (fused step minus the forward call)
        fused["bwd_added_ms"] = round(fused["ms"] - fwd_ms, 4)
        m["fused"] = fused
    return m


def config_parity(w, logp, k=32, seed=7):
    """max |dlogp| of the GPU logp against the oracle on k sampled active tokens (all of them
    when there are at most k)."""
    import oracle
    import workloads as wl
    act = np.nonzero(w.mask)[0]
    rows = act if act.size <= k else np.sort(np.random.default_rng(seed).choice(act, k, False))
    olp, _ = oracle.linear_logp(wl.as_f64(w.h[rows]), wl.as_f64(w.W), w.targets[rows],
                                np.ones(rows.size, np.uint8), w.T)
    got = logp[rows].astype(np.float64)
    return {"rows": int(rows.size), "max_abs_dlogp_vs_oracle": float(np.max(np.abs(got - olp)))}


def bench_configs(args, dev):
    """The other workloads, each timed the same way as the headline (forward + backward for
    bf16 heads, forward only for the fp32 one), with the oracle's logp on sampled tokens."""
    import torch
    out = {}
    for name, (cfg, _) in sorted(WORKLOADS.items(), key=lambda kv: kv[1][0]):
        if name == DEFAULT_WORKLOAD:
            continue
        t0 = time.perf_counter()
        w = make_workload(name)
        do_bwd = w.dtype == "bf16"
        m = measure(w, dev, args.steps, args.warmup, do_bwd)
        Na = w.n_active
        rec = {"config": cfg, "workload": name, "N": w.N, "H": w.H, "V": w.V, "T": w.T,
               "dtype": w.dtype, "n_active": Na,
               "fwd_ms": m["fwd"]["ms"], "fwd_active_tokens_per_s": m["fwd"]["active_tokens_per_s"],
               "fwd_tflops": m["fwd"]["tflops"], "fwd_mfma_frac": m["fwd"]["mfma_frac"],
               "tile_kernel_ms": m["roofline"]["avg_launch_ms"],
               "tile_kernel_frac": m["roofline"]["frac"], "peak_tflops": m["roofline"]["peak"],
               "workspace_bytes": m["workspace_bytes"]}
        if do_bwd:
            f = m["fused"]
            rec.update({"fwd_bwd_ms": round(f["ms"], 4),
                        "fwd_bwd_active_tokens_per_s": round(Na / (f["ms"] * 1e-3), 1),
                        "fwd_bwd_mfma_frac": f["mfma_frac"],
                        "fwd_bwd_frac_over_8NaHV": f["frac_over_8NaHV"],
                        "bwd_added_ms": f["bwd_added_ms"],
                        "fused_one_block_workspace": f.get("one_block"),
                        "two_calls": {k: m["two_calls"][k] for k in
                                      ("ms", "active_tokens_per_s", "bwd_ms", "bwd_mfma_frac",
                                       "mfma_frac")}})
        logp = m.pop("_logp").cpu().numpy()
        del m
        torch.cuda.empty_cache()
        rec["parity"] = config_parity(w, logp)
        rec["wall_s"] = round(time.perf_counter() - t0, 1)
        out[str(cfg)] = rec
        print(f"# config {cfg} ({name}) done in {rec['wall_s']} s", file=sys.stderr, flush=True)
    return out


if __name__ == "__main__":
    main()
