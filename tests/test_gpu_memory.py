"""Peak device memory of the fused path: the method exists to avoid the [N, V] logits, so the
memory a forward + backward adds beyond its inputs and outputs (the workspaces) must stay far
below those logits (RL-Kernel Roadmap (2026), P0.2, "Fused CE LogProb without materializing
logits"; the operator backlog's proactive workspace sizing).  Needs an MI355X."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import flush, upload

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_benchmark_step_peak_memory():
    import linear_selected_token_amd as rlk
    flush("qwen3-8b-head N=16384 T=0.7: generating inputs")
    targets = np.load(os.path.join(HERE, "golden", "cfg3_sampled_targets.npy"))
    w = wl.with_targets(wl.make(3), targets)
    d = upload(w)
    N, H, V = w.N, w.H, w.V
    dev = d["h"].device
    # outputs the caller owns in any case: dh and dW (fp32), logp and lse
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, d["adv"], lse, dh=dh,
                            dW=dW)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated(dev) - base
    logits_all = N * V * 2                 # bf16 logits of every token
    logits_active = w.n_active * V * 2     # ... of the active tokens only
    flush(f"  peak beyond inputs and outputs: {extra / 1e9:.3f} GB; bf16 logits would take "
          f"{logits_all / 1e9:.2f} GB ({logits_active / 1e9:.2f} GB for the {w.n_active} active "
          f"tokens)")
    assert extra <= 0.25 * logits_all
    assert extra <= 0.4 * logits_active
    assert torch.isfinite(logp).all()
