"""The fused forward + backward, the fused PPO step and the KL forward captured in a HIP graph
(torch.cuda.CUDAGraph around the bindings): every replay gives the eager call's bits (needs an
MI355X).

The library never allocates, synchronizes with the host or clears memory with hipMemsetAsync
(fill kernels do it), and its launch sequence depends only on the shapes, so a captured step
replays as it ran.  Each replay runs after eager work that overwrites the outputs with NaN, and
is checked on its own."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import flush, upload

pytestmark = pytest.mark.gpu

SPEC = wl.scaled_spec(5, N=3200, H=256, V=1000, n_seq=8, len_lo=200, len_hi=600, seed=181, T=0.8)


def _capture(fn):
    """fn() captured in a graph after a warm-up call on a side stream; returns (graph, outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _replays_match(g, out, eager, names, reps=3):
    for rep in range(reps):
        for o in out:
            if o.is_floating_point():
                o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, out, eager):
            assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes(), (rep, name)
    flush(f"  {reps} replays, each bit-identical to the eager call: {', '.join(names)}")


def test_fused_step_graph_replays():
    import linear_selected_token_amd as rlk
    w = wl.make(SPEC)
    d = upload(w)
    # 1024-token blocks: several blocks, so the capture holds the whole block loop
    nb = rlk.fwd_bwd_workspace_bytes_for_block(w.N, w.H, w.V, 0, 1024)
    ws = torch.empty(nb, dtype=torch.uint8, device=d["h"].device)

    def step():
        return rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                           d["adv"], workspace=ws)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, out = _capture(step)
    _replays_match(g, out, eager, ("logp", "lse", "dh", "dW"))


def test_fused_ppo_step_graph_replays():
    import linear_selected_token_amd as rlk
    w = wl.make(SPEC)
    d = upload(w)
    dev = d["h"].device
    r = np.random.default_rng(182)
    logp, _ = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    old = logp + torch.from_numpy(r.normal(0, 0.2, w.N).astype(np.float32)).to(dev)
    ref = logp + torch.from_numpy(r.normal(0, 0.2, w.N).astype(np.float32)).to(dev)
    ws = torch.empty(rlk.ppo_fwd_bwd_workspace_bytes(w.N, w.H, w.V, 0), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / int(w.mask.sum())

    def step():
        return rlk.rlk_linear_ppo_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, old, ref,
                                          d["adv"], 0.2, 0.2, 0.05, scale, workspace=ws)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, out = _capture(step)
    _replays_match(g, out, eager, ("logp", "lse", "loss", "bwd_adv", "ratio", "sums", "dh", "dW"))


def test_kl_forward_graph_replays():
    import linear_selected_token_amd as rlk
    w = wl.make(SPEC)
    d = upload(w)
    dev = d["h"].device
    g0 = torch.Generator(device=dev)
    g0.manual_seed(183)
    ht = torch.randn((w.N, 128), generator=g0, device=dev).to(torch.bfloat16)
    Wt = (torch.randn((w.V, 128), generator=g0, device=dev) / 128 ** 0.5).to(torch.bfloat16)
    ws = torch.empty(rlk.kl_fwd_workspace_bytes(w.N, w.H, 128, w.V, 0, 1024), dtype=torch.uint8,
                     device=dev)

    def step():
        return rlk.rlk_linear_kl_fwd(d["h"], d["W"], ht, Wt, d["mask"], w.T, workspace=ws,
                                     block_tokens=1024)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, out = _capture(step)
    _replays_match(g, out, eager, ("kl_fwd", "kl_rev", "lse_s", "lse_t"))
