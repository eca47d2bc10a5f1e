"""Forward parity of the HIP path against the float64 oracle (needs an MI355X).

Small shapes are compared in full (several vocabulary tiles, ragged tails, masked
prompts); the full-size workloads are compared on sampled active rows that the oracle
scores one by one."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (MAX_ABS_DLOGP, bits, flush, oracle_inputs, run_fwd, sample_rows,
                      upload)

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

SMALL = wl.scaled_spec(2, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=77)


def _compare(w, lp, lse, rows=None, tol=MAX_ABS_DLOGP):
    h64, W64 = oracle_inputs(w)
    if rows is None:
        olp, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
        act = w.mask.astype(bool)
        assert np.all(lp[~act] == 0) and np.all(lse[~act] == 0)
        d = np.abs(lp[act] - olp[act])
        dl = np.abs(lse[act] - olse[act])
    else:
        olp, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T, rows=rows)
        d = np.abs(lp[rows] - olp)
        dl = np.abs(lse[rows] - olse)
    flush(f"  {w.spec.name}: max_abs_dlogp={d.max():.3e} mean={d.mean():.3e} "
          f"max_abs_dlse={dl.max():.3e} over {d.size} active tokens")
    assert np.all(np.isfinite(lp[w.mask.astype(bool)]))
    assert d.max() <= tol
    assert dl.max() <= tol
    return d.max()


def _sweep_specs(n, seed):
    """Seeded forward shapes: N in [1, 2000], H a multiple of 64 in [64, 1024], V in [1, 70000]
    (log-uniform), bf16 or fp32, T in [0.3, 2]."""
    r = np.random.default_rng(seed)
    out = []
    for k in range(n):
        N = int(r.integers(1, 2001))
        V = int(np.exp(r.uniform(0.0, np.log(70000.0)))) + 1
        out.append(wl.scaled_spec(2, N=N, H=64 * int(r.integers(1, 17)), V=V,
                                  dtype=str(r.choice(["bf16", "fp32"])),
                                  n_seq=int(min(N, r.integers(1, 5))), len_lo=1, len_hi=N,
                                  seed=800 + k, T=float(r.uniform(0.3, 2.0))))
    return out


@pytest.mark.parametrize("spec", _sweep_specs(16, 311),
                         ids=lambda s: f"N{s.N}-H{s.H}-V{s.V}-{s.dtype}")
def test_random_shapes_sweep(spec):
    # logp and lse of every active token against the oracle, and the entropy forward's logp and
    # lse bit-identical to the plain forward's
    import linear_selected_token_amd as rlk
    w = wl.make(spec)
    d = upload(w)
    lp, lse = run_fwd(w, d)
    _compare(w, lp, lse)
    lp2, lse2, _ = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    torch.cuda.synchronize()
    assert np.array_equal(bits(lp2.cpu().numpy()), bits(lp))
    assert np.array_equal(bits(lse2.cpu().numpy()), bits(lse))


def test_device_is_gfx950():
    import linear_selected_token_amd as rlk
    props = torch.cuda.get_device_properties(0)
    flush(f"device {props.name} {getattr(props, 'gcnArchName', '?')} CUs={props.multi_processor_count}")
    flush(rlk.build_info())
    assert "gfx950" in getattr(props, "gcnArchName", "gfx950")


def test_config1_fp32_full():
    w = wl.make(1)
    lp, lse = run_fwd(w)
    assert _compare(w, lp, lse) < 1e-5


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_small_bf16_full(T):
    w = wl.make(wl.scaled_spec(2, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=77, T=T))
    lp, lse = run_fwd(w)
    _compare(w, lp, lse)


def test_small_fp32_full():
    w = wl.make(wl.scaled_spec(1, N=300, H=128, V=777, n_seq=3, len_lo=50, len_hi=150,
                               prompt="floor_half", seed=78, T=0.8))
    lp, lse = run_fwd(w)
    _compare(w, lp, lse, tol=1e-4)


def test_multi_tile_tokens_ragged():
    # 1100 active-heavy tokens: five token tiles, the last one ragged; V with a ragged
    # 128-column tail and a last 256-tile that is more than half empty
    w = wl.make(wl.scaled_spec(2, N=1100, H=256, V=2*256*3 + 100, n_seq=5, len_lo=100,
                               len_hi=400, prompt="none", seed=79))
    lp, lse = run_fwd(w)
    _compare(w, lp, lse)


def test_all_masked_and_empty():
    import linear_selected_token_amd as rlk
    w = wl.make(SMALL)
    d = upload(w)
    d["mask"].zero_()
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], 1.0)
    torch.cuda.synchronize()
    assert not logp.any() and not lse.any()
    e = torch.empty((0, 512), dtype=torch.bfloat16, device=d["h"].device)
    lp0, _ = rlk.rlk_linear_logp_fwd(e, d["W"], d["targets"][:0], d["mask"][:0], 1.0)
    assert lp0.numel() == 0


def test_single_token_and_tiny_vocab():
    for V in (1, 2, 3, 129):
        spec = wl.scaled_spec(2, N=1, H=64, V=V, n_seq=1, len_lo=1, len_hi=1, prompt="none",
                              seed=80 + V)
        w = wl.make(spec)
        lp, lse = run_fwd(w)
        _compare(w, lp, lse)
        if V == 1:
            assert abs(lp[0]) < 1e-6


def test_zero_weight_closed_form():
    w = wl.make(SMALL)
    w.W[:] = 0
    lp, lse = run_fwd(w)
    act = w.mask.astype(bool)
    assert np.abs(lp[act] + math.log(3000)).max() < 1e-6
    assert np.abs(lse[act] - math.log(3000)).max() < 1e-6


def test_targets_on_tile_boundaries():
    w = wl.make(SMALL)
    act = np.nonzero(w.mask)[0]
    edges = [0, 1, 127, 128, 129, 255, 256, 257, 2943, 2944, 2999]
    for k, t in enumerate(act[:len(edges) * 5]):
        w.targets[t] = edges[k % len(edges)]
    lp, lse = run_fwd(w)
    _compare(w, lp, lse)


def test_out_of_range_target_gives_nan():
    w = wl.make(SMALL)
    lp_ok, lse_ok = run_fwd(w)
    act = np.nonzero(w.mask)[0]
    bad = [int(act[3]), int(act[10])]
    w.targets[bad[0]] = 3000
    w.targets[bad[1]] = -5
    lp, lse = run_fwd(w)
    assert np.all(np.isnan(lp[bad]))
    assert np.array_equal(bits(lse), bits(lse_ok))
    keep = np.setdiff1d(np.arange(w.N), bad)
    assert np.array_equal(bits(lp[keep]), bits(lp_ok[keep]))


def test_large_logits():
    w = wl.make(SMALL)
    w.h = wl.bf16_bits(wl.bf16_to_f32(w.h) * np.float32(24.0))
    lp, lse = run_fwd(w)
    _compare(w, lp, lse)


def test_autograd_function_forward():
    import linear_selected_token_amd as rlk
    w = wl.make(SMALL)
    d = upload(w)
    lp = rlk.linear_logp(d["h"], d["W"], d["targets"], d["mask"], w.T)
    ref, _ = run_fwd(w, d)
    assert np.array_equal(bits(lp.detach().cpu().numpy()), bits(ref))


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_sampled(cfg):
    flush(f"config {cfg}: generating inputs")
    w = wl.make(cfg)
    lp, lse = run_fwd(w)
    rows = sample_rows(w, 48, seed=cfg)
    _compare(w, lp, lse, rows=rows)


def test_config3_sampled_targets():
    path = os.path.join(HERE, "golden", "cfg3_sampled_targets.npy")
    targets = np.load(path)
    w = wl.with_targets(wl.make(3), targets)
    lp, lse = run_fwd(w)
    rows = sample_rows(w, 48, seed=3)
    _compare(w, lp, lse, rows=rows)
