"""Loss fragments and dlogp diagnostics against the float64 oracle (needs an MI355X).

rlk_ratio_kl_loss: per-token loss, -dloss/dlogp and ratio within fp32 rounding of the
oracle (rtol 2e-6 plus an absolute 1e-6 of the token's scale); the clipped count exact on
inputs kept 1e-4 away from the clip edges (the decision is taken in fp32 on the GPU and in
fp64 by the oracle); per-token values bit-identical in another batch, the sums bit-identical
run to run.  Chained into rlk_linear_logp_bwd, it gives the loss's gradient within the
backward's rel-L2 gate.

rlk_dlogp_diagnostics: order statistics, maximum and worst token exact (dlogp is exact in
fp64 on both sides); means within 1e-12 relative (approx_kl0 within 1e-8: its terms are
differences of fp64 exponentials of small arguments)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.rl_loss as orl
import workloads as wl
from gpu_util import (assert_rows, assert_tiles, bits, device, flush, oracle_inputs,
                      upload)

pytestmark = pytest.mark.gpu


def _loss_inputs(seed, N, eps_lo, eps_hi, spread=0.3):
    r = np.random.default_rng(seed)
    logp = (-r.exponential(2.0, N)).astype(np.float32)
    old = (logp + r.normal(0, spread, N)).astype(np.float32)
    ref = (logp + r.normal(0, spread, N)).astype(np.float32)
    adv = r.normal(0, 1, N).astype(np.float32)
    mask = (r.random(N) < 0.75).astype(np.uint8)
    # keep every ratio away from the clip edges, where fp32 and fp64 may decide differently
    ratio = np.exp(logp.astype(np.float64) - old)
    near = (np.abs(ratio - (1 - eps_lo)) < 1e-4) | (np.abs(ratio - (1 + eps_hi)) < 1e-4)
    old[near] = logp[near]
    return logp, old, ref, adv, mask


def _gpu_loss(logp, old, ref, adv, mask, eps_lo, eps_hi, beta, scale):
    import linear_selected_token_amd as rlk
    dev = device()
    t = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    loss, badv, ratio, sums = rlk.rlk_ratio_kl_loss(
        t(logp), t(old), None if ref is None else t(ref), t(adv), t(mask), eps_lo, eps_hi, beta,
        scale, want_ratio=True)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), badv.cpu().numpy(), ratio.cpu().numpy(), sums.cpu().numpy()


@pytest.mark.parametrize("N,with_ref,beta", [(5000, True, 0.05), (1, True, 0.1),
                                              (3072, False, 0.0), (1025, True, 0.0)])
def test_loss_matches_oracle(N, with_ref, beta):
    eps_lo, eps_hi, scale = 0.2, 0.28, 1.0 / max(N, 1)
    logp, old, ref, adv, mask = _loss_inputs(N, N, eps_lo, eps_hi)
    if N == 1:
        mask[:] = 1
    ref_in = ref if with_ref else None
    loss, badv, ratio, sums = _gpu_loss(logp, old, ref_in, adv, mask, eps_lo, eps_hi, beta, scale)
    ol, og, orat, ocl, osums = orl.ratio_kl_loss(logp, old, ref_in, adv, mask, eps_lo, eps_hi,
                                                 beta, scale)
    tol = 1e-6 * scale
    el = np.abs(loss - ol).max()
    eg = np.abs(badv + og).max()
    flush(f"  ratio_kl N={N} ref={with_ref} beta={beta}: max|dloss|={el:.2e} "
          f"max|dgrad|={eg:.2e} clipped={sums[1]:.0f}/{osums['clipped']:.0f}")
    np.testing.assert_allclose(loss, ol, rtol=2e-6, atol=tol)
    np.testing.assert_allclose(badv, -og, rtol=2e-6, atol=tol)
    np.testing.assert_allclose(ratio, orat, rtol=2e-6, atol=0)
    m = mask.astype(bool)
    assert not loss[~m].any() and not badv[~m].any() and not ratio[~m].any()
    assert sums[1] == osums["clipped"] and sums[3] == osums["active"]
    assert abs(sums[0] - osums["loss"]) <= 1e-5 * max(1e-30, np.abs(ol).sum())
    assert abs(sums[2] - osums["kl"]) <= 1e-5 * max(1e-30, abs(osums["kl"]))


def test_loss_batch_invariance_and_determinism():
    N = 7000
    eps_lo, eps_hi, beta, scale = 0.2, 0.2, 0.1, 1e-3
    logp, old, ref, adv, mask = _loss_inputs(3, N, eps_lo, eps_hi)
    loss, badv, ratio, sums = _gpu_loss(logp, old, ref, adv, mask, eps_lo, eps_hi, beta, scale)
    _, _, _, sums2 = _gpu_loss(logp, old, ref, adv, mask, eps_lo, eps_hi, beta, scale)
    assert np.array_equal(sums.view(np.int64), sums2.view(np.int64))
    sel = np.arange(N - 1, 0, -7)
    sl, sb, sr, _ = _gpu_loss(*(np.ascontiguousarray(x[sel]) for x in (logp, old, ref, adv, mask)),
                              eps_lo, eps_hi, beta, scale)
    assert np.array_equal(bits(sl), bits(loss[sel]))
    assert np.array_equal(bits(sb), bits(badv[sel]))
    assert np.array_equal(bits(sr), bits(ratio[sel]))


def test_loss_empty_and_all_masked():
    import linear_selected_token_amd as rlk
    dev = device()
    z = torch.zeros(0, dtype=torch.float32, device=dev)
    _, _, _, sums = rlk.rlk_ratio_kl_loss(z, z, None, z, torch.zeros(0, dtype=torch.uint8,
                                                                      device=dev), 0.2, 0.2)
    assert not sums.cpu().numpy().any()
    logp, old, ref, adv, mask = _loss_inputs(4, 300, 0.2, 0.2)
    loss, badv, _, sums = _gpu_loss(logp, old, ref, adv, np.zeros_like(mask), 0.2, 0.2, 0.1, 1.0)
    assert not loss.any() and not badv.any() and not sums.any()


def test_ppo_step_through_the_backward():
    # forward -> clipped loss with a KL penalty -> backward, against the oracle's chain rule
    import linear_selected_token_amd as rlk
    spec = wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=101,
                          T=0.9)
    w = wl.make(spec)
    d = upload(w)
    dev = d["h"].device
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    r = np.random.default_rng(102)
    lp = logp.cpu().numpy()
    old = (lp + r.normal(0, 0.2, w.N)).astype(np.float32)
    ref = (lp + r.normal(0, 0.2, w.N)).astype(np.float32)
    ratio = np.exp(lp.astype(np.float64) - old)
    near = (np.abs(ratio - 0.8) < 1e-4) | (np.abs(ratio - 1.2) < 1e-4)
    old[near] = lp[near]
    n_act = int(w.mask.sum())
    _, badv, _, _ = rlk.rlk_ratio_kl_loss(logp, torch.from_numpy(old).to(dev),
                                          torch.from_numpy(ref).to(dev), d["adv"], d["mask"],
                                          0.2, 0.2, 0.05, 1.0 / n_act)
    dh, dW = rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, badv, lse)
    torch.cuda.synchronize()
    h64, W64 = oracle_inputs(w)
    olp, _ = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    _, og, _, _, _ = orl.ratio_kl_loss(olp, old, ref, w.adv, w.mask, 0.2, 0.2, 0.05, 1.0 / n_act)
    odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, -og)
    dh, dW = dh.cpu().numpy(), dW.cpu().numpy()
    act = np.nonzero(w.mask)[0]
    flush(f"  PPO step N={w.N} H={w.H} V={w.V}")
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert_tiles("dW", dW, odW)


# ------------------------------------------------------------------ diagnostics

def _gpu_diag(a, b, mask, eps):
    import linear_selected_token_amd as rlk
    dev = device()
    t = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    out, worst = rlk.rlk_dlogp_diagnostics(t(a), t(b), t(mask), eps)
    torch.cuda.synchronize()
    return dict(zip(rlk.DIAG_FIELDS, out.cpu().numpy().tolist())), int(worst.item())


def _diag_inputs(seed, N, scale=1e-3):
    r = np.random.default_rng(seed)
    a = (-r.exponential(2.0, N)).astype(np.float32)
    b = (a + r.normal(0, scale, N) * r.exponential(1.0, N)).astype(np.float32)
    mask = (r.random(N) < 0.6).astype(np.uint8)
    return a, b, mask


@pytest.mark.parametrize("N", [1, 999, 4096, 100003, (1 << 20) + 7])
def test_diagnostics_match_oracle(N):
    a, b, mask = _diag_inputs(N, N)
    if N == 1:
        mask[:] = 1
    g, worst = _gpu_diag(a, b, mask, 2e-3)
    o = orl.dlogp_diagnostics(a, b, mask, 2e-3)
    flush(f"  diagnostics N={N}: active={g['active']:.0f} p50={g['p50']:.3e} p99={g['p99']:.3e} "
          f"max={g['max']:.3e} worst={worst}")
    assert g["active"] == o["active"] and worst == o["worst"]
    assert g["max"] == o["max"] and g["clipfrac"] == o["clipfrac"]
    for k in ("mean", "p50", "p90", "p99", "ratio_mean"):
        assert abs(g[k] - o[k]) <= 1e-12 * max(abs(o[k]), 1e-300), (k, g[k], o[k])
    # each term exp(d) - 1 - d ~ d^2 / 2 carries the last-bit difference of two fp64 exps
    assert abs(g["approx_kl"] - o["approx_kl"]) <= 1e-8 * o["approx_kl"]
    # the order statistics themselves are exact
    act = np.nonzero(mask)[0]
    s = np.sort(np.abs(a[act].astype(np.float64) - b[act]))
    pos = 50 * (s.size - 1) / 100
    if pos == int(pos):
        assert g["p50"] == s[int(pos)]


def test_diagnostics_ties_empty_and_identical():
    a = np.array([0.0, -1.0, -2.0, -3.0, -4.0], np.float32)
    b = np.array([0.5, -1.5, -2.0, -3.5, -4.0], np.float32)
    g, worst = _gpu_diag(a, b, np.ones(5, np.uint8), 0.1)
    assert worst == 0 and g["max"] == 0.5 and g["p50"] == 0.5
    g, worst = _gpu_diag(a, b, np.zeros(5, np.uint8), 0.1)
    assert worst == -1 and not any(g.values())
    a2, _, m2 = _diag_inputs(7, 5000)
    g, worst = _gpu_diag(a2, a2.copy(), m2, 0.1)
    assert g["max"] == 0 and g["p99"] == 0 and g["approx_kl"] == 0 and g["ratio_mean"] == 1
    assert worst == int(np.nonzero(m2)[0][0])
