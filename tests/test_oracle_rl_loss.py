"""Pins of the loss-fragment oracle (oracle/rl_loss.py) against what the definitions fix (no
GPU): library autograd, a pure-Python walk of each token, closed forms and order statistics
read off a sorted copy."""
import math

import numpy as np
import torch

import oracle.rl_loss as rl


def _inputs(seed, N, spread=0.4):
    r = np.random.default_rng(seed)
    logp = -r.exponential(2.0, N)
    old = logp + r.normal(0, spread, N)
    ref = logp + r.normal(0, spread, N)
    adv = r.normal(0, 1, N)
    mask = (r.random(N) < 0.8).astype(np.uint8)
    return logp, old, ref, adv, mask


def test_loss_matches_library_autograd():
    logp, old, ref, adv, mask = _inputs(1, 300)
    eps_lo, eps_hi, beta, scale = 0.2, 0.28, 0.05, 1.0 / 300
    loss, grad, ratio, clipped, sums = rl.ratio_kl_loss(logp, old, ref, adv, mask, eps_lo, eps_hi,
                                                        beta, scale)
    lp = torch.tensor(logp, requires_grad=True)
    r = torch.exp(lp - torch.tensor(old))
    A = torch.tensor(adv)
    pg = torch.maximum(-A * r, -A * torch.clamp(r, 1 - eps_lo, 1 + eps_hi))
    d = torch.tensor(ref) - lp
    kl = torch.exp(d) - 1 - d
    m = torch.tensor(mask, dtype=torch.float64)
    L = (scale * m * (pg + beta * kl)).sum()
    L.backward()
    np.testing.assert_allclose(grad, lp.grad.numpy(), rtol=0, atol=1e-15)
    assert abs(sums["loss"] - L.item()) < 1e-12
    assert 0 < sums["clipped"] < mask.sum()          # both branches are exercised
    assert sums["active"] == mask.sum()


def test_loss_pure_python_walk():
    logp, old, ref, adv, mask = _inputs(2, 64, spread=0.6)
    eps_lo, eps_hi, beta, scale = 0.1, 0.3, 0.2, 0.5
    loss, grad, ratio, clipped, sums = rl.ratio_kl_loss(logp, old, ref, adv, mask, eps_lo, eps_hi,
                                                        beta, scale)
    tot = 0.0
    for t in range(64):
        if not mask[t]:
            assert loss[t] == 0 and grad[t] == 0 and ratio[t] == 0 and clipped[t] == 0
            continue
        r = math.exp(logp[t] - old[t])
        rc = min(max(r, 1 - eps_lo), 1 + eps_hi)
        a, b = -adv[t] * r, -adv[t] * rc
        take_clip = b > a
        pg = b if take_clip else a
        g = 0.0 if take_clip else -adv[t] * r
        dd = ref[t] - logp[t]
        kl = math.exp(dd) - 1 - dd
        g += beta * (1 - math.exp(dd))
        assert abs(loss[t] - scale * (pg + beta * kl)) < 1e-14
        assert abs(grad[t] - scale * g) < 1e-14
        assert clipped[t] == int(take_clip)
        assert abs(ratio[t] - r) < 1e-14
        tot += scale * (pg + beta * kl)
    assert abs(sums["loss"] - tot) < 1e-12


def test_loss_closed_forms():
    N = 50
    r = np.random.default_rng(3)
    logp = -r.exponential(1.0, N)
    adv = r.normal(0, 1, N)
    mask = np.ones(N, np.uint8)
    # on-policy (r = 1), no KL: L = -scale A, dL/dlogp = -scale A, nothing clipped
    loss, grad, ratio, clipped, sums = rl.ratio_kl_loss(logp, logp, None, adv, mask, 0.2, 0.2, 0.0,
                                                        2.0)
    np.testing.assert_array_equal(ratio, 1.0)
    np.testing.assert_allclose(loss, -2.0 * adv, rtol=0, atol=1e-15)
    np.testing.assert_allclose(grad, -2.0 * adv, rtol=0, atol=1e-15)
    assert sums["clipped"] == 0
    # policy equal to the reference: the KL term and its gradient vanish
    l2, g2, _, _, s2 = rl.ratio_kl_loss(logp, logp, logp, adv, mask, 0.2, 0.2, 0.7, 2.0)
    np.testing.assert_array_equal(l2, loss)
    np.testing.assert_array_equal(g2, grad)
    assert s2["kl"] == 0
    # A = 0: no policy-gradient term at all
    l3, g3, _, c3, _ = rl.ratio_kl_loss(logp, logp + 0.5, None, np.zeros(N), mask, 0.2, 0.2, 0.0,
                                        1.0)
    assert not l3.any() and not g3.any() and not c3.any()
    # far outside the clip range with A > 0 and r > 1 + eps: clipped, gradient 0
    l4, g4, _, c4, _ = rl.ratio_kl_loss(np.array([0.0]), np.array([-1.0]), None, np.array([1.0]),
                                        np.array([1]), 0.2, 0.2, 0.0, 1.0)
    assert c4[0] == 1 and g4[0] == 0 and abs(l4[0] + 1.2) < 1e-15


def _percentile(sorted_vals, q):
    pos = q / 100.0 * (len(sorted_vals) - 1)
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(sorted_vals) - 1)
    return sorted_vals[lo] + (pos - lo) * (sorted_vals[hi] - sorted_vals[lo])


def test_diagnostics_against_sorted_copy():
    r = np.random.default_rng(4)
    N = 1001
    a = -r.exponential(2.0, N)
    b = a + r.normal(0, 1e-3, N)
    mask = (r.random(N) < 0.6).astype(np.uint8)
    out = rl.dlogp_diagnostics(a, b, mask, 0.002)
    act = [t for t in range(N) if mask[t]]
    d = [a[t] - b[t] for t in act]
    s = sorted(abs(x) for x in d)
    assert out["active"] == len(act)
    assert abs(out["mean"] - math.fsum(s) / len(s)) < 1e-15
    assert out["max"] == s[-1]
    for q in (50, 90, 99):
        assert abs(out[f"p{q}"] - _percentile(s, q)) < 1e-15
    assert abs(out["ratio_mean"] - math.fsum(math.exp(x) for x in d) / len(d)) < 1e-15
    assert out["clipfrac"] == sum(abs(math.exp(x) - 1) > 0.002 for x in d) / len(d)
    assert abs(out["approx_kl"] - math.fsum(math.exp(x) - 1 - x for x in d) / len(d)) < 1e-15
    worst = max(act, key=lambda t: abs(a[t] - b[t]))
    assert out["worst"] == worst


def test_diagnostics_ties_and_empty():
    a = np.array([0.0, -1.0, -2.0, -3.0])
    b = np.array([0.5, -1.5, -2.0, -3.5])   # |d| = .5 .5 0 .5: the first of the tied maxima
    out = rl.dlogp_diagnostics(a, b, np.array([1, 1, 1, 1]), 0.1)
    assert out["worst"] == 0 and out["p50"] == 0.5 and out["max"] == 0.5
    empty = rl.dlogp_diagnostics(a, b, np.zeros(4, np.uint8), 0.1)
    assert empty["active"] == 0 and empty["worst"] == -1


def test_kl_reported_without_penalty():
    logp, old, ref, adv, mask = _inputs(5, 200)
    l0, g0, _, _, s0 = rl.ratio_kl_loss(logp, old, None, adv, mask, 0.2, 0.2, 0.0, 1.0)
    l1, g1, _, _, s1 = rl.ratio_kl_loss(logp, old, ref, adv, mask, 0.2, 0.2, 0.0, 1.0)
    np.testing.assert_array_equal(l0, l1)
    np.testing.assert_array_equal(g0, g1)
    m = mask.astype(bool)
    d = ref[m] - logp[m]
    assert s0["kl"] == 0
    assert abs(s1["kl"] - math.fsum(math.exp(x) - 1 - x for x in d)) < 1e-10
