"""Pins of the full-vocabulary KL oracle (oracle/distill.py) against what mathematics fixes
(no GPU): library KL, pure-Python brute force, identities, closed forms, autograd and
finite differences.  Student and teacher have different hidden sizes throughout, so that a
swapped operand cannot pass by accident."""
import math

import numpy as np
import pytest
import torch

import oracle.distill as od


def _heads(seed, N=9, Hs=7, Ht=5, V=23, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((N, Hs)) * scale, r.standard_normal((V, Hs)),
            r.standard_normal((N, Ht)) * scale, r.standard_normal((V, Ht)))


def test_library_kl_div():
    hs, Ws, ht, Wt = _heads(1)
    T = 0.8
    m = np.array([1, 0, 1, 1, 1, 0, 1, 1, 1], np.uint8)
    f, r = od.kl_divergences(hs, Ws, ht, Wt, m, T)
    ls = torch.log_softmax(torch.from_numpy(hs @ Ws.T / T), 1)
    lt = torch.log_softmax(torch.from_numpy(ht @ Wt.T / T), 1)
    lib_f = torch.nn.functional.kl_div(ls, lt, log_target=True, reduction="none").sum(1).numpy()
    lib_r = torch.nn.functional.kl_div(lt, ls, log_target=True, reduction="none").sum(1).numpy()
    act = m == 1
    np.testing.assert_allclose(f[act], lib_f[act], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r[act], lib_r[act], rtol=0, atol=1e-12)
    assert not f[~act].any() and not r[~act].any()


def test_brute_force_tiny():
    hs, Ws, ht, Wt = _heads(2, N=3, V=6)
    T = 1.3
    f, r = od.kl_divergences(hs, Ws, ht, Wt, np.ones(3, np.uint8), T)
    for t in range(3):
        zs = [math.fsum(a * b for a, b in zip(hs[t], Ws[v])) / T for v in range(6)]
        zt = [math.fsum(a * b for a, b in zip(ht[t], Wt[v])) / T for v in range(6)]
        ls = [z - max(zs) - math.log(math.fsum(math.exp(x - max(zs)) for x in zs)) for z in zs]
        lt = [z - max(zt) - math.log(math.fsum(math.exp(x - max(zt)) for x in zt)) for z in zt]
        assert abs(f[t] - math.fsum(math.exp(b) * (b - a) for a, b in zip(ls, lt))) < 1e-13
        assert abs(r[t] - math.fsum(math.exp(a) * (a - b) for a, b in zip(ls, lt))) < 1e-13


def test_identities_and_closed_forms():
    hs, Ws, ht, Wt = _heads(3, scale=2.0)
    T = 0.9
    ones = np.ones(9, np.uint8)
    # identical heads: both directions vanish
    f, r = od.kl_divergences(hs, Ws, hs, Ws, ones, T)
    assert np.abs(f).max() < 1e-13 and np.abs(r).max() < 1e-13
    # Gibbs: KL >= 0, with different heads strictly
    f, r = od.kl_divergences(hs, Ws, ht, Wt, ones, T)
    assert (f > 0).all() and (r > 0).all()
    # a uniform teacher: KL_fwd = -ln V - mean_v log p_s, KL_rev = ln V - H(p_s)
    V = Ws.shape[0]
    f, r = od.kl_divergences(hs, Ws, ht, np.zeros_like(Wt), ones, T)
    ls = hs @ Ws.T / T
    ls = ls - (ls.max(1, keepdims=True) + np.log(np.exp(ls - ls.max(1, keepdims=True)).sum(1,
                                                                                      keepdims=True)))
    np.testing.assert_allclose(f, -math.log(V) - ls.mean(1), rtol=0, atol=1e-12)
    ent = -(np.exp(ls) * ls).sum(1)
    np.testing.assert_allclose(r, math.log(V) - ent, rtol=0, atol=1e-12)
    # temperature folds into the hidden states
    f1, r1 = od.kl_divergences(hs, Ws, ht, Wt, ones, 0.5)
    f2, r2 = od.kl_divergences(hs / 0.5, Ws, ht / 0.5, Wt, ones, 1.0)
    np.testing.assert_allclose(f1, f2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r1, r2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_grads_match_autograd(reverse):
    hs, Ws, ht, Wt = _heads(4, N=11, V=29)
    T = 0.7
    m = (np.random.default_rng(5).random(11) < 0.7).astype(np.uint8)
    c = np.random.default_rng(6).uniform(0.2, 2, 11)
    dh, dW = od.kl_grads(hs, Ws, ht, Wt, m, T, c, reverse)
    th = torch.tensor(hs, requires_grad=True)
    tW = torch.tensor(Ws, requires_grad=True)
    ls = torch.log_softmax(th @ tW.T / T, 1)
    lt = torch.log_softmax(torch.from_numpy(ht @ Wt.T / T), 1)
    kl = ((ls.exp() * (ls - lt)) if reverse else (lt.exp() * (lt - ls))).sum(1)
    L = (torch.from_numpy(m * c) * kl).sum()
    L.backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=0, atol=1e-12)
    assert not dh[m == 0].any()


@pytest.mark.parametrize("reverse", [False, True])
def test_grads_finite_differences_and_rows(reverse):
    hs, Ws, ht, Wt = _heads(7, N=4, Hs=3, Ht=4, V=6)
    T = 1.1
    m = np.array([1, 1, 0, 1], np.uint8)
    c = np.array([0.5, 2.0, 1.0, 1.5])
    dh, dW = od.kl_grads(hs, Ws, ht, Wt, m, T, c, reverse)

    def loss(h, W):
        f, r = od.kl_divergences(h, W, ht, Wt, m, T)
        return float(np.sum(m * c * (r if reverse else f)))

    eps = 1e-6
    for (i, j) in [(0, 0), (1, 2), (3, 1)]:
        hp, hm = hs.copy(), hs.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        assert abs((loss(hp, Ws) - loss(hm, Ws)) / (2 * eps) - dh[i, j]) < 1e-7
    for (i, j) in [(0, 0), (5, 2), (3, 1)]:
        Wp, Wm = Ws.copy(), Ws.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        assert abs((loss(hs, Wp) - loss(hs, Wm)) / (2 * eps) - dW[i, j]) < 1e-7
    rows = [3, 0]
    np.testing.assert_allclose(od.kl_grad_h_rows(hs, Ws, ht, Wt, m, T, c, reverse, rows),
                               dh[rows], rtol=0, atol=1e-14)
    vr = [5, 0, 2]
    np.testing.assert_allclose(od.kl_grad_W_rows(hs, Ws, ht, Wt, m, T, c, reverse, vr),
                               dW[vr], rtol=0, atol=1e-13)
