"""Pins of the CPU oracle against what mathematics fixes (no GPU).

Each check is chosen so that a plausible slip in the oracle (a dropped temperature, a
wrong sign, a transposed operand, an off-by-one target index, a missing max shift, a
wrong upstream gradient) fails at least one of them.  Non-square shapes (N != H != V)
are used throughout so that a transposed operand cannot pass by accident."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(seed, N, H, V, scale_w=None):
    r = np.random.default_rng(seed)
    h = r.standard_normal((N, H))
    W = r.standard_normal((V, H)) * (scale_w if scale_w is not None else 1.0 / math.sqrt(H))
    y = r.integers(0, V, size=N)
    return h, W, y


def _brute_logp(h, W, y, mask, T):
    """Pure-Python definition: exact-sum dot products, max-shifted log-sum-exp."""
    N, V = len(h), len(W)
    out_lp, out_lse = [], []
    for t in range(N):
        if not mask[t]:
            out_lp.append(0.0)
            out_lse.append(0.0)
            continue
        z = [math.fsum(a * b for a, b in zip(h[t], W[v])) / T for v in range(V)]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(zz - m) for zz in z))
        out_lp.append(z[y[t]] - lse)
        out_lse.append(lse)
    return np.array(out_lp), np.array(out_lse)


@pytest.mark.parametrize("T", [1.0, 0.7, 1.9])
def test_brute_force_tiny(T):
    h, W, y = _rand(1, 6, 7, 11)
    mask = np.array([1, 1, 0, 1, 0, 1], dtype=np.uint8)
    lp, lse = oracle.linear_logp(h, W, y, mask, T)
    blp, blse = _brute_logp(h.tolist(), W.tolist(), y.tolist(), mask.tolist(), T)
    np.testing.assert_allclose(lp, blp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    assert np.all(lp[mask == 0] == 0) and np.all(lse[mask == 0] == 0)


def test_brute_force_large_logits():
    # logits of size ~ +-1e3: the max shift must keep exp in range
    h, W, y = _rand(2, 4, 5, 9, scale_w=150.0)
    mask = np.ones(4, dtype=np.uint8)
    lp, lse = oracle.linear_logp(h, W, y, mask, 0.5)
    assert np.all(np.isfinite(lp)) and np.abs(lse).max() > 300
    blp, blse = _brute_logp(h.tolist(), W.tolist(), y.tolist(), mask.tolist(), 0.5)
    np.testing.assert_allclose(lp, blp, rtol=1e-13, atol=1e-9)
    np.testing.assert_allclose(lse, blse, rtol=1e-13, atol=1e-9)


def test_library_cross_entropy():
    # -cross_entropy(z, y) is the selected log-prob (torch, float64, CPU)
    h, W, y = _rand(3, 200, 48, 3001)
    T = 0.7
    mask = np.ones(200, dtype=np.uint8)
    lp, _ = oracle.linear_logp(h, W, y, mask, T)
    z = torch.from_numpy(h) @ torch.from_numpy(W).T / T
    ref = -torch.nn.functional.cross_entropy(z, torch.from_numpy(y), reduction="none")
    np.testing.assert_allclose(lp, ref.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("V", [1, 7, 1000, 151936])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_zero_weight_closed_form(V, T):
    h, _, _ = _rand(4, 5, 64, 1)
    W = np.zeros((V, 64))
    y = np.random.default_rng(5).integers(0, V, size=5)
    lp, lse = oracle.linear_logp(h, W, y, np.ones(5, dtype=np.uint8), T)
    np.testing.assert_allclose(lp, -math.log(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, math.log(V), rtol=0, atol=1e-12)


def test_single_token_vocab():
    h, W, _ = _rand(6, 8, 16, 1, scale_w=3.0)
    lp, _ = oracle.linear_logp(h, W, np.zeros(8, dtype=np.int64), np.ones(8, np.uint8), 0.9)
    assert np.all(np.abs(lp) < 1e-15)


def test_two_token_vocab_softplus():
    h, W, y = _rand(7, 9, 13, 2, scale_w=2.0)
    T = 1.3
    lp, _ = oracle.linear_logp(h, W, y, np.ones(9, np.uint8), T)
    for t in range(9):
        zy = math.fsum(a * b for a, b in zip(h[t], W[y[t]])) / T
        zo = math.fsum(a * b for a, b in zip(h[t], W[1 - y[t]])) / T
        d = zo - zy
        softplus = d + math.log1p(math.exp(-d)) if d > 0 else math.log1p(math.exp(d))
        assert abs(lp[t] + softplus) < 1e-13


def test_normalised_and_nonpositive():
    h, W, _ = _rand(8, 10, 32, 257)
    flp = oracle.full_logp(h, W, 0.8)
    assert np.all(flp <= 0)
    np.testing.assert_allclose(np.exp(flp).sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_temperature_folds_into_h():
    h, W, y = _rand(9, 12, 40, 500)
    m = np.ones(12, np.uint8)
    a, la = oracle.linear_logp(h, W, y, m, 0.7)
    b, lb = oracle.linear_logp(h / 0.7, W, y, m, 1.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)
    c, _ = oracle.linear_logp(h, W, y, m, 1.0)
    assert np.abs(a - c).max() > 1e-3  # T really enters


def test_vocab_permutation_and_duplicates():
    h, W, y = _rand(10, 7, 24, 300)
    m = np.ones(7, np.uint8)
    lp, _ = oracle.linear_logp(h, W, y, m, 1.1)
    perm = np.random.default_rng(11).permutation(300)
    inv = np.argsort(perm)
    lp2, _ = oracle.linear_logp(h, W[perm], inv[y], m, 1.1)
    np.testing.assert_allclose(lp, lp2, rtol=0, atol=1e-12)
    Wd = W.copy()
    Wd[5] = Wd[17]
    y5 = np.full(7, 5)
    y17 = np.full(7, 17)
    np.testing.assert_array_equal(oracle.linear_logp(h, Wd, y5, m, 1.1)[0],
                                  oracle.linear_logp(h, Wd, y17, m, 1.1)[0])


def test_rows_subset_and_invalid_target():
    h, W, y = _rand(12, 30, 16, 77)
    m = (np.arange(30) % 3 != 0).astype(np.uint8)
    lp, lse = oracle.linear_logp(h, W, y, m, 1.0)
    rows = [29, 1, 2, 14, 3]
    lp2, lse2 = oracle.linear_logp(h, W, y, m, 1.0, rows=rows)
    np.testing.assert_array_equal(lp2, lp[rows])
    np.testing.assert_array_equal(lse2, lse[rows])
    yb = y.copy()
    yb[4] = 77
    with pytest.raises(ValueError):
        oracle.linear_logp(h, W, yb, m, 1.0)
    yb[4] = -1
    yb[3] = 77  # inactive row: ignored
    with pytest.raises(ValueError):
        oracle.linear_logp(h, W, yb, m, 1.0)
    yb[4] = 0
    oracle.linear_logp(h, W, yb, m, 1.0)


# ------------------------------------------------------------------ backward

def _grad_setup(seed, N=9, H=10, V=23):
    h, W, y = _rand(seed, N, H, V, scale_w=0.8)
    r = np.random.default_rng(seed + 100)
    mask = (r.random(N) < 0.7).astype(np.uint8)
    mask[0] = 1
    adv = r.standard_normal(N)
    return h, W, y, mask, adv


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_grads_match_library_autograd(T):
    h, W, y, mask, adv = _grad_setup(20, N=17, H=12, V=41)
    dh, dW = oracle.linear_logp_grads(h, W, y, mask, T, adv)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    logp = -torch.nn.functional.cross_entropy(th @ tW.T / T, torch.tensor(y), reduction="none")
    loss = -(torch.tensor(mask, dtype=torch.float64) * torch.tensor(adv) * logp).sum()
    loss.backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=0, atol=1e-12)


def test_grads_finite_differences():
    h, W, y, mask, adv = _grad_setup(21, N=4, H=5, V=6)
    T = 0.85
    dh, dW = oracle.linear_logp_grads(h, W, y, mask, T, adv)

    def loss(hh, WW):
        lp, _ = oracle.linear_logp(hh, WW, y, mask, T)
        return -float(np.sum(mask * adv * lp))

    eps = 1e-6
    for (i, j) in [(0, 0), (1, 3), (3, 4), (2, 2)]:
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        assert abs((loss(hp, W) - loss(hm, W)) / (2 * eps) - dh[i, j]) < 1e-7
    for (i, j) in [(0, 0), (5, 1), (y[0], 2), (3, 4)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        assert abs((loss(h, Wp) - loss(h, Wm)) / (2 * eps) - dW[i, j]) < 1e-7


def test_grad_invariants():
    h, W, y, mask, adv = _grad_setup(22, N=13, H=8, V=31)
    dh, dW = oracle.linear_logp_grads(h, W, y, mask, 1.2, adv)
    # every row of dL/dz sums to zero, so the columns of dW sum to zero
    np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-13)
    assert np.all(dh[mask == 0] == 0)
    z0h, z0W = oracle.linear_logp_grads(h, W, y, mask, 1.2, np.zeros_like(adv))
    assert not z0h.any() and not z0W.any()


def test_grad_zero_weight_closed_form():
    h, _, y, mask, adv = _grad_setup(23, N=11, H=6, V=19)
    T = 0.6
    V = 19
    W = np.zeros((V, 6))
    dh, dW = oracle.linear_logp_grads(h, W, y, mask, T, adv)
    assert not dh.any()
    ref = np.zeros((V, 6))
    for t in range(11):
        g = -float(mask[t]) * adv[t]
        for v in range(V):
            ref[v] += g * ((1.0 if v == y[t] else 0.0) - 1.0 / V) * h[t] / T
    np.testing.assert_allclose(dW, ref, rtol=0, atol=1e-13)


def test_grad_row_variants_match_full():
    h, W, y, mask, adv = _grad_setup(24, N=40, H=9, V=70)
    T = 0.9
    dh, dW = oracle.linear_logp_grads(h, W, y, mask, T, adv)
    rows = [0, 5, 39, 7]
    np.testing.assert_allclose(oracle.grad_h_rows(h, W, y, mask, T, adv, rows), dh[rows],
                               rtol=0, atol=1e-14)
    vr = [0, 69, int(y[0]), 33]
    np.testing.assert_allclose(oracle.grad_W_rows(h, W, y, mask, T, adv, vr), dW[vr],
                               rtol=0, atol=1e-14)


# ------------------------------------------------------------------ sampler

def test_sampler_inverse_cdf_walk():
    h, W, _ = _rand(30, 8, 5, 6, scale_w=1.5)
    T = 0.9
    r = np.random.default_rng(31)
    for t in range(8):
        us = r.random(25)
        got = oracle.sample_targets(np.repeat(h[t:t + 1], 25, axis=0), W, T, us)
        z = [math.fsum(a * b for a, b in zip(h[t], W[v])) / T for v in range(6)]
        m = max(z)
        e = [math.exp(zz - m) for zz in z]
        p = [x / math.fsum(e) for x in e]
        for k, u in enumerate(us):
            acc, pick = 0.0, 5
            for v in range(6):
                acc += p[v]
                if acc > u:
                    pick = v
                    break
            assert got[k] == pick


def test_sampler_frequencies():
    from scipy.stats import chisquare
    h, W, _ = _rand(32, 1, 4, 8, scale_w=1.0)
    T = 0.7
    n = 40000
    u = np.random.default_rng(33).random(n)
    ys = oracle.sample_targets(np.repeat(h, n, axis=0), W, T, u)
    p = np.exp(oracle.full_logp(h, W, T)[0])
    counts = np.bincount(ys, minlength=8)
    assert chisquare(counts, p * n).pvalue > 1e-4


# ---------------------------------------------------------------- log-prob from existing logits

def test_logits_path_equals_fused_definition():
    # logits formed from h and W give exactly what the fused definition gives
    r = np.random.default_rng(31)
    N, H, V, T = 37, 24, 301, 0.7
    h = r.standard_normal((N, H))
    W = r.standard_normal((V, H)) / np.sqrt(H)
    y = r.integers(0, V, N)
    m = (r.random(N) < 0.7).astype(np.uint8)
    a_lp, a_lse = oracle.logp_from_logits(h @ W.T, y, m, T)
    b_lp, b_lse = oracle.linear_logp(h, W, y, m, T)
    assert np.allclose(a_lp, b_lp, rtol=0, atol=1e-12)
    assert np.allclose(a_lse, b_lse, rtol=0, atol=1e-12)
    assert not a_lp[m == 0].any() and not a_lse[m == 0].any()


def test_logits_path_brute_force_and_library():
    # pure-Python brute force with math.fsum, and the library cross-entropy
    r = np.random.default_rng(32)
    N, V, T = 9, 13, 1.3
    z = r.standard_normal((N, V)) * 4
    y = r.integers(0, V, N)
    m = np.ones(N, dtype=np.uint8)
    lp, lse = oracle.logp_from_logits(z, y, m, T)
    for t in range(N):
        zt = [float(v) / T for v in z[t]]
        mx = max(zt)
        l = mx + math.log(math.fsum(math.exp(v - mx) for v in zt))
        assert abs(lse[t] - l) < 1e-12 and abs(lp[t] - (zt[y[t]] - l)) < 1e-12
    ce = torch.nn.functional.cross_entropy(torch.from_numpy(z / T), torch.from_numpy(y),
                                           reduction="none").numpy()
    assert np.allclose(lp, -ce, rtol=0, atol=1e-12)


def test_logits_path_closed_forms_and_errors():
    # constant logits: logp = -ln V at any temperature; an out-of-range target raises
    z = np.full((4, 50), 3.25)
    lp, lse = oracle.logp_from_logits(z, np.array([0, 7, 49, 3]), np.ones(4, np.uint8), 0.3)
    assert np.allclose(lp, -math.log(50), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.logp_from_logits(z, np.array([0, 50, 1, 1]), np.ones(4, np.uint8), 1.0)
    # but an inactive token's target is never looked at
    oracle.logp_from_logits(z, np.array([0, 50, 1, 1]), np.array([1, 0, 1, 1], np.uint8), 1.0)


# ---------------------------------------------------------------- entropy

def test_entropy_brute_force_and_library():
    r = np.random.default_rng(41)
    N, H, V, T = 7, 6, 11, 0.8
    h = r.standard_normal((N, H)) * 2
    W = r.standard_normal((V, H))
    m = np.array([1, 1, 0, 1, 1, 0, 1], dtype=np.uint8)
    ent = oracle.entropy(h, W, m, T)
    for t in range(N):
        if not m[t]:
            assert ent[t] == 0.0
            continue
        z = [math.fsum(h[t, k] * W[v, k] for k in range(H)) / T for v in range(V)]
        mx = max(z)
        e = [math.exp(v - mx) for v in z]
        S = math.fsum(e)
        want = -math.fsum((x / S) * math.log(x / S) for x in e)
        assert abs(ent[t] - want) < 1e-12
    lib = torch.distributions.Categorical(logits=torch.from_numpy(h @ W.T / T)).entropy().numpy()
    assert np.allclose(ent[m == 1], lib[m == 1], rtol=0, atol=1e-12)


def test_entropy_closed_forms():
    r = np.random.default_rng(42)
    h = r.standard_normal((5, 8))
    ones = np.ones(5, dtype=np.uint8)
    # uniform distribution: ln V; one entry: 0
    assert np.allclose(oracle.entropy(h, np.zeros((37, 8)), ones, 0.6), math.log(37),
                       rtol=0, atol=1e-12)
    assert np.allclose(oracle.entropy(h, r.standard_normal((1, 8)), ones, 1.0), 0.0,
                       rtol=0, atol=1e-12)
    # two entries: the binary entropy of sigmoid(z1 - z0)
    W = r.standard_normal((2, 8))
    d = (h @ (W[1] - W[0])) / 1.7
    q = 1 / (1 + np.exp(-d))
    want = -(q * np.log(q) + (1 - q) * np.log(1 - q))
    assert np.allclose(oracle.entropy(h, W, ones, 1.7), want, rtol=0, atol=1e-12)


def test_entropy_equals_lse_minus_mean_logit():
    # H = lse - E_p[z]: the form the fused epilogue accumulates
    r = np.random.default_rng(43)
    h = r.standard_normal((9, 16))
    W = r.standard_normal((200, 16)) / 4
    T = 0.9
    ones = np.ones(9, dtype=np.uint8)
    z = h @ W.T / T
    lse = oracle.logsumexp_rows(z)
    ez = np.sum(np.exp(z - lse[:, None]) * z, axis=1)
    assert np.allclose(oracle.entropy(h, W, ones, T), lse - ez, rtol=0, atol=1e-11)


# ------------------------------------------------------------------ entropy-bonus gradients

def _ent_loss(h, W, y, mask, T, adv, c):
    lp, _ = oracle.linear_logp(h, W, y, mask, T)
    H = oracle.entropy(h, W, mask, T)
    return -float(np.sum(mask * (adv * lp + c * H)))


def test_entropy_grads_finite_differences():
    h, W, y, mask, adv = _grad_setup(40, N=5, H=4, V=7)
    c = np.random.default_rng(41).uniform(0.2, 2.0, 5)
    T = 0.8
    dh, dW = oracle.linear_logp_entropy_grads(h, W, y, mask, T, adv, c)
    eps = 1e-6
    for (i, j) in [(0, 0), (1, 3), (4, 2), (2, 1)]:
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        fd = (_ent_loss(hp, W, y, mask, T, adv, c) - _ent_loss(hm, W, y, mask, T, adv, c)) / (2 * eps)
        assert abs(fd - dh[i, j]) < 1e-7, (i, j, fd, dh[i, j])
    for (i, j) in [(0, 0), (6, 3), (int(y[0]), 2), (3, 1)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        fd = (_ent_loss(h, Wp, y, mask, T, adv, c) - _ent_loss(h, Wm, y, mask, T, adv, c)) / (2 * eps)
        assert abs(fd - dW[i, j]) < 1e-7, (i, j, fd, dW[i, j])


def test_entropy_grads_match_library_autograd():
    h, W, y, mask, adv = _grad_setup(42, N=19, H=11, V=37)
    c = np.random.default_rng(43).standard_normal(19)
    T = 1.3
    dh, dW = oracle.linear_logp_entropy_grads(h, W, y, mask, T, adv, c)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    lsm = torch.log_softmax(th @ tW.T / T, dim=1)
    logp = lsm.gather(1, torch.tensor(y)[:, None])[:, 0]
    ent = -(lsm.exp() * lsm).sum(1)
    m = torch.tensor(mask, dtype=torch.float64)
    loss = -(m * (torch.tensor(adv) * logp + torch.tensor(c) * ent)).sum()
    loss.backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=0, atol=1e-12)


def test_entropy_grads_special_cases():
    h, W, y, mask, adv = _grad_setup(44, N=13, H=6, V=23)
    T = 0.9
    # no entropy bonus: the plain gradients
    dh0, dW0 = oracle.linear_logp_grads(h, W, y, mask, T, adv)
    dh1, dW1 = oracle.linear_logp_entropy_grads(h, W, y, mask, T, adv, np.zeros(13))
    np.testing.assert_array_equal(dh0, dh1)
    np.testing.assert_array_equal(dW0, dW1)
    # W = 0: every distribution is uniform, where the entropy is at its maximum and its
    # gradient vanishes; with adv = 0 nothing is left
    dh, dW = oracle.linear_logp_entropy_grads(h, np.zeros((23, 6)), y, mask, T, np.zeros(13),
                                              np.ones(13))
    assert np.abs(dh).max() < 1e-15 and np.abs(dW).max() < 1e-15
    # every row of dL/dz sums to zero (p-weighted log p + H has mean zero), so dW's columns do
    _, dW = oracle.linear_logp_entropy_grads(h, W, y, mask, T, adv, np.full(13, 0.5))
    np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-13)


def test_entropy_grad_row_variants_match_full():
    h, W, y, mask, adv = _grad_setup(45, N=30, H=7, V=50)
    c = np.random.default_rng(46).uniform(0, 1, 30)
    T = 0.75
    dh, dW = oracle.linear_logp_entropy_grads(h, W, y, mask, T, adv, c)
    rows = [0, 29, 11, 4]
    np.testing.assert_allclose(oracle.grad_h_rows(h, W, y, mask, T, adv, rows, ent_coef=c),
                               dh[rows], rtol=0, atol=1e-14)
    vr = [0, 49, int(y[0]), 17]
    np.testing.assert_allclose(oracle.grad_W_rows(h, W, y, mask, T, adv, vr, ent_coef=c),
                               dW[vr], rtol=0, atol=1e-14)
