"""Full-vocabulary KL between a student and a teacher head against the float64 oracle (needs
an MI355X).

Gates: |dKL| <= 1e-3 in both directions (KL is a difference of log-sum-exps and a
probability-weighted mean of logits, each within the logp gate's reach of per-logit error),
each head's lse as for the plain forward; a token's results bit-identical in any batch;
identical heads give exactly 0.  Backward: rel-L2 of dh_s and dW_s <= 1e-2 for both
directions."""
import numpy as np
import pytest
import torch

import oracle
import oracle.distill as od
import workloads as wl
from gpu_util import (MAX_ABS_DLOGP, assert_rows, assert_tiles, bits, device, edge_rows, flush,
                      sample_rows)

pytestmark = pytest.mark.gpu


def _teacher(w, Ht, seed, close=None):
    """Teacher hidden states and head for workload w: independent draws, or (close = eps) the
    student's own head with N(0, eps^2 / H) added to W."""
    if close is not None:
        Wt = wl.bf16_to_f32(w.W) + wl.normal_rows(seed, 97, 0, w.V, w.H, close / np.sqrt(w.H),
                                                  "fp32")
        return w.h.copy(), (wl.bf16_bits(Wt) if w.dtype == "bf16" else Wt)
    ht = wl.normal_rows(seed, 96, 0, w.N, Ht, 1.0, w.dtype)
    return ht, wl.weight_matrix(seed + 7, w.V, Ht, w.dtype)


def _dev(x):
    dev = device()
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _fwd(w, ht, Wt, mask=None, block=None):
    import linear_selected_token_amd as rlk
    m = w.mask if mask is None else mask
    out = rlk.rlk_linear_kl_fwd(_dev(w.h), _dev(w.W), _dev(ht), _dev(Wt), _dev(m), w.T,
                                block_tokens=block)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _lse(h64, W64, T, rows):
    z = oracle.logits(h64[rows], W64, T)
    return oracle.logsumexp_rows(z)


def _check_fwd(w, ht, Wt, rows=None, tol=MAX_ABS_DLOGP, block=None):
    kf, kr, ls, lt = _fwd(w, ht, Wt, block=block)
    hs64, Ws64, ht64, Wt64 = (wl.as_f64(x) for x in (w.h, w.W, ht, Wt))
    act = w.mask.astype(bool)
    if rows is None:
        of, orv = od.kl_divergences(hs64, Ws64, ht64, Wt64, w.mask, w.T)
        rows = np.nonzero(act)[0]
        assert not kf[~act].any() and not kr[~act].any() and not ls[~act].any()
        of, orv = of[rows], orv[rows]
    else:
        of, orv = od.kl_divergences(hs64[rows], Ws64, ht64[rows], Wt64,
                                    np.ones(rows.size, np.uint8), w.T)
    ef = np.abs(kf[rows] - of).max()
    er = np.abs(kr[rows] - orv).max()
    els = np.abs(ls[rows] - _lse(hs64, Ws64, w.T, rows)).max()
    elt = np.abs(lt[rows] - _lse(ht64, Wt64, w.T, rows)).max()
    flush(f"  KL {w.dtype} N={w.N} Hs={w.H} Ht={ht.shape[1]} V={w.V}: KL_fwd~{of.mean():.3g} "
          f"max|d|={ef:.2e}  KL_rev~{orv.mean():.3g} max|d|={er:.2e}  lse {els:.1e}/{elt:.1e} "
          f"over {rows.size} tokens")
    assert ef <= tol and er <= tol and els <= tol and elt <= tol
    return kf, kr, ls, lt


SMALL = wl.scaled_spec(2, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=111,
                       T=0.8)


def test_small_full_independent_heads():
    w = wl.make(SMALL)
    ht, Wt = _teacher(w, 256, 112)
    _check_fwd(w, ht, Wt)


def test_small_full_close_heads():
    # a teacher near the student: small divergences, where the cancellation matters most
    w = wl.make(SMALL)
    ht, Wt = _teacher(w, w.H, 113, close=0.05)
    kf, kr, _, _ = _check_fwd(w, ht, Wt, tol=2e-5)
    act = w.mask.astype(bool)
    assert (kf[act] < 0.05).all()


def _chunk():
    """Vocabulary entries per backward / KL chunk of the loaded build."""
    import re
    import linear_selected_token_amd as rlk
    m = re.search(r"bwd chunk (\d+), dh split at (\d+)", rlk.build_info())
    assert m, rlk.build_info()
    return int(m.group(1)), int(m.group(2))


def test_fp32_ragged_and_two_chunks():
    w = wl.make(wl.scaled_spec(1, N=200, H=128, V=777, n_seq=2, len_lo=50, len_hi=150,
                               prompt="floor_half", seed=114, T=1.2))
    ht, Wt = _teacher(w, 64, 115)
    _check_fwd(w, ht, Wt, tol=1e-4)
    # two vocabulary chunks, the second ragged
    chunk, _ = _chunk()
    w2 = wl.make(wl.scaled_spec(2, N=260, H=256, V=chunk + 300, n_seq=2, len_lo=100,
                                len_hi=200, seed=116))
    ht2, Wt2 = _teacher(w2, 192, 117)
    _check_fwd(w2, ht2, Wt2)


def test_identical_heads_and_invariance():
    w = wl.make(SMALL)
    kf, kr, ls, lt = _fwd(w, w.h, w.W)
    act = w.mask.astype(bool)
    assert not kf.any() and not kr.any()
    assert np.array_equal(bits(ls), bits(lt))
    # a reversed subset of the tokens in a batch of its own, some masked
    ht, Wt = _teacher(w, 320, 118)
    full = _fwd(w, ht, Wt)
    sel = np.nonzero(act)[0][::-3].copy()
    import dataclasses
    sub = dataclasses.replace(w, h=np.ascontiguousarray(w.h[sel]), targets=w.targets[sel],
                              mask=w.mask[sel].copy(), adv=w.adv[sel], u=w.u[sel],
                              seq_id=w.seq_id[sel], pos=w.pos[sel])
    sub.mask[::4] = 0
    part = _fwd(sub, np.ascontiguousarray(ht[sel]), Wt)
    keep = sub.mask.astype(bool)
    mism = sum(int((bits(p[keep]) != bits(f[sel][keep])).sum()) for p, f in zip(part, full))
    flush(f"  KL invariance: {mism} mismatches over {int(keep.sum())} tokens x 4 outputs")
    assert mism == 0


def test_qwen_head_sampled():
    # the Qwen3-8B student head (H=4096, V=151936) against a smaller teacher (H=2048)
    w = wl.make(wl.scaled_spec(2, N=512, n_seq=2, len_lo=200, len_hi=300, seed=119, T=0.7))
    ht, Wt = _teacher(w, 2048, 120)
    _check_fwd(w, ht, Wt, rows=sample_rows(w, 16, seed=121))


# ------------------------------------------------------------------ backward

def _bwd(w, ht, Wt, reverse, coef):
    import linear_selected_token_amd as rlk
    d = [_dev(x) for x in (w.h, w.W, ht, Wt, w.mask)]
    kf, kr, ls, lt = rlk.rlk_linear_kl_fwd(*d, w.T)
    c = _dev(coef)
    dh, dW = rlk.rlk_linear_kl_bwd(*d, w.T, None if reverse else c, c if reverse else None, ls,
                                   lt, kr)
    torch.cuda.synchronize()
    return dh.cpu().numpy(), dW.cpu().numpy()


def _sweep_cases(n, seed):
    """Seeded (spec, H_t, reverse) cases: N in [1, 700], H_s and H_t multiples of 256 up to 768,
    V in [1, 40000] (log-uniform), T in [0.5, 1.5]."""
    r = np.random.default_rng(seed)
    out = []
    for k in range(n):
        N = int(r.integers(1, 701))
        V = int(np.exp(r.uniform(0.0, np.log(40000.0)))) + 1
        spec = wl.scaled_spec(5, N=N, H=256 * int(r.integers(1, 4)), V=V,
                              n_seq=int(min(N, r.integers(1, 4))), len_lo=1, len_hi=N,
                              seed=900 + k, T=float(r.uniform(0.5, 1.5)))
        out.append((spec, 256 * int(r.integers(1, 4)), bool(r.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _sweep_cases(10, 411),
                         ids=lambda c: f"N{c[0].N}-Hs{c[0].H}-Ht{c[1]}-V{c[0].V}-"
                                       f"{'rev' if c[2] else 'fwd'}")
def test_random_shapes_sweep(case):
    # both KL directions and both heads' lse of every active token, and the gradient of one
    # direction (every dh_s and dW_s row), against the oracle
    spec, Ht, reverse = case
    w = wl.make(spec)
    ht, Wt = _teacher(w, Ht, spec.seed + 50)
    _check_fwd(w, ht, Wt)
    c = np.random.default_rng(spec.seed + 51).uniform(0.5, 1.5, w.N).astype(np.float32)
    dh, dW = _bwd(w, ht, Wt, reverse, c)
    odh, odW = od.kl_grads(*(wl.as_f64(x) for x in (w.h, w.W, ht, Wt)), w.mask, w.T, c, reverse)
    act = np.nonzero(w.mask)[0]
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert not dh[w.mask == 0].any()


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_small_full(reverse):
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=122, T=0.9))
    ht, Wt = _teacher(w, 256, 123)
    c = np.random.default_rng(124).uniform(0.5, 1.5, w.N).astype(np.float32)
    dh, dW = _bwd(w, ht, Wt, reverse, c)
    odh, odW = od.kl_grads(*(wl.as_f64(x) for x in (w.h, w.W, ht, Wt)), w.mask, w.T, c, reverse)
    act = np.nonzero(w.mask)[0]
    flush(f"  KL bwd reverse={reverse}")
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert_tiles("dW", dW, odW)
    assert not dh[w.mask == 0].any()


def test_bwd_two_chunks_and_dh_invariance():
    chunk, split = _chunk()
    w = wl.make(wl.scaled_spec(5, N=260, H=256, V=chunk + split + 300, n_seq=2, len_lo=100,
                               len_hi=200, seed=125))
    ht, Wt = _teacher(w, 128, 126)
    c = np.random.default_rng(127).uniform(0.5, 1.5, w.N).astype(np.float32)
    dh, dW = _bwd(w, ht, Wt, False, c)
    odh, odW = od.kl_grads(*(wl.as_f64(x) for x in (w.h, w.W, ht, Wt)), w.mask, w.T, c, False)
    act = np.nonzero(w.mask)[0]
    flush("  KL bwd two chunks")
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert_tiles("dW", dW, odW)
    # the first 100 tokens alone give the same dh rows, bit for bit
    import dataclasses
    k = 100
    sub = dataclasses.replace(w, h=np.ascontiguousarray(w.h[:k]), targets=w.targets[:k],
                              mask=w.mask[:k].copy(), adv=w.adv[:k], u=w.u[:k],
                              seq_id=w.seq_id[:k], pos=w.pos[:k])
    dh2, _ = _bwd(sub, np.ascontiguousarray(ht[:k]), Wt, False, c[:k])
    act = sub.mask.astype(bool)
    assert np.array_equal(bits(dh2[act]), bits(dh[:k][act]))


def test_bwd_qwen_head_sampled():
    w = wl.make(wl.scaled_spec(5, N=512, n_seq=2, len_lo=200, len_hi=300, seed=128, T=0.7))
    ht, Wt = _teacher(w, 1024, 129)
    c = np.full(w.N, 1.0 / 256, np.float32)
    dh, dW = _bwd(w, ht, Wt, True, c)
    hs64, Ws64, ht64, Wt64 = (wl.as_f64(x) for x in (w.h, w.W, ht, Wt))
    rows = sample_rows(w, 12, seed=130)
    odh = od.kl_grad_h_rows(hs64, Ws64, ht64, Wt64, w.mask, w.T, c, True, rows)
    act = np.nonzero(w.mask)[0]
    vr = np.unique(np.concatenate([np.random.default_rng(131).integers(0, w.V, 20),
                                   edge_rows(w.V, 16384, 2), edge_rows(w.V, 256, 1)[::23]]))
    odW = od.kl_grad_W_rows(hs64, Ws64, ht64, Wt64, w.mask, w.T, c, True, vr)
    flush(f"  KL bwd qwen head (reverse), {act.size} active tokens")
    assert_rows("dh (sampled rows)", dh[rows], odh, rows)
    assert_rows("dW (sampled rows)", dW[vr], odW, vr)


def test_token_blocks_forward_and_backward():
    # 18750 active tokens of 20000: the KL forward in blocks of 3584 tokens (six blocks, set by
    # the workspace) and in its default one block, and the backward's own blocks (13824 tokens
    # at H = 256 beside the scratch, two blocks), both directions against the oracle
    w = wl.make(wl.scaled_spec(5, N=20000, H=256, V=2000, n_seq=40, len_lo=400, len_hi=600,
                               seed=161, prompt="none", T=0.8))
    w.mask[::16] = 0
    ht, Wt = _teacher(w, 128, 162)
    kb = _check_fwd(w, ht, Wt, block=3584)
    k1 = _fwd(w, ht, Wt)
    mism = sum(int((bits(a) != bits(b)).sum()) for a, b in zip(kb, k1))
    flush(f"  KL forward, six blocks against one: {mism} mismatches")
    assert mism == 0
    c = np.random.default_rng(164).uniform(0.5, 1.5, w.N).astype(np.float32)
    for reverse in (False, True):
        dh, dW = _bwd(w, ht, Wt, reverse, c)
        odh, odW = od.kl_grads(*(wl.as_f64(x) for x in (w.h, w.W, ht, Wt)), w.mask, w.T, c,
                               reverse)
        act = np.nonzero(w.mask)[0]
        flush(f"  KL bwd over token blocks, reverse={reverse}, {act.size} active")
        assert_rows("dh (every active row)", dh[act], odh[act], act)
        assert_rows("dW (every vocabulary row)", dW, odW)
        assert not dh[w.mask == 0].any()


def test_empty_and_all_masked():
    import linear_selected_token_amd as rlk
    w = wl.make(SMALL)
    ht, Wt = _teacher(w, 256, 132)
    # all tokens masked: every output is 0, dW_s is 0
    m0 = np.zeros(w.N, np.uint8)
    outs = _fwd(w, ht, Wt, mask=m0)
    assert not any(o.any() for o in outs)
    d = [_dev(x) for x in (w.h, w.W, ht, Wt)]
    z = torch.zeros(w.N, dtype=torch.float32, device=d[0].device)
    dh, dW = rlk.rlk_linear_kl_bwd(*d, _dev(m0), w.T, z + 1, z + 1, z, z, z)
    torch.cuda.synchronize()
    assert not dh.any() and not dW.any()
    # no tokens at all
    e = [x[:0] for x in d[:1]] + [d[1]] + [d[2][:0], d[3]]
    em = torch.zeros(0, dtype=torch.uint8, device=d[0].device)
    out0 = rlk.rlk_linear_kl_fwd(e[0], e[1], e[2], e[3], em, 1.0)
    assert all(o.numel() == 0 for o in out0)
    z0 = torch.zeros(0, dtype=torch.float32, device=d[0].device)
    dh0, dW0 = rlk.rlk_linear_kl_bwd(e[0], e[1], e[2], e[3], em, 1.0, None, z0, z0, z0, z0)
    torch.cuda.synchronize()
    assert dh0.numel() == 0 and not dW0.any()


def test_autograd_matches_direct_calls():
    import linear_selected_token_amd as rlk
    w = wl.make(wl.scaled_spec(5, N=300, H=256, V=2000, n_seq=2, len_lo=100, len_hi=200,
                               seed=133))
    ht, Wt = _teacher(w, 128, 134)
    d = [_dev(x) for x in (w.h, w.W, ht, Wt, w.mask)]
    hs = d[0].clone().requires_grad_(True)
    Ws = d[1].clone().requires_grad_(True)
    kf, kr = rlk.linear_kl(hs, Ws, d[2], d[3], d[4], w.T)
    cf = torch.from_numpy(np.random.default_rng(135).uniform(0.5, 1.5, w.N).astype(np.float32))
    cr = torch.from_numpy(np.random.default_rng(136).uniform(0.5, 1.5, w.N).astype(np.float32))
    cf, cr = cf.to(hs.device), cr.to(hs.device)
    ((cf * kf).sum() + (cr * kr).sum()).backward()
    _, kr0, ls, lt = rlk.rlk_linear_kl_fwd(*d, w.T)
    a, b = rlk.rlk_linear_kl_bwd(*d, w.T, cf, cr, ls, lt, kr0)
    torch.cuda.synchronize()
    assert torch.equal(hs.grad, a.to(torch.bfloat16))
    assert torch.equal(Ws.grad, b.to(torch.bfloat16))
    # against the oracle: the two directions' gradients add
    hs64, Ws64, ht64, Wt64 = (wl.as_f64(x) for x in (w.h, w.W, ht, Wt))
    f1 = od.kl_grads(hs64, Ws64, ht64, Wt64, w.mask, w.T, cf.cpu().numpy(), False)
    f2 = od.kl_grads(hs64, Ws64, ht64, Wt64, w.mask, w.T, cr.cpu().numpy(), True)
    act = np.nonzero(w.mask)[0]
    assert_rows("dh (both directions, every active row)", a.cpu().numpy()[act],
                (f1[0] + f2[0])[act], act)
    assert_rows("dW (both directions, every vocabulary row)", b.cpu().numpy(), f1[1] + f2[1])


@pytest.mark.parametrize("V", [1, 2, 129])
def test_tiny_vocabularies(V):
    # V = 1: both distributions are the same point mass, KL = 0 up to the rounding of the
    # exponents; V = 2 and 129: ragged columns
    w = wl.make(wl.scaled_spec(2, N=70, H=64, V=V, n_seq=1, len_lo=70, len_hi=70,
                               prompt="none", seed=140 + V))
    ht, Wt = _teacher(w, 128, 141 + V)
    kf, kr, _, _ = _check_fwd(w, ht, Wt)
    if V == 1:
        assert np.abs(kf).max() < 1e-6 and np.abs(kr).max() < 1e-6
