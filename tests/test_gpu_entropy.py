"""Entropy forward and entropy-bonus backward against the float64 oracle (needs an MI355X).

rlk_linear_logp_fwd_entropy returns logp and lse bit-identical to rlk_linear_logp_fwd and,
per active token, the entropy of softmax(h W^T / T).  Gates: logp and lse as for the plain
forward; |dH| <= 1e-3 absolute against the oracle (H = lse - E_p[z], so an error of delta
in every logit moves it by at most 2 delta, the bound the logp gate already puts on lse);
a token's entropy is bit-identical in any batch; 0 at inactive tokens.

rlk_linear_logp_bwd_entropy: gradients of L = -sum_t mask_t (adv_t logp_t + c_t H_t) within
rel-L2 1e-2 of the oracle's, a token's dL/dh row bit-identical across batch layouts, and
with c = 0 exactly the plain backward."""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (assert_rows, assert_tiles, bits, edge_rows, flush, oracle_inputs, run_bwd,
                      run_fwd, sample_rows, upload)

pytestmark = pytest.mark.gpu

MAX_ABS_DH = 1e-3
HERE = os.path.dirname(os.path.abspath(__file__))


def _run(w, d=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    lp, lse, ent = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    torch.cuda.synchronize()
    return lp.cpu().numpy(), lse.cpu().numpy(), ent.cpu().numpy()


def _check(w, ent, rows=None, tol=MAX_ABS_DH):
    h64, W64 = oracle_inputs(w)
    act = w.mask.astype(bool)
    if rows is None:
        oe = oracle.entropy(h64, W64, w.mask, w.T)
        assert not ent[~act].any()
        d = np.abs(ent[act] - oe[act])
    else:
        oe = oracle.entropy(h64[rows], W64, np.ones(rows.size, np.uint8), w.T)
        d = np.abs(ent[rows] - oe)
    flush(f"  {w.spec.name} N={w.N} H={w.H} V={w.V} {w.dtype} T={w.T}: max_abs_dH={d.max():.3e} "
          f"over {d.size} active tokens")
    assert np.all(np.isfinite(ent[act]))
    assert d.max() <= tol
    return d.max()


def _same_as_plain(w, lp, lse, d=None):
    ref_lp, ref_lse = run_fwd(w, d)
    act = w.mask.astype(bool)
    assert np.array_equal(bits(lp), bits(ref_lp))
    assert np.array_equal(bits(lse[act]), bits(ref_lse[act]))


SPECS = [
    wl.scaled_spec(1, N=300, H=128, V=777, n_seq=3, len_lo=50, len_hi=150, prompt="floor_half",
                   seed=91, T=0.8),                                          # fp32, ragged V
    wl.scaled_spec(2, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=92, T=0.7),
    wl.scaled_spec(2, N=1100, H=256, V=2 * 256 * 3 + 100, n_seq=5, len_lo=100, len_hi=400,
                   prompt="none", seed=93),                                  # 5 token tiles
]


@pytest.mark.parametrize("k", range(len(SPECS)))
def test_small_full(k):
    w = wl.make(SPECS[k])
    d = upload(w)
    lp, lse, ent = _run(w, d)
    _check(w, ent, tol=1e-4 if w.dtype == "fp32" else MAX_ABS_DH)
    _same_as_plain(w, lp, lse, d)


def test_closed_forms():
    # W = 0: every token's distribution is uniform, H = log V
    w = wl.make(SPECS[1])
    w.W[:] = 0
    _, _, ent = _run(w)
    act = w.mask.astype(bool)
    assert np.abs(ent[act] - math.log(w.V)).max() < 1e-5
    # a one-entry vocabulary: H = 0 up to the rounding of one exponent
    w1 = wl.make(wl.scaled_spec(2, N=40, H=64, V=1, n_seq=1, len_lo=40, len_hi=40,
                                prompt="none", seed=94))
    _, _, e1 = _run(w1)
    assert np.all(e1 >= 0) and np.all(e1 < 1e-6)


def test_peaked_distributions():
    # logits scaled 24x: most of the mass on a few entries, most exponents underflow
    w = wl.make(SPECS[1])
    w.h = wl.bf16_bits(wl.bf16_to_f32(w.h) * np.float32(24.0))
    d = upload(w)
    lp, lse, ent = _run(w, d)
    _check(w, ent)
    _same_as_plain(w, lp, lse, d)
    assert np.all(ent[w.mask.astype(bool)] >= 0)


def test_batch_invariance():
    w = wl.make(SPECS[2])
    _, _, ent = _run(w)
    act = np.nonzero(w.mask)[0]
    # a reversed subset of the tokens, in a batch of its own with other tokens masked
    sel = act[::-3].copy()
    sub = dataclasses.replace(w, h=np.ascontiguousarray(w.h[sel]), targets=w.targets[sel].copy(),
                              mask=w.mask[sel].copy(), adv=w.adv[sel], u=w.u[sel],
                              seq_id=w.seq_id[sel], pos=w.pos[sel])
    sub.mask[1::4] = 0
    _, _, es = _run(sub)
    keep = sub.mask.astype(bool)
    mism = int((bits(es[keep]) != bits(ent[sel][keep])).sum())
    flush(f"  entropy invariance: {mism} mismatches over {int(keep.sum())} tokens")
    assert mism == 0
    assert not es[~keep].any()


def test_qwen_head_sampled():
    # the Qwen3-8B LM head (H=4096, V=151936), 1024 tokens, oracle on sampled rows
    spec = wl.scaled_spec(2, N=1024, n_seq=4, len_lo=200, len_hi=300, seed=95)
    w = wl.make(spec)
    d = upload(w)
    lp, lse, ent = _run(w, d)
    _check(w, ent, rows=sample_rows(w, 24, seed=95))
    _same_as_plain(w, lp, lse, d)


def _full_size():
    # the benchmark step: 16384 tokens, the Qwen3-8B head, T = 0.7, stored sampled targets
    flush("qwen3-8b-head N=16384 T=0.7: generating inputs")
    targets = np.load(os.path.join(HERE, "golden", "cfg3_sampled_targets.npy"))
    return wl.with_targets(wl.make(3), targets)


def test_full_size_sampled():
    w = _full_size()
    d = upload(w)
    lp, lse, ent = _run(w, d)
    _check(w, ent, rows=sample_rows(w, 24, seed=2))
    _same_as_plain(w, lp, lse, d)


# ------------------------------------------------------------------ entropy-bonus backward

def _ent_coef(w, seed, lo=0.5, hi=1.5):
    return np.random.default_rng(seed).uniform(lo, hi, w.N).astype(np.float32)


def _run_bwd(w, c, d=None, adv=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    dev = d["h"].device
    _, lse, ent = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    a = d["adv"] if adv is None else torch.from_numpy(adv).to(dev)
    dh, dW = rlk.rlk_linear_logp_bwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T, a,
                                             torch.from_numpy(c).to(dev), lse, ent)
    torch.cuda.synchronize()
    return dh, dW


def _bwd_full_compare(w, c, adv=None):
    dh, dW = _run_bwd(w, c, adv=adv)
    dh, dW = dh.cpu().numpy(), dW.cpu().numpy()
    h64, W64 = oracle_inputs(w)
    odh, odW = oracle.linear_logp_entropy_grads(h64, W64, w.targets, w.mask, w.T,
                                                w.adv if adv is None else adv, c)
    act = np.nonzero(w.mask)[0]
    flush(f"  entropy bwd {w.spec.name} N={w.N} H={w.H} V={w.V} "
          f"adv={'0' if adv is not None else 'w'}")
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert_tiles("dW", dW, odW)
    assert not dh[w.mask == 0].any()


BWD_SMALL = wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=97,
                           T=0.8)


def test_bwd_small_full():
    w = wl.make(BWD_SMALL)
    _bwd_full_compare(w, _ent_coef(w, 1))
    # the entropy term alone
    _bwd_full_compare(w, _ent_coef(w, 2), adv=np.zeros(w.N, np.float32))


def test_bwd_two_chunks_ragged():
    import re
    import linear_selected_token_amd as rlk
    m = re.search(r"bwd chunk (\d+), dh split at (\d+)", rlk.build_info())
    chunk, split = int(m.group(1)), int(m.group(2))
    w = wl.make(wl.scaled_spec(5, N=300, H=256, V=chunk + split + 300, n_seq=2, len_lo=100,
                               len_hi=200, seed=98))
    _bwd_full_compare(w, _ent_coef(w, 3))


def test_bwd_zero_coefficient_is_plain_backward():
    w = wl.make(BWD_SMALL)
    d = upload(w)
    dh, dW = _run_bwd(w, np.zeros(w.N, np.float32), d)
    _, _, dh0, dW0 = run_bwd(w, d)
    assert torch.equal(dh, dh0) and torch.equal(dW, dW0)


def test_bwd_dh_invariance():
    fam = wl.Family(BWD_SMALL)
    base = fam.batch()
    c_of = {}
    r = np.random.default_rng(4)
    for k in base.key():
        c_of[k] = np.float32(r.uniform(0.5, 1.5))

    def coef(w):
        return np.array([c_of.get(k, np.float32(0)) for k in w.key()], np.float32)

    dh, _ = _run_bwd(base, coef(base))
    dh = dh.cpu().numpy()
    ref = {k: dh[i] for i, k in enumerate(base.key()) if base.mask[i]}
    for w in (fam.alone(1), fam.shuffled(7), fam.padded(8)):
        dh2, _ = _run_bwd(w, coef(w))
        dh2 = dh2.cpu().numpy()
        for i, k in enumerate(w.key()):
            if k[0] >= 0 and w.mask[i]:
                assert np.array_equal(bits(dh2[i]), bits(ref[k])), k


def test_bwd_qwen_head_sampled():
    # the Qwen3-8B LM head, 1024 tokens: sampled dh rows and dW rows against the oracle
    w = wl.make(wl.scaled_spec(5, N=1024, n_seq=4, len_lo=200, len_hi=300, seed=99))
    c = _ent_coef(w, 5)
    dh, dW = _run_bwd(w, c)
    h64, W64 = oracle_inputs(w)
    rows = sample_rows(w, 16, seed=99)
    odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows, ent_coef=c)
    assert_rows("entropy bwd qwen head dh (sampled rows)",
                dh[torch.from_numpy(rows).to(dh.device)].cpu().numpy(), odh, rows)
    _, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    oent = oracle.entropy(h64, W64, w.mask, w.T)
    act = np.nonzero(w.mask)[0]
    vr = np.unique(np.concatenate([w.targets[act[:8]], edge_rows(w.V, 16384, 2),
                                   edge_rows(w.V, 256, 1)[::17],
                                   np.random.default_rng(6).integers(0, w.V, 16)]))
    odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, w.adv, vr, lse=olse,
                             ent_coef=c, entropy_=oent)
    assert_rows("entropy bwd qwen head dW (sampled rows)",
                dW[torch.from_numpy(vr).to(dW.device)].cpu().numpy(), odW, vr)


def test_bwd_full_size_sampled():
    # the benchmark step: sampled dh rows against the oracle, and the columns of dW sum to ~0
    # (every row of dL/dz does)
    w = _full_size()
    c = _ent_coef(w, 7, lo=0.005, hi=0.02)
    dh, dW = _run_bwd(w, c)
    h64, W64 = oracle_inputs(w)
    rows = sample_rows(w, 12, seed=7)
    odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows, ent_coef=c)
    assert_rows("entropy bwd full size dh (sampled rows)",
                dh[torch.from_numpy(rows).to(dh.device)].cpu().numpy(), odh, rows)
    colsum = dW.double().sum(0).abs().max().item()
    scale = dW.double().abs().sum(0).max().item()
    assert colsum <= 1e-3 * scale


def test_empty_and_all_masked():
    import linear_selected_token_amd as rlk
    w = wl.make(SPECS[1])
    d = upload(w)
    d["mask"].zero_()
    lp, lse, ent = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    c = torch.ones(w.N, dtype=torch.float32, device=d["h"].device)
    dh, dW = rlk.rlk_linear_logp_bwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                             d["adv"], c, lse, ent)
    torch.cuda.synchronize()
    assert not lp.any() and not lse.any() and not ent.any() and not dh.any() and not dW.any()
    e = d["h"][:0]
    lp0, _, ent0 = rlk.rlk_linear_logp_fwd_entropy(e, d["W"], d["targets"][:0], d["mask"][:0],
                                                   1.0)
    assert lp0.numel() == 0 and ent0.numel() == 0


def test_autograd_matches_direct_calls():
    import linear_selected_token_amd as rlk
    w = wl.make(BWD_SMALL)
    d = upload(w)
    h = d["h"].clone().requires_grad_(True)
    W = d["W"].clone().requires_grad_(True)
    lp, ent = rlk.linear_logp_entropy(h, W, d["targets"], d["mask"], w.T)
    m = d["mask"].float()
    c = torch.from_numpy(_ent_coef(w, 9)).to(h.device)
    loss = -(m * (d["adv"] * lp + c * ent)).sum()
    loss.backward()
    dh, dW = _run_bwd(w, c.cpu().numpy(), d)
    assert torch.equal(h.grad, dh.to(torch.bfloat16))
    assert torch.equal(W.grad, dW.to(torch.bfloat16))
