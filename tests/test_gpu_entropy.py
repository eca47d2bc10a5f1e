"""Entropy forward against the float64 oracle (needs an MI355X).

rlk_linear_logp_fwd_entropy returns logp and lse bit-identical to rlk_linear_logp_fwd and,
per active token, the entropy of softmax(h W^T / T).  Gates: logp and lse as for the plain
forward; |dH| <= 1e-3 absolute against the oracle (H = lse - E_p[z], so an error of delta
in every logit moves it by at most 2 delta, the bound the logp gate already puts on lse);
a token's entropy is bit-identical in any batch; 0 at inactive tokens."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (MAX_ABS_DLOGP, bits, flush, oracle_inputs, run_fwd, sample_rows,
                      upload)

pytestmark = pytest.mark.gpu

MAX_ABS_DH = 1e-3


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


def test_full_size_sampled():
    # the full-size step (16384 tokens, the Qwen3-8B head), oracle on sampled rows
    flush("config 2: generating inputs")
    w = wl.make(2)
    d = upload(w)
    lp, lse, ent = _run(w, d)
    _check(w, ent, rows=sample_rows(w, 24, seed=2))
    _same_as_plain(w, lp, lse, d)
