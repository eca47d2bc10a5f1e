"""Bitwise batch invariance of the HIP path (needs an MI355X).

A token's logp and lse (and, from the entropy forward, its entropy) must be bit-identical whether its sequence is scored alone, in
the full batch, in shuffled order, with extra padding, with its prompt tokens also
active, on a repeat run or on another stream (RL-Kernel integration roadmap for vime,
"Consistency Contract": same-backend bitwise stability across batch size, row position,
dense vs indexed rows, sparse-row density and stream/repeat runs)."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bits, flush, run_fwd, upload

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _keyed(w, *outs):
    out = {}
    for i, k in enumerate(w.key()):
        if k[0] < 0 or not w.mask[i]:
            continue
        out[k] = tuple(int(bits(o[i:i + 1])[0]) for o in outs)
    return out


def _fwd_entropy(w, d=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    outs = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in outs)


def _mismatches(ref, got):
    n = 0
    for k, v in got.items():
        if k in ref and ref[k] != v:
            n += 1
    return n


def _sweep(fam, n_alone, label, fwd=run_fwd):
    base = fam.batch()
    ref = _keyed(base, *fwd(base))
    cases = []
    for s in range(min(n_alone, fam.n_seq)):
        cases.append((f"alone {s}", fam.alone(s)))
    for k in range(3):
        cases.append((f"shuffle {k}", fam.shuffled(100 + k)))
        cases.append((f"padded {k}", fam.padded(200 + k)))
    cases.append(("all active", fam.all_active()))
    cases.append(("subset", fam.subset(list(range(0, fam.n_seq, 3)))))
    total = 0
    checked = 0
    for name, w in cases:
        got = _keyed(w, *fwd(w))
        common = [k for k in got if k in ref]
        m = _mismatches(ref, got)
        total += m
        checked += len(common)
        if m:
            flush(f"  {label} {name}: {m} mismatches of {len(common)}")
    # repeat runs and a second stream on the full batch
    d = upload(base)
    import linear_selected_token_amd as rlk
    call = (rlk.rlk_linear_logp_fwd if fwd is run_fwd else rlk.rlk_linear_logp_fwd_entropy)
    outs = []
    for k in range(3):
        outs.append(call(d["h"], d["W"], d["targets"], d["mask"], base.T))
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        outs.append(call(d["h"], d["W"], d["targets"], d["mask"], base.T))
    torch.cuda.synchronize()
    for o in outs:
        got = _keyed(base, *(x.cpu().numpy() for x in o))
        total += _mismatches(ref, got)
        checked += len(got)
    flush(f"  {label}: {total} mismatches over {checked} active-token comparisons")
    return total


def test_invariance_small():
    fam = wl.Family(wl.scaled_spec(2, N=1500, H=256, V=2000, n_seq=8, len_lo=64, len_hi=400,
                                   seed=90, T=0.7))
    assert _sweep(fam, 8, "small") == 0


def test_invariance_config3_full():
    """The N=16384, T=0.7 workload with its sampled targets: every sequence alone, the full
    batch, shuffles, paddings, all-active density, repeats and a second stream."""
    fam = wl.Family(wl.CONFIGS[3])
    fam.use_targets(np.load(os.path.join(HERE, "golden", "cfg3_sampled_targets.npy")))
    assert _sweep(fam, fam.n_seq, "config3") == 0


def test_entropy_invariance_small():
    # logp, lse and entropy of the entropy forward, over the same kinds of layouts
    fam = wl.Family(wl.scaled_spec(2, N=1500, H=256, V=2000, n_seq=8, len_lo=64, len_hi=400,
                                   seed=91, T=0.7))
    assert _sweep(fam, 8, "entropy small", fwd=_fwd_entropy) == 0


def test_entropy_invariance_config3():
    """The entropy forward on the N=16384 workload: 8 sequences alone, shuffles, paddings,
    all-active density, a subset, repeats and a second stream."""
    fam = wl.Family(wl.CONFIGS[3])
    fam.use_targets(np.load(os.path.join(HERE, "golden", "cfg3_sampled_targets.npy")))
    assert _sweep(fam, 8, "entropy config3", fwd=_fwd_entropy) == 0


def _fused_keyed(w):
    """logp and lse bits and a digest of the dL/dh row's bytes of every active token of w, keyed
    by (sequence, position), from one fused forward + backward call."""
    import hashlib
    import linear_selected_token_amd as rlk
    d = upload(w)
    logp, lse, dh, _ = rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                                   d["adv"])
    torch.cuda.synchronize()
    lp, ls, dh = logp.cpu().numpy(), lse.cpu().numpy(), dh.cpu().numpy()
    out = {}
    for i, k in enumerate(w.key()):
        if k[0] < 0 or not w.mask[i]:
            continue
        out[k] = (int(bits(lp[i:i + 1])[0]), int(bits(ls[i:i + 1])[0]),
                  hashlib.sha1(dh[i].tobytes()).hexdigest())
    return out


def test_fused_invariance_config3():
    """The fused forward + backward on the N=16384 workload (four token blocks of the default
    workspace): each active token's logp, lse and dL/dh row bit-identical with 8 sequences alone
    (one block each), shuffled, padded, all-active (five blocks) and a subset."""
    fam = wl.Family(wl.CONFIGS[3])
    fam.use_targets(np.load(os.path.join(HERE, "golden", "cfg3_sampled_targets.npy")))
    ref = _fused_keyed(fam.batch())
    cases = [(f"alone {s}", fam.alone(s)) for s in range(8)]
    cases += [("shuffle", fam.shuffled(300)), ("padded", fam.padded(301)),
              ("all active", fam.all_active()),
              ("subset", fam.subset(list(range(0, fam.n_seq, 3))))]
    total = checked = 0
    for name, w in cases:
        got = _fused_keyed(w)
        m = _mismatches(ref, got)
        total += m
        checked += sum(1 for k in got if k in ref)
        if m:
            flush(f"  fused {name}: {m} mismatches")
    flush(f"  fused config3: {total} mismatches over {checked} active-token comparisons "
          "(logp, lse and the dL/dh row)")
    assert checked > 0 and total == 0

