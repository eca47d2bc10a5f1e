"""Log-prob from existing logits against the float64 oracle (needs an MI355X).

Gates: max |dlogp| <= 1e-3 over active tokens; a token's logp and lse are bit-identical
whatever else is in the batch; an out-of-range target gives NaN."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import MAX_ABS_DLOGP, bits, device, flush

pytestmark = pytest.mark.gpu


def _inputs(seed, N, V, dtype, ld=None, scale=3.0, active=0.7):
    r = np.random.default_rng(seed)
    z = wl.logits_rows(seed, N, V, scale, dtype, ld=ld)
    y = r.integers(0, V, N).astype(np.int32)
    m = (r.random(N) < active).astype(np.uint8)
    return z, y, m


def _gpu(z, y, m, V, T):
    import linear_selected_token_amd as rlk
    dev = device()
    if z.dtype == np.uint16:
        lg = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        lg = torch.from_numpy(z).to(dev)
    logp, lse = rlk.rlk_logp_from_logits(lg, torch.from_numpy(y).to(dev),
                                         torch.from_numpy(m).to(dev), T, V=V)
    torch.cuda.synchronize()
    return logp.cpu().numpy(), lse.cpu().numpy()


def _oracle(z, y, m, V, T, rows=None):
    z64 = wl.as_f64(z[:, :V] if rows is None else z[rows, :V])
    if rows is None:
        return oracle.logp_from_logits(z64, y, m, T)
    return oracle.logp_from_logits(z64, y[rows], m[rows], T)


@pytest.mark.parametrize("dtype,N,V,ld,T", [
    ("bf16", 300, 1000, None, 1.0),
    ("bf16", 257, 5000, 5008, 0.7),     # padded rows, ragged last column
    ("fp32", 200, 3001, 3004, 1.3),     # odd V, fp32
    ("bf16", 64, 1, 8, 1.0),            # a one-entry vocabulary
    ("fp32", 33, 128, None, 0.5),       # exactly one column
])
def test_small_full(dtype, N, V, ld, T):
    z, y, m = _inputs(11 + N, N, V, dtype, ld=ld)
    logp, lse = _gpu(z, y, m, V, T)
    olp, olse = _oracle(z, y, m, V, T)
    act = m != 0
    err = float(np.max(np.abs(logp[act] - olp[act]))) if act.any() else 0.0
    flush(f"  logits {dtype} N={N} V={V} ld={ld or V} T={T}: max_abs_dlogp={err:.3e}")
    assert err <= MAX_ABS_DLOGP
    assert np.max(np.abs(lse[act] - olse[act])) <= MAX_ABS_DLOGP
    assert not logp[~act].any() and not lse[~act].any()


def test_batch_invariance_and_out_of_range_target():
    N, V, T = 512, 20000, 0.8
    z, y, m = _inputs(5, N, V, "bf16")
    m[:] = 1
    logp, lse = _gpu(z, y, m, V, T)
    # the same rows scored in a smaller batch, in reverse order, next to masked rows
    sel = np.arange(N - 1, 0, -3)
    sz, sy, sm = z[sel], y[sel].copy(), m[sel].copy()
    sm[::5] = 0
    sl, ss = _gpu(np.ascontiguousarray(sz), sy, sm, V, T)
    act = sm != 0
    mism = int((bits(sl[act]) != bits(logp[sel][act])).sum() +
               (bits(ss[act]) != bits(lse[sel][act])).sum())
    flush(f"  logits invariance: {mism} mismatches over {int(act.sum())} tokens")
    assert mism == 0
    # out-of-range targets: NaN logp, finite lse
    y2 = y.copy()
    y2[:4] = [-1, V, V + 7, 2 ** 30]
    lp2, ls2 = _gpu(z, y2, m, V, T)
    assert np.isnan(lp2[:4]).all() and np.isfinite(ls2[:4]).all()
    assert (bits(lp2[4:]) == bits(logp[4:])).all()


def test_qwen_vocab_sampled_rows():
    # the Qwen3-8B vocabulary, bf16 logits; the oracle scores a sample of rows
    N, V, T = 1024, 151936, 0.7
    z, y, m = _inputs(9, N, V, "bf16", scale=2.5)
    logp, lse = _gpu(z, y, m, V, T)
    act = np.nonzero(m)[0]
    rows = np.unique(np.concatenate([act[:3], act[-3:], np.random.default_rng(1).choice(act, 40)]))
    olp, olse = _oracle(z, y, m, V, T, rows=rows)
    err = float(np.max(np.abs(logp[rows] - olp)))
    flush(f"  logits bf16 N={N} V={V}: max_abs_dlogp={err:.3e} over {rows.size} sampled rows")
    assert err <= MAX_ABS_DLOGP
    assert np.max(np.abs(lse[rows] - olse)) <= MAX_ABS_DLOGP
