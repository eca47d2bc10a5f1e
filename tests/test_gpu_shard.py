"""Vocabulary-parallel forward on one GPU (needs an MI355X).

The LM head is cut into vocabulary shards on 128-entry column boundaries.  Each shard's
partial statistics go into the full-vocabulary partial arrays through
rlk_linear_logp_partials_shard, and one fixed-order merge gives logp and lse.  The result
must be bit-identical to the single-call forward: the merge is the same, and each column's
statistics come from the same arithmetic whichever call computes them.  Shards run in
shuffled order, some on a second stream."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import MAX_ABS_DLOGP, bits, flush, oracle_inputs, run_fwd, upload

pytestmark = pytest.mark.gpu


def _sharded_fwd(w, d, bounds, order, streams):
    import linear_selected_token_amd as rlk
    N, V = w.N, w.V
    bufs = rlk.ForwardBuffers(N, V, d["h"].device)
    rlk.rlk_compact_active(d["mask"], bufs.idx, bufs.n_active, bufs.target_logit, bufs.logp,
                           bufs.lse)
    main = torch.cuda.current_stream()
    done = []
    for n, s in enumerate(order):
        lo, hi = bounds[s], bounds[s + 1]
        st = streams[n % len(streams)]
        st.wait_stream(main)
        with torch.cuda.stream(st):
            rlk.rlk_linear_logp_partials_shard(d["h"], d["W"][lo:hi], d["targets"], bufs.idx,
                                               bufs.n_active, lo, V, w.T, bufs.part_max,
                                               bufs.part_sum, bufs.target_logit)
        done.append(st)
    for st in done:
        main.wait_stream(st)
    rlk.rlk_linear_logp_merge(bufs.part_max, bufs.part_sum, bufs.target_logit, bufs.idx,
                              bufs.n_active, N, V, bufs.logp, bufs.lse)
    torch.cuda.synchronize()
    return bufs.logp[:N].cpu().numpy(), bufs.lse[:N].cpu().numpy()


def _bounds(V, cuts):
    return [0] + [128 * c for c in cuts] + [V]


CASES = [
    # (spec, column cuts) -- cuts at 128-entry columns, several not on 256-entry tile edges
    (wl.scaled_spec(1, seed=71), [1, 3, 5]),                              # fp32, V=1000
    (wl.scaled_spec(2, N=700, V=5000, n_seq=4, len_lo=100, len_hi=250, seed=72), [3, 17, 18]),
    (wl.scaled_spec(3, N=900, V=9000, n_seq=6, len_lo=100, len_hi=200, seed=73,
                    targets="uniform"), [1, 2, 33, 50]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_shards_merge_bit_identical(case):
    spec, cuts = CASES[case]
    w = wl.make(spec)
    d = upload(w)
    ref_logp, ref_lse = run_fwd(w, d)
    bounds = _bounds(w.V, cuts)
    order = [int(x) for x in np.random.default_rng(case).permutation(len(bounds) - 1)]
    side = torch.cuda.Stream()
    logp, lse = _sharded_fwd(w, d, bounds, order, [torch.cuda.current_stream(), side])
    act = w.mask != 0
    nl = int((bits(logp) != bits(ref_logp))[act].sum())
    ns = int((bits(lse) != bits(ref_lse))[act].sum())
    flush(f"  N={w.N} H={w.H} V={w.V} {w.dtype} shards {bounds} order {order}: "
          f"{nl} logp / {ns} lse mismatches over {int(act.sum())} active tokens")
    assert nl == 0 and ns == 0
    assert not logp[~act].any() and not lse[~act].any()
    # and the sharded result is the oracle's, like the single call
    h64, W64 = oracle_inputs(w)
    olp, _ = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    assert np.max(np.abs(logp[act] - olp[act])) <= MAX_ABS_DLOGP


def test_qwen_head_sampled_rows_sharded():
    # the Qwen3-8B head shape, sharded 8 ways at uneven column boundaries
    spec = wl.scaled_spec(2, N=1024, n_seq=4, len_lo=200, len_hi=300, seed=74)
    w = wl.make(spec)
    d = upload(w)
    ref_logp, ref_lse = run_fwd(w, d)
    J = (w.V + 127) // 128
    cuts = sorted({int(x) for x in np.linspace(0, J, 9)[1:-1] + np.arange(7)})
    bounds = _bounds(w.V, cuts)
    order = [int(x) for x in np.random.default_rng(7).permutation(len(bounds) - 1)]
    logp, lse = _sharded_fwd(w, d, bounds, order, [torch.cuda.current_stream()])
    act = w.mask != 0
    nl = int((bits(logp) != bits(ref_logp))[act].sum())
    flush(f"  N={w.N} H={w.H} V={w.V} shards {len(bounds) - 1}: {nl} logp mismatches over "
          f"{int(act.sum())} active tokens")
    assert nl == 0
    assert int((bits(lse) != bits(ref_lse))[act].sum()) == 0
