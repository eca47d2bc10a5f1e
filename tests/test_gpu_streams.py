"""Calls from several host threads at once, each on a stream of its own with its own
workspace (needs an MI355X).

The library keeps no state between calls beyond read-only device properties, so concurrent
calls on different streams must each give the bits the same call gives alone.  Four threads
run the fused forward + backward and the two calls on four workloads at the same time; every
output is compared bit for bit with a sequential run."""
import threading

import pytest
import torch

import workloads as wl
from gpu_util import flush, upload

pytestmark = pytest.mark.gpu

SPECS = [wl.scaled_spec(5, N=1500, H=512, V=5000, n_seq=6, len_lo=100, len_hi=400,
                        seed=201 + k, T=0.6 + 0.2 * k) for k in range(4)]


def _step(w, d):
    import linear_selected_token_amd as rlk
    out = list(rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                           d["adv"]))
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    out += [logp, lse]
    out += list(rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, d["adv"],
                                        lse))
    return out


def test_concurrent_threads_and_streams():
    ws = [wl.make(s) for s in SPECS]
    ds = [upload(w) for w in ws]
    ref = []
    for w, d in zip(ws, ds):
        ref.append([t.clone() for t in _step(w, d)])
    torch.cuda.synchronize()

    got = [None] * len(ws)
    errors = []
    start = threading.Barrier(len(ws))

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(3):  # repeated, so that the threads' launches interleave
                    out = _step(ws[k], ds[k])
                s.synchronize()
                got[k] = [t.clone() for t in out]
                s.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(ws))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    names = ("fused logp", "fused lse", "fused dh", "fused dW", "logp", "lse", "dh", "dW")
    for k in range(len(ws)):
        for name, a, b in zip(names, got[k], ref[k]):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (k, name)
    flush(f"  {len(ws)} threads x 3 steps on their own streams: every output bit-identical to "
          "the sequential run")
