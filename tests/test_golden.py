"""The stored sampled targets of the N=16384, T=0.7 workload are in step with the input
generator and with the oracle's sampler (no GPU)."""
import hashlib
import json
import os

import numpy as np

import oracle
import workloads as wl

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_cfg3_targets_match_generator_and_oracle():
    meta = json.load(open(os.path.join(HERE, "cfg3_sampled_targets.json")))
    targets = np.load(os.path.join(HERE, "cfg3_sampled_targets.npy"))
    w = wl.make(3)
    assert meta["N"] == w.N == targets.size and meta["n_active"] == w.n_active
    assert _digest(w.h) == meta["h_sha256"]
    assert _digest(w.W) == meta["W_sha256"]
    assert _digest(w.u) == meta["u_sha256"]
    assert _digest(targets) == meta["targets_sha256"]
    act = np.nonzero(w.mask)[0]
    # prompt tokens keep their uniform targets
    inact = np.nonzero(w.mask == 0)[0]
    assert np.array_equal(targets[inact], w.targets[inact])
    # a few active rows re-sampled by the oracle
    rows = act[[0, 1, act.size // 2, act.size - 1]]
    W64 = wl.as_f64(w.W)
    y = oracle.sample_targets(wl.as_f64(w.h[rows]), W64, w.T, w.u[rows])
    assert np.array_equal(y, targets[rows])
    assert targets.min() >= 0 and targets.max() < w.V
