"""Write the sampled targets of the N=16384, T=0.7 Qwen3-8B-head workload.

That workload's targets are drawn from each row's softmax as the oracle computes it, by
inverse-CDF with the per-token uniforms of the input generator; prompt tokens keep their
uniform targets.  Only the oracle computes the softmax here.  Output:
``cfg3_sampled_targets.npy`` (int32 [16384]) and ``cfg3_sampled_targets.json`` (digests of
the inputs it was computed from, so a test can tell whether it is still in step with the
generator).  Run from the repository root: ``python tests/golden/make_sampled_targets.py``.
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main() -> None:
    spec = wl.CONFIGS[3]
    w = wl.Family(spec).batch()
    act = np.nonzero(w.mask)[0]
    t0 = time.time()
    W64 = wl.as_f64(w.W)
    y = oracle.sample_targets(wl.as_f64(w.h[act]), W64, spec.T, w.u[act], block=256)
    targets = w.targets.copy()
    targets[act] = y.astype(np.int32)
    np.save(os.path.join(HERE, "cfg3_sampled_targets.npy"), targets)
    meta = {"spec": spec.name, "seed": spec.seed, "N": spec.N, "n_active": int(act.size),
            "h_sha256": digest(w.h), "W_sha256": digest(w.W), "u_sha256": digest(w.u),
            "targets_sha256": digest(targets), "seconds": round(time.time() - t0, 1)}
    with open(os.path.join(HERE, "cfg3_sampled_targets.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(meta)


if __name__ == "__main__":
    main()
