"""Shared helpers of the GPU tests: upload a workload, call the library through the
binding, compare with the oracle."""
import numpy as np
import torch

import workloads as wl

MAX_ABS_DLOGP = 1e-3   # gate on active tokens against the float64 oracle
GRAD_REL_L2 = 1e-2     # gate on dL/dh and dL/dW


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda", 0)


def upload(w: wl.Workload, dev=None):
    dev = dev or device()

    def mat(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    return dict(h=mat(w.h), W=mat(w.W), targets=torch.from_numpy(w.targets).to(dev),
                mask=torch.from_numpy(w.mask).to(dev),
                adv=torch.from_numpy(w.adv).to(dev))


def run_fwd(w: wl.Workload, d=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    torch.cuda.synchronize()
    return logp.cpu().numpy(), lse.cpu().numpy()


def run_bwd(w: wl.Workload, d=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    dh, dW = rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, d["adv"], lse)
    torch.cuda.synchronize()
    return logp, lse, dh, dW


def oracle_inputs(w: wl.Workload):
    return wl.as_f64(w.h), wl.as_f64(w.W)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.int32)


def sample_rows(w: wl.Workload, k: int, seed: int):
    """k active rows: the first and last active tokens plus seeded random ones."""
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(seed)
    pick = set([int(act[0]), int(act[-1])])
    pick.update(int(x) for x in r.choice(act, size=min(k, act.size), replace=False))
    return np.array(sorted(pick))[:max(k, 2)]


def flush(msg: str) -> None:
    print(msg, flush=True)
