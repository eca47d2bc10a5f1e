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


def row_rel_l2(got, ref):
    """rel-L2 of every row of a 2-D gradient against its reference row (float64); a row whose
    reference is exactly zero gets the absolute norm of the computed row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_rows(name, got, ref, row_ids=None, gate=GRAD_REL_L2):
    """Gate every row of a gradient on its own rel-L2 (not only the whole tensor's): an error
    confined to a few rows, a piece boundary or one tile cannot hide in the total.  Prints
    the worst row."""
    e = row_rel_l2(got, ref)
    if e.size == 0:
        return e
    k = int(np.argmax(e))
    rid = k if row_ids is None else int(np.asarray(row_ids)[k])
    flush(f"  {name}: worst row {rid} relL2 {e[k]:.3e} over {e.size} rows "
          f"(whole tensor {rel_l2(got, ref):.3e})")
    assert e[k] <= gate, (name, rid, float(e[k]))
    return e


def assert_tiles(name, got, ref, tile=256, gate=GRAD_REL_L2):
    """Gate every tile x tile block of a 2-D gradient on its own rel-L2 (the kernels' output
    tiles are 256 x 256); a block whose reference is exactly zero gets the absolute norm of the
    computed block, as rows do in row_rel_l2.  Prints the worst block."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst, at = 0.0, (0, 0)
    for r0 in range(0, ref.shape[0], tile):
        for c0 in range(0, ref.shape[1], tile):
            g = got[r0:r0 + tile, c0:c0 + tile]
            rb = ref[r0:r0 + tile, c0:c0 + tile]
            e = rel_l2(g, rb) if rb.any() else float(np.linalg.norm(g))
            if e > worst:
                worst, at = e, (r0, c0)
    flush(f"  {name}: worst {tile}x{tile} block at {at} relL2 {worst:.3e}")
    assert worst <= gate, (name, at, worst)
    return worst


def edge_rows(n, step, k=1):
    """Indices next to every multiple of ``step`` below n (m - k .. m + k - 1), plus the
    first and last index: the rows on tile, piece and chunk boundaries."""
    out = {0, n - 1}
    for m in range(step, n, step):
        out.update(range(max(0, m - k), min(n, m + k)))
    return np.array(sorted(out), dtype=np.int64)


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
