"""CPU float64 oracle of the loss fragments that consume the selected-token log-prob.
TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path shares no code with it.

Two operations (RL-Kernel integration roadmap for vime, "RL Loss Operators: ratio_kl,
GRPO/PPO/DPO Loss Fragments", and the minimum diagnostics list under "Consistency
Contract"):

ratio_kl_loss -- the per-token clipped policy-gradient loss with a KL penalty towards a
reference policy, written from the definitions (plain reading where the pages leave the
formula to the caller):

    r_t     = exp(logp_t - old_logp_t)
    pg_t    = max(-A_t r_t, -A_t clip(r_t, 1 - eps_lo, 1 + eps_hi))
    kl_t    = exp(d_t) - 1 - d_t,  d_t = ref_logp_t - logp_t
              (the same function of a log-ratio as the pages' approx_kl0)
    L_t     = scale * mask_t * (pg_t + beta * kl_t)
    dL/dlogp_t = scale * mask_t * (-A_t r_t [pg_t takes the unclipped term]
                                   + beta * (1 - exp(d_t)))

  clipped_t = 1 where the clipped term is strictly the larger one (its gradient is 0).
  Also returned: the masked sums of L, clipped and kl and the active count.

dlogp_diagnostics -- for two log-prob tensors of the same tokens (say a training recompute
and the rollout's), over active tokens: mean, max and the 50/90/99th percentiles of
|dlogp| (linear interpolation between order statistics, numpy's default), the mean of
ratio0 = exp(dlogp), clipfrac0 = fraction with |ratio0 - 1| > eps, approx_kl0 =
mean(exp(dlogp) - 1 - dlogp), the active count and the first token of largest |dlogp|.

Pins (tests/test_oracle_rl_loss.py): library autograd of the loss, closed forms (r = 1,
A = 0, beta = 0), a pure-Python walk of the definitions, and order statistics against a
sorted copy.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def ratio_kl_loss(logp, old_logp, ref_logp: Optional[np.ndarray], adv, mask, eps_lo: float,
                  eps_hi: float, beta: float, scale: float,
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, Dict[str, float]]:
    """(loss [N], dL/dlogp [N], ratio [N], clipped [N] int, sums) in float64; 0 at
    inactive tokens.  ref_logp None means no KL term; with a reference the KL sum is
    reported even when beta = 0 (monitoring without a penalty)."""
    lp = _f64(logp)
    m = np.asarray(mask).astype(bool)
    A = _f64(adv)
    r = np.exp(lp - _f64(old_logp))
    unclipped = -A * r
    clipped_term = -A * np.clip(r, 1.0 - eps_lo, 1.0 + eps_hi)
    pg = np.maximum(unclipped, clipped_term)
    clipped = clipped_term > unclipped
    dpg = np.where(clipped, 0.0, -A * r)
    if ref_logp is not None:
        d = _f64(ref_logp) - lp
        kl = np.exp(d) - 1.0 - d
        dkl = 1.0 - np.exp(d)
    else:
        kl = np.zeros_like(lp)
        dkl = np.zeros_like(lp)
    loss = np.where(m, scale * (pg + beta * kl), 0.0)
    grad = np.where(m, scale * (dpg + beta * dkl), 0.0)
    sums = {"loss": float(loss.sum()), "clipped": float((clipped & m).sum()),
            "kl": float(np.where(m, kl, 0.0).sum()), "active": float(m.sum())}
    return loss, grad, np.where(m, r, 0.0), (clipped & m).astype(np.int64), sums


def dlogp_diagnostics(logp_a, logp_b, mask, eps: float) -> Dict[str, float]:
    """Diagnostics of dlogp = logp_a - logp_b over active tokens (see the module header)."""
    m = np.asarray(mask).astype(bool)
    act = np.nonzero(m)[0]
    out = {"active": float(act.size)}
    if act.size == 0:
        for k in ("mean", "max", "p50", "p90", "p99", "ratio_mean", "clipfrac", "approx_kl"):
            out[k] = 0.0
        out["worst"] = -1
        return out
    d = _f64(logp_a)[act] - _f64(logp_b)[act]
    a = np.abs(d)
    out["mean"] = float(a.mean())
    out["max"] = float(a.max())
    for q in (50, 90, 99):
        out[f"p{q}"] = float(np.percentile(a, q))
    ratio = np.exp(d)
    out["ratio_mean"] = float(ratio.mean())
    out["clipfrac"] = float((np.abs(ratio - 1.0) > eps).mean())
    out["approx_kl"] = float((ratio - 1.0 - d).mean())
    out["worst"] = int(act[int(np.argmax(a))])
    return out
