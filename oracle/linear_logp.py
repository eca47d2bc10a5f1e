"""CPU float64 oracle of the fused linear log-prob.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
module.  The product path (the HIP library and its Python binding) never does and shares
no code with it.

What it computes (the plain definition, no blocking or reordering beyond it):

    z[t, v]  = (h_t . W_v) / T
    lse[t]   = log sum_v exp(z[t, v])
    logp[t]  = z[t, y_t] - lse[t]           for active tokens, 0 for inactive ones

The selected-token log-prob is computed from hidden states, the LM-head weight, target ids,
the active mask and the rollout temperature (RL-Kernel integration roadmap for vime,
"Operator Integration Plan", linear_logp "vime hook"); only active response tokens take
part (same page, "Consistency Contract").  The fused method reaches this definition
exactly, apart from rounding: its gain comes from not materialising the logits, not from
changing the maths (same page, "Fast and Consistency Compatibility").  So the oracle is the
definition itself, evaluated in float64 on the exact values of the (bf16- or fp32-valued)
inputs, one block of rows at a time; a block's full [rows, V] logit matrix is formed with a
library matmul.

The backward pass follows the loss L = -sum_t mask_t * adv_t * logp_t.  With
g_t = -mask_t * adv_t and p = softmax(z_t):

    dL/dz[t, v] = g_t * (delta(v, y_t) - p[t, v])
    dL/dh_t     = (1/T) sum_v dL/dz[t, v] W_v
    dL/dW_v     = (1/T) sum_t dL/dz[t, v] h_t

(the backward keeps the operator's own softmax statistics: RL-Kernel Roadmap (2026), P0.2,
"Fused CE LogProb without materializing logits + fused backward").

Pins: every function here is checked against values fixed by mathematics rather than by
itself: pure-Python brute force, closed forms (W = 0, V = 1, V = 2), identities
(sum_v exp(logp_v) = 1, temperature folding, vocabulary permutation), a library
cross-entropy and library autograd, and central finite differences (tests/test_oracle.py).
The sampler ``sample_targets`` is pinned by a pure-Python inverse-CDF walk and a
chi-square frequency check.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 64


def _f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float64:
        raise TypeError("the oracle takes float64 arrays (exact copies of the inputs)")
    return x


def logits(h: np.ndarray, W: np.ndarray, T: float) -> np.ndarray:
    """z = h W^T / T for a block of rows, float64."""
    return (_f64(h) @ _f64(W).T) / float(T)


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log sum_v exp(z[:, v]) per row, shifted by the row maximum for range."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def linear_logp(h: np.ndarray, W: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                T: float, rows: Optional[Sequence[int]] = None,
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Selected-token log-prob and log-sum-exp.

    Returns (logp, lse), float64.  With ``rows`` given, only those token rows are scored
    and the arrays follow ``rows``; otherwise all N rows are returned, with 0 at inactive
    tokens.  An active token whose target is outside [0, V) raises ValueError."""
    h = _f64(h)
    W = _f64(W)
    V = W.shape[0]
    targets = np.asarray(targets).astype(np.int64)
    active = np.asarray(mask).astype(bool)
    sel = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    logp = np.zeros(sel.shape[0])
    lse = np.zeros(sel.shape[0])
    todo = np.nonzero(active[sel])[0]
    bad = todo[(targets[sel[todo]] < 0) | (targets[sel[todo]] >= V)]
    if bad.size:
        raise ValueError(f"target out of range for active token row {int(sel[bad[0]])}")
    for b0 in range(0, todo.size, ROW_BLOCK):
        pos = todo[b0:b0 + ROW_BLOCK]
        t = sel[pos]
        z = logits(h[t], W, T)
        l = logsumexp_rows(z)
        lse[pos] = l
        logp[pos] = z[np.arange(t.size), targets[t]] - l
    return logp, lse


def full_logp(h: np.ndarray, W: np.ndarray, T: float) -> np.ndarray:
    """log softmax over the whole vocabulary, [N, V] (small shapes only)."""
    z = logits(h, W, T)
    return z - logsumexp_rows(z)[:, None]


def entropy(h: np.ndarray, W: np.ndarray, mask: np.ndarray, T: float) -> np.ndarray:
    """Entropy of the temperature-scaled next-token distribution, H_t = -sum_v p[t,v] log
    p[t,v] with p = softmax(h_t W^T / T), at active tokens (0 elsewhere): the entropy
    statistic the RL-Kernel Roadmap (2026) lists beside the fused log-prob (P0.2 and the
    entropy item of its RL-loss list).  Computed from the definition, one block of rows at a
    time."""
    h = _f64(h)
    W = _f64(W)
    active = np.nonzero(np.asarray(mask).astype(bool))[0]
    out = np.zeros(h.shape[0])
    for b0 in range(0, active.size, ROW_BLOCK):
        t = active[b0:b0 + ROW_BLOCK]
        z = logits(h[t], W, T)
        lp = z - logsumexp_rows(z)[:, None]
        out[t] = -np.sum(np.exp(lp) * lp, axis=1)
    return out


def logp_from_logits(z_raw: np.ndarray, targets: np.ndarray, mask: np.ndarray, T: float,
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Selected-token log-prob and log-sum-exp from logits that already exist (the
    reference-scoring sibling of the fused path: RL-Kernel integration roadmap for vime,
    "Operator Integration Plan", logp Reference Scoring).  z = z_raw / T, applied once;
    returns (logp, lse) with 0 at inactive tokens.  An active token whose target is outside
    [0, V) raises ValueError."""
    z_raw = _f64(z_raw)
    V = z_raw.shape[1]
    targets = np.asarray(targets).astype(np.int64)
    active = np.nonzero(np.asarray(mask).astype(bool))[0]
    if active.size and ((targets[active] < 0) | (targets[active] >= V)).any():
        raise ValueError("target out of range for an active token")
    logp = np.zeros(z_raw.shape[0])
    lse = np.zeros(z_raw.shape[0])
    for b0 in range(0, active.size, ROW_BLOCK):
        t = active[b0:b0 + ROW_BLOCK]
        z = z_raw[t] / float(T)
        l = logsumexp_rows(z)
        lse[t] = l
        logp[t] = z[np.arange(t.size), targets[t]] - l
    return logp, lse


def _upstream(adv: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """g_t = dL/dlogp_t = -mask_t * adv_t for L = -sum_t mask_t adv_t logp_t."""
    return -np.asarray(mask).astype(bool).astype(np.float64) * np.asarray(adv, dtype=np.float64)


def dlogits(h: np.ndarray, W: np.ndarray, targets: np.ndarray, g: np.ndarray, T: float,
            lse: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/dz = g_t (delta(v, y_t) - p[t, v]) for a block of rows, [rows, V]."""
    z = logits(h, W, T)
    l = logsumexp_rows(z) if lse is None else np.asarray(lse, dtype=np.float64)
    G = -np.exp(z - l[:, None])
    G[np.arange(z.shape[0]), np.asarray(targets).astype(np.int64)] += 1.0
    return G * np.asarray(g, dtype=np.float64)[:, None]


def entropy_dlogits(h: np.ndarray, W: np.ndarray, b: np.ndarray, T: float,
                    lse: Optional[np.ndarray] = None, ent: Optional[np.ndarray] = None,
                    ) -> np.ndarray:
    """dL/dz for a loss that depends on the entropy, for a block of rows, [rows, V]:
    b_t = dL/dH_t times dH_t/dz[t, v] = -p[t, v] (log p[t, v] + H_t), the derivative of
    H = -sum_v p_v log p_v through the softmax."""
    z = logits(h, W, T)
    l = logsumexp_rows(z) if lse is None else np.asarray(lse, dtype=np.float64)
    lp = z - l[:, None]
    p = np.exp(lp)
    H = -np.sum(p * lp, axis=1) if ent is None else np.asarray(ent, dtype=np.float64)
    return -np.asarray(b, dtype=np.float64)[:, None] * p * (lp + H[:, None])


def _entropy_upstream(ent_coef: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """b_t = dL/dH_t = -mask_t * c_t for L = -sum_t mask_t (adv_t logp_t + c_t H_t)."""
    return -np.asarray(mask).astype(bool).astype(np.float64) * np.asarray(ent_coef,
                                                                           dtype=np.float64)


def linear_logp_entropy_grads(h: np.ndarray, W: np.ndarray, targets: np.ndarray,
                              mask: np.ndarray, T: float, adv: np.ndarray,
                              ent_coef: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(dL/dh, dL/dW) in float64 for the policy-gradient loss with an entropy bonus,
    L = -sum_t mask_t (adv_t logp_t + c_t H_t) (the entropy-bonus term the RL-Kernel Roadmap
    (2026) lists in its operator backlog).  dL/dz is the log-prob term of dlogits plus
    entropy_dlogits; dh and dW follow from it as for linear_logp_grads."""
    h = _f64(h)
    W = _f64(W)
    g = _upstream(adv, mask)
    b = _entropy_upstream(ent_coef, mask)
    dh = np.zeros_like(h)
    dW = np.zeros_like(W)
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    for b0 in range(0, act.size, ROW_BLOCK):
        t = act[b0:b0 + ROW_BLOCK]
        G = dlogits(h[t], W, np.asarray(targets)[t], g[t], T) + entropy_dlogits(h[t], W, b[t], T)
        dh[t] = (G @ W) / T
        dW += (G.T @ h[t]) / T
    return dh, dW


def linear_logp_grads(h: np.ndarray, W: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                      T: float, adv: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(dL/dh [N, H], dL/dW [V, H]) in float64 for L = -sum_t mask_t adv_t logp_t.

    Holds dW in full: for shapes whose [V, H] float64 fits in memory."""
    h = _f64(h)
    W = _f64(W)
    g = _upstream(adv, mask)
    dh = np.zeros_like(h)
    dW = np.zeros_like(W)
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    for b0 in range(0, act.size, ROW_BLOCK):
        t = act[b0:b0 + ROW_BLOCK]
        G = dlogits(h[t], W, np.asarray(targets)[t], g[t], T)
        dh[t] = (G @ W) / T
        dW += (G.T @ h[t]) / T
    return dh, dW


def grad_h_rows(h: np.ndarray, W: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                T: float, adv: np.ndarray, rows: Sequence[int],
                ent_coef: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/dh for the listed token rows only, [len(rows), H] (with ``ent_coef``, of the loss
    with the entropy bonus, as in linear_logp_entropy_grads)."""
    h = _f64(h)
    W = _f64(W)
    rows = np.asarray(rows, dtype=np.int64)
    g = _upstream(adv, mask)[rows]
    b = None if ent_coef is None else _entropy_upstream(ent_coef, mask)[rows]
    out = np.zeros((rows.size, h.shape[1]))
    for b0 in range(0, rows.size, ROW_BLOCK):
        r = rows[b0:b0 + ROW_BLOCK]
        G = dlogits(h[r], W, np.asarray(targets)[r], g[b0:b0 + ROW_BLOCK], T)
        if b is not None:
            G += entropy_dlogits(h[r], W, b[b0:b0 + ROW_BLOCK], T)
        out[b0:b0 + r.size] = (G @ W) / T
    return out


def grad_W_rows(h: np.ndarray, W: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                T: float, adv: np.ndarray, vocab_rows: Sequence[int],
                lse: Optional[np.ndarray] = None, ent_coef: Optional[np.ndarray] = None,
                entropy_: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/dW for the listed vocabulary rows only, [len(vocab_rows), H].

    Needs every active token's lse; pass ``lse`` (from ``linear_logp``) to reuse it.  With
    ``ent_coef``, of the loss with the entropy bonus; it then needs every active token's
    entropy too (``entropy_``, from ``entropy``, or computed here)."""
    h = _f64(h)
    W = _f64(W)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    if lse is None:
        _, lse = linear_logp(h, W, targets, mask, T)
    g = _upstream(adv, mask)[act]
    z = (h[act] @ W[vocab_rows].T) / T                       # [Na, k]
    p = np.exp(z - np.asarray(lse, dtype=np.float64)[act][:, None])
    y = np.asarray(targets).astype(np.int64)[act]
    G = -p
    G += (y[:, None] == vocab_rows[None, :])
    G *= g[:, None]
    if ent_coef is not None:
        if entropy_ is None:
            entropy_ = entropy(h, W, mask, T)
        b = _entropy_upstream(ent_coef, mask)[act]
        lp = z - np.asarray(lse, dtype=np.float64)[act][:, None]
        G -= b[:, None] * p * (lp + np.asarray(entropy_, dtype=np.float64)[act][:, None])
    return (G.T @ h[act]) / T


def sample_targets(h: np.ndarray, W: np.ndarray, T: float, u: np.ndarray,
                   block: int = ROW_BLOCK) -> np.ndarray:
    """Draw one token per row from softmax(z_t) by inverse-CDF: the smallest v whose
    cumulative probability exceeds u_t (u_t uniform in [0, 1), supplied by the caller).

    If rounding leaves the total below u_t, the last token with nonzero probability is
    taken."""
    h = _f64(h)
    W = _f64(W)
    u = np.asarray(u, dtype=np.float64)
    out = np.empty(h.shape[0], dtype=np.int64)
    for b0 in range(0, h.shape[0], block):
        z = logits(h[b0:b0 + block], W, T)
        p = np.exp(z - logsumexp_rows(z)[:, None])
        c = np.cumsum(p, axis=1)
        for i in range(z.shape[0]):
            k = int(np.searchsorted(c[i], u[b0 + i], side="right"))
            if k >= c.shape[1]:
                k = int(np.nonzero(p[i] > 0)[0][-1])
            out[b0 + i] = k
    return out
