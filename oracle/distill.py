"""CPU float64 oracle of the full-vocabulary KL between two LM-head distributions.
TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path shares no code with it.

The RL-Kernel Roadmap (2026) lists, in its operator backlog, a chunked full-vocabulary KL /
distillation KL fused with the LM head, forward and reverse, beyond the sampled-token path.
Written from the definitions, for a student (h_s, W_s) and a teacher (h_t, W_t) sharing the
vocabulary and the temperature T:

    z_s = h_s W_s^T / T,  z_t = h_t W_t^T / T,  p_s = softmax(z_s),  p_t = softmax(z_t)
    KL_fwd[t] = sum_v p_t (log p_t - log p_s)        (teacher || student)
    KL_rev[t] = sum_v p_s (log p_s - log p_t)        (student || teacher)

at active tokens, 0 elsewhere.  For L = sum_t mask_t c_t KL[t] the gradients reach the student
only (the teacher is frozen):

    forward KL:  dL/dz_s[t, v] = c_t (p_s - p_t)
    reverse KL:  dL/dz_s[t, v] = c_t p_s (log p_s - log p_t - KL_rev[t])
    dL/dh_s = (1/T) dL/dz_s W_s,   dL/dW_s = (1/T) dL/dz_s^T h_s

Pins (tests/test_oracle_distill.py): library KL (torch kl_div), pure-Python brute force,
identical heads give 0, Gibbs' inequality, a uniform teacher's closed forms, and the
gradients against fp64 autograd and central finite differences.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 64


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float64:
        raise TypeError("the oracle takes float64 arrays (exact copies of the inputs)")
    return x


def _log_softmax(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))


def _block(h_s, W_s, h_t, W_t, T, t):
    ls = _log_softmax(h_s[t] @ W_s.T / T)
    lt = _log_softmax(h_t[t] @ W_t.T / T)
    return ls, lt


def kl_divergences(h_s, W_s, h_t, W_t, mask, T: float) -> Tuple[np.ndarray, np.ndarray]:
    """(KL_fwd [N], KL_rev [N]) in float64, 0 at inactive tokens."""
    h_s, W_s, h_t, W_t = (_f64(x) for x in (h_s, W_s, h_t, W_t))
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    fwd = np.zeros(h_s.shape[0])
    rev = np.zeros(h_s.shape[0])
    for b0 in range(0, act.size, ROW_BLOCK):
        t = act[b0:b0 + ROW_BLOCK]
        ls, lt = _block(h_s, W_s, h_t, W_t, T, t)
        fwd[t] = np.sum(np.exp(lt) * (lt - ls), axis=1)
        rev[t] = np.sum(np.exp(ls) * (ls - lt), axis=1)
    return fwd, rev


def _dz(ls, lt, c, reverse: bool):
    ps = np.exp(ls)
    if not reverse:
        return c[:, None] * (ps - np.exp(lt))
    kl = np.sum(ps * (ls - lt), axis=1)
    return c[:, None] * ps * (ls - lt - kl[:, None])


def kl_grads(h_s, W_s, h_t, W_t, mask, T: float, coef, reverse: bool,
             ) -> Tuple[np.ndarray, np.ndarray]:
    """(dL/dh_s [N, H_s], dL/dW_s [V, H_s]) for L = sum_t mask_t coef_t KL[t] (forward KL, or
    reverse with ``reverse``)."""
    h_s, W_s, h_t, W_t = (_f64(x) for x in (h_s, W_s, h_t, W_t))
    c = np.asarray(mask).astype(bool) * np.asarray(coef, dtype=np.float64)
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    dh = np.zeros_like(h_s)
    dW = np.zeros_like(W_s)
    for b0 in range(0, act.size, ROW_BLOCK):
        t = act[b0:b0 + ROW_BLOCK]
        ls, lt = _block(h_s, W_s, h_t, W_t, T, t)
        G = _dz(ls, lt, c[t], reverse)
        dh[t] = (G @ W_s) / T
        dW += (G.T @ h_s[t]) / T
    return dh, dW


def kl_grad_h_rows(h_s, W_s, h_t, W_t, mask, T: float, coef, reverse: bool,
                   rows: Sequence[int]) -> np.ndarray:
    """dL/dh_s for the listed token rows only."""
    h_s, W_s, h_t, W_t = (_f64(x) for x in (h_s, W_s, h_t, W_t))
    rows = np.asarray(rows, dtype=np.int64)
    c = np.asarray(mask).astype(bool) * np.asarray(coef, dtype=np.float64)
    out = np.zeros((rows.size, h_s.shape[1]))
    for b0 in range(0, rows.size, ROW_BLOCK):
        r = rows[b0:b0 + ROW_BLOCK]
        ls, lt = _block(h_s, W_s, h_t, W_t, T, r)
        out[b0:b0 + r.size] = (_dz(ls, lt, c[r], reverse) @ W_s) / T
    return out


def kl_grad_W_rows(h_s, W_s, h_t, W_t, mask, T: float, coef, reverse: bool,
                   vocab_rows: Sequence[int], lse_s: Optional[np.ndarray] = None,
                   lse_t: Optional[np.ndarray] = None, kl_rev: Optional[np.ndarray] = None,
                   ) -> np.ndarray:
    """dL/dW_s for the listed vocabulary rows only.  Needs every active token's lse under both
    heads (and KL_rev for the reverse direction); pass them to reuse them."""
    h_s, W_s, h_t, W_t = (_f64(x) for x in (h_s, W_s, h_t, W_t))
    vr = np.asarray(vocab_rows, dtype=np.int64)
    act = np.nonzero(np.asarray(mask).astype(bool))[0]
    c = np.asarray(coef, dtype=np.float64)[act]
    if lse_s is None or lse_t is None or (reverse and kl_rev is None):
        lse_s = np.zeros(h_s.shape[0])
        lse_t = np.zeros(h_s.shape[0])
        for b0 in range(0, act.size, ROW_BLOCK):
            t = act[b0:b0 + ROW_BLOCK]
            for z, out in ((h_s[t] @ W_s.T / T, lse_s), (h_t[t] @ W_t.T / T, lse_t)):
                m = z.max(axis=1)
                out[t] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        if reverse:
            _, kl_rev = kl_divergences(h_s, W_s, h_t, W_t, mask, T)
    ls = h_s[act] @ W_s[vr].T / T - np.asarray(lse_s, dtype=np.float64)[act][:, None]
    lt = h_t[act] @ W_t[vr].T / T - np.asarray(lse_t, dtype=np.float64)[act][:, None]
    ps = np.exp(ls)
    if not reverse:
        G = c[:, None] * (ps - np.exp(lt))
    else:
        G = c[:, None] * ps * (ls - lt - np.asarray(kl_rev, dtype=np.float64)[act][:, None])
    return (G.T @ h_s[act]) / T
