"""CPU float64 oracle (test infrastructure only; see linear_logp.py)."""
from .linear_logp import (  # noqa: F401
    dlogits,
    entropy,
    entropy_dlogits,
    full_logp,
    grad_W_rows,
    grad_h_rows,
    linear_logp,
    linear_logp_entropy_grads,
    linear_logp_grads,
    logits,
    logp_from_logits,
    logsumexp_rows,
    sample_targets,
)
