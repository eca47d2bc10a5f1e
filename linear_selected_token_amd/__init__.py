"""Fused linear log-prob for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``librlk.so`` (C ABI in include/rlk.h); this package
binds it.  Importing it requires the built library: there is no other path."""
from ._lib import RlkError, build_info, lib, status_string  # noqa: F401

lib()  # fail loudly at import when the library is missing

from .ops import (  # noqa: E402,F401
    DIAG_FIELDS,
    ForwardBuffers,
    LinearKL,
    LinearLogp,
    LinearLogpEntropy,
    LinearLogpPGLoss,
    bwd_workspace_bytes,
    fwd_bwd_workspace_bytes,
    fwd_bwd_workspace_bytes_for_block,
    fwd_bwd_entropy_workspace_bytes,
    fwd_entropy_workspace_bytes,
    fwd_workspace_bytes,
    kl_fwd_workspace_bytes,
    linear_kl,
    linear_logp,
    linear_logp_entropy,
    linear_logp_pg_loss,
    logits_workspace_bytes,
    num_vocab_partials,
    ppo_fwd_bwd_workspace_bytes,
    rlk_compact_active,
    rlk_dlogp_diagnostics,
    rlk_linear_kl_bwd,
    rlk_linear_kl_fwd,
    rlk_linear_logp_bwd,
    rlk_linear_logp_bwd_entropy,
    rlk_linear_logp_fwd,
    rlk_linear_logp_fwd_bwd,
    rlk_linear_logp_fwd_bwd_entropy,
    rlk_linear_ppo_fwd_bwd,
    rlk_linear_logp_fwd_entropy,
    rlk_linear_logp_fwd_noalloc,
    rlk_linear_logp_merge,
    rlk_linear_logp_partials,
    rlk_linear_logp_partials_shard,
    rlk_logp_from_logits,
    rlk_ratio_kl_loss,
)
