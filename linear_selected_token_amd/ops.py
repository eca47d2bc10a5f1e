"""Python binding of the C ABI (include/rlk.h), with the same names.

Argument marshalling only: tensors must already live on the GPU; PyTorch provides device
memory (outputs and workspaces) and the current stream, and every step of the path runs
in the library's HIP kernels.  Errors from the library raise ``RlkError``."""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib as L

RlkError = L.RlkError


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.RLK_BF16
    if t.dtype == torch.float32:
        return L.RLK_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or float32")


def _mask_u8(mask: torch.Tensor) -> torch.Tensor:
    if mask.dtype == torch.bool:
        return mask.view(torch.uint8)
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8 or bool")
    return mask


def _check(h, W, targets, mask):
    for name, t in (("h", h), ("W", W), ("targets", targets), ("mask", mask)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if h.dim() != 2 or W.dim() != 2 or h.shape[1] != W.shape[1]:
        raise ValueError("h must be [N, H] and W [V, H]")
    if h.dtype != W.dtype:
        raise TypeError("h and W must share a dtype")
    if targets.dtype != torch.int32 or targets.shape != (h.shape[0],):
        raise ValueError("targets must be int32 [N]")
    if mask.shape != (h.shape[0],):
        raise ValueError("mask must be [N]")


def num_vocab_partials(V: int) -> int:
    return int(L.lib().rlk_num_vocab_partials(V))


def fwd_workspace_bytes(N: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_fwd_workspace_size(N, H, V, dtype, ctypes.byref(out)),
            "rlk_linear_logp_fwd_workspace_size")
    return int(out.value)


def bwd_workspace_bytes(N: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_bwd_workspace_size(N, H, V, dtype, ctypes.byref(out)),
            "rlk_linear_logp_bwd_workspace_size")
    return int(out.value)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _sized_workspace(default_bytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """For calls whose token blocks follow the workspace's size: the caller's workspace as given
    (the library refuses one too small for its smallest blocks), else one of the default size."""
    if ws is not None:
        return ws
    return torch.empty(max(default_bytes, 256), dtype=torch.uint8, device=device)


def rlk_linear_logp_fwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                        mask: torch.Tensor, temperature: float,
                        workspace: Optional[torch.Tensor] = None,
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Selected-token log-prob; returns (logp [N] float32, lse [N] float32)."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    logp = torch.empty(N, dtype=torch.float32, device=h.device)
    lse = torch.empty(N, dtype=torch.float32, device=h.device)
    ws = _workspace(fwd_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_fwd(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H, V, dt,
                                        float(temperature), _vp(logp), _vp(lse), _vp(ws),
                                        ws.numel() * ws.element_size(), _stream(h.device)),
            "rlk_linear_logp_fwd")
    return logp, lse


def rlk_linear_logp_fwd_noalloc(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                                mask: torch.Tensor, temperature: float,
                                logp: Optional[torch.Tensor] = None,
                                lse: Optional[torch.Tensor] = None,
                                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """rlk_linear_logp_fwd with the library's static scratch as its workspace (the library
    allocates nothing); returns (logp, lse).  Pass preallocated logp and lse ([N] float32) to
    make the call allocate nothing at all."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    for name, t in (("logp", logp), ("lse", lse)):
        if t is not None and (not t.is_cuda or t.dtype != torch.float32 or t.shape != (N,)
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [N]")
    if logp is None:
        logp = torch.empty(N, dtype=torch.float32, device=h.device)
    if lse is None:
        lse = torch.empty(N, dtype=torch.float32, device=h.device)
    L.check(L.lib().rlk_linear_logp_fwd_noalloc(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H, V,
                                                dt, float(temperature), _vp(logp), _vp(lse),
                                                _stream(h.device)),
            "rlk_linear_logp_fwd_noalloc")
    return logp, lse


def fwd_entropy_workspace_bytes(N: int, H: int, V: int, dtype_code: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_fwd_entropy_workspace_size(N, H, V, dtype_code,
                                                               ctypes.byref(out)),
            "rlk_linear_logp_fwd_entropy_workspace_size")
    return int(out.value)


def rlk_linear_logp_fwd_entropy(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                                mask: torch.Tensor, temperature: float,
                                workspace: Optional[torch.Tensor] = None,
                                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Selected-token log-prob and the entropy of each token's distribution; returns
    (logp, lse, entropy), each [N] float32."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    logp = torch.empty(N, dtype=torch.float32, device=h.device)
    lse = torch.empty(N, dtype=torch.float32, device=h.device)
    ent = torch.empty(N, dtype=torch.float32, device=h.device)
    ws = _workspace(fwd_entropy_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_fwd_entropy(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H,
                                                V, dt, float(temperature), _vp(logp), _vp(lse),
                                                _vp(ent), _vp(ws), ws.numel() * ws.element_size(),
                                                _stream(h.device)),
            "rlk_linear_logp_fwd_entropy")
    return logp, lse, ent


def logits_workspace_bytes(N: int, V: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_logp_from_logits_workspace_size(N, V, ctypes.byref(out)),
            "rlk_logp_from_logits_workspace_size")
    return int(out.value)


def rlk_logp_from_logits(logits: torch.Tensor, targets: torch.Tensor, mask: torch.Tensor,
                         temperature: float, V: Optional[int] = None,
                         workspace: Optional[torch.Tensor] = None,
                         ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Selected-token log-prob from existing logits [N, ld] (the first V entries of each row,
    V = ld by default); returns (logp [N] float32, lse [N] float32)."""
    mask = _mask_u8(mask)
    if not (logits.is_cuda and targets.is_cuda and mask.is_cuda):
        raise ValueError("logits, targets and mask must be GPU tensors")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [N, ld] with unit stride along the vocabulary")
    if targets.dtype != torch.int32 or targets.shape != (logits.shape[0],) or \
            mask.shape != (logits.shape[0],) or not targets.is_contiguous():
        raise ValueError("targets must be int32 [N] and mask [N]")
    N, ld = logits.shape[0], logits.stride(0) if logits.shape[0] > 1 else logits.shape[1]
    V = logits.shape[1] if V is None else int(V)
    dt = _dtype_code(logits)
    logp = torch.empty(N, dtype=torch.float32, device=logits.device)
    lse = torch.empty(N, dtype=torch.float32, device=logits.device)
    ws = _workspace(logits_workspace_bytes(N, V), logits.device, workspace)
    L.check(L.lib().rlk_logp_from_logits(_vp(logits), ld, _vp(targets), _vp(mask), N, V, dt,
                                         float(temperature), _vp(logp), _vp(lse), _vp(ws),
                                         ws.numel() * ws.element_size(),
                                         _stream(logits.device)), "rlk_logp_from_logits")
    return logp, lse


def rlk_linear_logp_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                        mask: torch.Tensor, temperature: float, adv: torch.Tensor,
                        lse: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                        dh: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gradients of L = -sum_t mask_t adv_t logp_t; returns (dh [N,H], dW [V,H]) float32."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    for name, t in (("adv", adv), ("lse", lse)):
        if not t.is_cuda or t.dtype != torch.float32 or t.shape != (N,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [N]")
    if dh is None:
        dh = torch.empty((N, H), dtype=torch.float32, device=h.device)
    if dW is None:
        dW = torch.empty((V, H), dtype=torch.float32, device=h.device)
    ws = _workspace(bwd_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_bwd(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H, V, dt,
                                        float(temperature), _vp(adv), _vp(lse), _vp(dh), _vp(dW),
                                        _vp(ws), ws.numel() * ws.element_size(),
                                        _stream(h.device)),
            "rlk_linear_logp_bwd")
    return dh, dW


def rlk_linear_logp_bwd_entropy(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                                mask: torch.Tensor, temperature: float, adv: torch.Tensor,
                                ent_coef: torch.Tensor, lse: torch.Tensor, entropy: torch.Tensor,
                                workspace: Optional[torch.Tensor] = None,
                                dh: Optional[torch.Tensor] = None,
                                dW: Optional[torch.Tensor] = None,
                                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gradients of L = -sum_t mask_t (adv_t logp_t + ent_coef_t H_t), with lse and entropy
    from rlk_linear_logp_fwd_entropy; returns (dh [N,H], dW [V,H]) float32."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    for name, t in (("adv", adv), ("ent_coef", ent_coef), ("lse", lse), ("entropy", entropy)):
        if not t.is_cuda or t.dtype != torch.float32 or t.shape != (N,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [N]")
    if dh is None:
        dh = torch.empty((N, H), dtype=torch.float32, device=h.device)
    if dW is None:
        dW = torch.empty((V, H), dtype=torch.float32, device=h.device)
    ws = _workspace(bwd_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_bwd_entropy(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H,
                                                V, dt, float(temperature), _vp(adv),
                                                _vp(ent_coef), _vp(lse), _vp(entropy), _vp(dh),
                                                _vp(dW), _vp(ws), ws.numel() * ws.element_size(),
                                                _stream(h.device)),
            "rlk_linear_logp_bwd_entropy")
    return dh, dW


def fwd_bwd_workspace_bytes(N: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_fwd_bwd_workspace_size(N, H, V, dtype, ctypes.byref(out)),
            "rlk_linear_logp_fwd_bwd_workspace_size")
    return int(out.value)


def fwd_bwd_workspace_bytes_for_block(N: int, H: int, V: int, dtype: int,
                                      block_tokens: int) -> int:
    """Workspace bytes with which rlk_linear_logp_fwd_bwd takes token blocks of block_tokens
    tokens, rounded up to 256 (0: the default's blocks; N or more: one block)."""
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_fwd_bwd_workspace_size_for_block(N, H, V, dtype, block_tokens,
                                                                     ctypes.byref(out)),
            "rlk_linear_logp_fwd_bwd_workspace_size_for_block")
    return int(out.value)


def rlk_linear_logp_fwd_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                            mask: torch.Tensor, temperature: float, adv: torch.Tensor,
                            workspace: Optional[torch.Tensor] = None,
                            dh: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
                            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Forward and gradients of L = -sum_t mask_t adv_t logp_t in one call; returns
    (logp [N], lse [N], dh [N,H], dW [V,H]), all float32."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    if not adv.is_cuda or adv.dtype != torch.float32 or adv.shape != (N,) or not adv.is_contiguous():
        raise ValueError("adv must be a contiguous float32 GPU tensor [N]")
    logp = torch.empty(N, dtype=torch.float32, device=h.device)
    lse = torch.empty(N, dtype=torch.float32, device=h.device)
    if dh is None:
        dh = torch.empty((N, H), dtype=torch.float32, device=h.device)
    if dW is None:
        dW = torch.empty((V, H), dtype=torch.float32, device=h.device)
    ws = _sized_workspace(fwd_bwd_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_fwd_bwd(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H, V, dt,
                                            float(temperature), _vp(adv), _vp(logp), _vp(lse),
                                            _vp(dh), _vp(dW), _vp(ws),
                                            ws.numel() * ws.element_size(), _stream(h.device)),
            "rlk_linear_logp_fwd_bwd")
    return logp, lse, dh, dW


# ---- building blocks of the forward

def rlk_compact_active(mask: torch.Tensor, idx: torch.Tensor, n_active: torch.Tensor,
                       target_logit: Optional[torch.Tensor] = None,
                       logp: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None) -> None:
    mask = _mask_u8(mask)
    L.check(L.lib().rlk_compact_active(_vp(mask), mask.numel(), _vp(idx), _vp(n_active),
                                       _vp(target_logit), _vp(logp), _vp(lse),
                                       _stream(mask.device)), "rlk_compact_active")


def rlk_linear_logp_partials(h, W, targets, idx, n_active, temperature, part_max, part_sum,
                             target_logit) -> None:
    N, H = h.shape
    V = W.shape[0]
    L.check(L.lib().rlk_linear_logp_partials(_vp(h), _vp(W), _vp(targets), _vp(idx),
                                             _vp(n_active), N, H, V, _dtype_code(h),
                                             float(temperature), _vp(part_max), _vp(part_sum),
                                             _vp(target_logit), _stream(h.device)),
            "rlk_linear_logp_partials")


def rlk_linear_logp_partials_shard(h, W_shard, targets, idx, n_active, vocab_start, V_global,
                                   temperature, part_max, part_sum, target_logit) -> None:
    """Partial statistics of the vocabulary rows vocab_start .. vocab_start + len(W_shard) - 1,
    written into the full-vocabulary part_max / part_sum ([num_vocab_partials(V_global), N])."""
    N, H = h.shape
    V = W_shard.shape[0]
    L.check(L.lib().rlk_linear_logp_partials_shard(
        _vp(h), _vp(W_shard), _vp(targets), _vp(idx), _vp(n_active), N, H, V, int(vocab_start),
        int(V_global), _dtype_code(h), float(temperature), _vp(part_max), _vp(part_sum),
        _vp(target_logit), _stream(h.device)), "rlk_linear_logp_partials_shard")


def rlk_linear_logp_merge(part_max, part_sum, target_logit, idx, n_active, N, V, logp,
                          lse=None) -> None:
    L.check(L.lib().rlk_linear_logp_merge(_vp(part_max), _vp(part_sum), _vp(target_logit),
                                          _vp(idx), _vp(n_active), N, V, _vp(logp), _vp(lse),
                                          _stream(logp.device)), "rlk_linear_logp_merge")


class ForwardBuffers:
    """Preallocated buffers for calling the three forward building blocks in sequence."""

    def __init__(self, N: int, V: int, device):
        J = num_vocab_partials(V)
        self.idx = torch.empty(max(N, 1), dtype=torch.int32, device=device)
        self.n_active = torch.empty(1, dtype=torch.int32, device=device)
        self.target_logit = torch.empty(max(N, 1), dtype=torch.float32, device=device)
        self.part_max = torch.empty((J, max(N, 1)), dtype=torch.float32, device=device)
        self.part_sum = torch.empty((J, max(N, 1)), dtype=torch.float32, device=device)
        self.logp = torch.empty(max(N, 1), dtype=torch.float32, device=device)
        self.lse = torch.empty(max(N, 1), dtype=torch.float32, device=device)


# ---- autograd

class LinearLogp(torch.autograd.Function):
    """logp = linear_logp(h, W, targets, mask, T); backward through rlk_linear_logp_bwd
    with adv = -dL/dlogp."""

    @staticmethod
    def forward(ctx, h, W, targets, mask, temperature):
        logp, lse = rlk_linear_logp_fwd(h, W, targets, mask, temperature)
        ctx.save_for_backward(h, W, targets, mask, lse)
        ctx.temperature = float(temperature)
        return logp

    @staticmethod
    def backward(ctx, grad_logp):
        h, W, targets, mask, lse = ctx.saved_tensors
        adv = (-grad_logp).to(torch.float32).contiguous()
        dh, dW = rlk_linear_logp_bwd(h, W, targets, mask, ctx.temperature, adv, lse)
        return dh.to(h.dtype), dW.to(W.dtype), None, None, None


def linear_logp(h, W, targets, mask, temperature) -> torch.Tensor:
    """Differentiable selected-token log-prob [N] (float32)."""
    return LinearLogp.apply(h, W, targets, mask, temperature)


class LinearLogpEntropy(torch.autograd.Function):
    """(logp, entropy) = linear_logp_entropy(h, W, targets, mask, T); backward through
    rlk_linear_logp_bwd_entropy with adv = -dL/dlogp and ent_coef = -dL/dentropy (through
    rlk_linear_logp_bwd when no gradient reaches the entropy)."""

    @staticmethod
    def forward(ctx, h, W, targets, mask, temperature):
        logp, lse, ent = rlk_linear_logp_fwd_entropy(h, W, targets, mask, temperature)
        ctx.save_for_backward(h, W, targets, mask, lse, ent)
        ctx.temperature = float(temperature)
        return logp, ent

    @staticmethod
    def backward(ctx, grad_logp, grad_ent):
        h, W, targets, mask, lse, ent = ctx.saved_tensors
        adv = (torch.zeros_like(lse) if grad_logp is None else
               (-grad_logp).to(torch.float32).contiguous())
        if grad_ent is None:
            dh, dW = rlk_linear_logp_bwd(h, W, targets, mask, ctx.temperature, adv, lse)
        else:
            coef = (-grad_ent).to(torch.float32).contiguous()
            dh, dW = rlk_linear_logp_bwd_entropy(h, W, targets, mask, ctx.temperature, adv, coef,
                                                 lse, ent)
        return dh.to(h.dtype), dW.to(W.dtype), None, None, None


def linear_logp_entropy(h, W, targets, mask, temperature):
    """Differentiable selected-token log-prob and entropy, each [N] (float32)."""
    return LinearLogpEntropy.apply(h, W, targets, mask, temperature)


def fwd_bwd_entropy_workspace_bytes(N: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_logp_fwd_bwd_entropy_workspace_size(N, H, V, dtype,
                                                                   ctypes.byref(out)),
            "rlk_linear_logp_fwd_bwd_entropy_workspace_size")
    return int(out.value)


def rlk_linear_logp_fwd_bwd_entropy(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                                    mask: torch.Tensor, temperature: float, adv: torch.Tensor,
                                    ent_coef: torch.Tensor,
                                    workspace: Optional[torch.Tensor] = None,
                                    dh: Optional[torch.Tensor] = None,
                                    dW: Optional[torch.Tensor] = None):
    """Forward with the entropy and gradients of L = -sum mask (adv logp + c H) in one call;
    returns (logp, lse, entropy [N], dh [N,H], dW [V,H]), all float32."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    _vec("adv", adv, N)
    _vec("ent_coef", ent_coef, N)
    f32 = dict(dtype=torch.float32, device=h.device)
    logp, lse, ent = (torch.empty(N, **f32) for _ in range(3))
    if dh is None:
        dh = torch.empty((N, H), **f32)
    if dW is None:
        dW = torch.empty((V, H), **f32)
    ws = _sized_workspace(fwd_bwd_entropy_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_logp_fwd_bwd_entropy(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H,
                                                    V, dt, float(temperature), _vp(adv),
                                                    _vp(ent_coef), _vp(logp), _vp(lse), _vp(ent),
                                                    _vp(dh), _vp(dW), _vp(ws),
                                                    ws.numel() * ws.element_size(),
                                                    _stream(h.device)),
            "rlk_linear_logp_fwd_bwd_entropy")
    return logp, lse, ent, dh, dW


def ppo_fwd_bwd_workspace_bytes(N: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_ppo_fwd_bwd_workspace_size(N, H, V, dtype, ctypes.byref(out)),
            "rlk_linear_ppo_fwd_bwd_workspace_size")
    return int(out.value)


def rlk_linear_ppo_fwd_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                           mask: torch.Tensor, temperature: float, old_logp: torch.Tensor,
                           ref_logp: Optional[torch.Tensor], adv: torch.Tensor, eps_lo: float,
                           eps_hi: float, beta: float, scale: float,
                           workspace: Optional[torch.Tensor] = None,
                           dh: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None):
    """Forward, clipped policy-gradient loss with a KL penalty and its gradients in one call;
    returns (logp, lse, loss, bwd_adv, ratio [N] float32, sums [4] float64, dh [N,H],
    dW [V,H])."""
    mask = _mask_u8(mask)
    _check(h, W, targets, mask)
    N, H = h.shape
    V = W.shape[0]
    dt = _dtype_code(h)
    _vec("old_logp", old_logp, N)
    _vec("adv", adv, N)
    if ref_logp is not None:
        _vec("ref_logp", ref_logp, N)
    f32 = dict(dtype=torch.float32, device=h.device)
    logp, lse, loss, badv, ratio = (torch.empty(N, **f32) for _ in range(5))
    sums = torch.empty(4, dtype=torch.float64, device=h.device)
    if dh is None:
        dh = torch.empty((N, H), **f32)
    if dW is None:
        dW = torch.empty((V, H), **f32)
    ws = _sized_workspace(ppo_fwd_bwd_workspace_bytes(N, H, V, dt), h.device, workspace)
    L.check(L.lib().rlk_linear_ppo_fwd_bwd(_vp(h), _vp(W), _vp(targets), _vp(mask), N, H, V, dt,
                                           float(temperature), _vp(old_logp), _vp(ref_logp),
                                           _vp(adv), float(eps_lo), float(eps_hi), float(beta),
                                           float(scale), _vp(logp), _vp(lse), _vp(loss),
                                           _vp(badv), _vp(ratio), _vp(sums), _vp(dh), _vp(dW),
                                           _vp(ws), ws.numel() * ws.element_size(),
                                           _stream(h.device)),
            "rlk_linear_ppo_fwd_bwd")
    return logp, lse, loss, badv, ratio, sums, dh, dW


class LinearLogpPGLoss(torch.autograd.Function):
    """loss = -sum_t mask_t adv_t logp_t with its gradients computed in the forward
    (rlk_linear_logp_fwd_bwd); the backward scales them by the incoming scalar gradient."""

    @staticmethod
    def forward(ctx, h, W, targets, mask, temperature, adv):
        adv32 = adv.to(torch.float32).contiguous()
        logp, _, dh, dW = rlk_linear_logp_fwd_bwd(h, W, targets, mask, temperature, adv32)
        m = _mask_u8(mask).to(torch.float32)
        loss = -(m * adv32 * torch.nan_to_num(logp)).sum()
        ctx.save_for_backward(dh, dW)
        ctx.dtypes = (h.dtype, W.dtype)
        ctx.mark_non_differentiable(logp)
        return loss, logp

    @staticmethod
    def backward(ctx, grad_loss, grad_logp):
        dh, dW = ctx.saved_tensors
        g = grad_loss.to(torch.float32)
        return (dh * g).to(ctx.dtypes[0]), (dW * g).to(ctx.dtypes[1]), None, None, None, None


def linear_logp_pg_loss(h, W, targets, mask, temperature, adv):
    """(loss, logp): the policy-gradient loss -sum mask * adv * logp as a differentiable
    scalar (gradients into h and W, formed in the forward in one fused call), and the
    selected-token log-prob [N] (float32, not differentiable)."""
    return LinearLogpPGLoss.apply(h, W, targets, mask, temperature, adv)


# ---- loss fragments on the log-prob

def _vec(name: str, t: torch.Tensor, N: int, dtype=torch.float32) -> None:
    if not t.is_cuda or t.dtype != dtype or t.shape != (N,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor [{N}]")


def rlk_ratio_kl_loss(logp: torch.Tensor, old_logp: torch.Tensor,
                      ref_logp: Optional[torch.Tensor], adv: torch.Tensor, mask: torch.Tensor,
                      eps_lo: float, eps_hi: float, beta: float = 0.0, scale: float = 1.0,
                      want_ratio: bool = False, workspace: Optional[torch.Tensor] = None):
    """Clipped policy-gradient loss with a KL penalty, per token.  Returns (loss [N],
    bwd_adv [N] = -dloss/dlogp, ratio [N] or None, sums [4] float64 on the device:
    sum loss, clipped count, sum kl, active count)."""
    mask = _mask_u8(mask)
    N = logp.shape[0]
    for name, t in (("logp", logp), ("old_logp", old_logp), ("adv", adv)):
        _vec(name, t, N)
    if ref_logp is not None:
        _vec("ref_logp", ref_logp, N)
    _vec("mask", mask, N, torch.uint8)
    dev = logp.device
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    badv = torch.empty(N, dtype=torch.float32, device=dev)
    ratio = torch.empty(N, dtype=torch.float32, device=dev) if want_ratio else None
    sums = torch.empty(4, dtype=torch.float64, device=dev)
    nb = ctypes.c_size_t(0)
    L.check(L.lib().rlk_ratio_kl_loss_workspace_size(N, ctypes.byref(nb)),
            "rlk_ratio_kl_loss_workspace_size")
    ws = _workspace(int(nb.value), dev, workspace)
    L.check(L.lib().rlk_ratio_kl_loss(_vp(logp), _vp(old_logp), _vp(ref_logp), _vp(adv),
                                      _vp(mask), N, float(eps_lo), float(eps_hi), float(beta),
                                      float(scale), _vp(loss), _vp(badv), _vp(ratio), _vp(sums),
                                      _vp(ws), ws.numel() * ws.element_size(), _stream(dev)),
            "rlk_ratio_kl_loss")
    return loss, badv, ratio, sums


DIAG_FIELDS = ("active", "mean", "max", "p50", "p90", "p99", "ratio_mean", "clipfrac",
               "approx_kl")


def rlk_dlogp_diagnostics(logp_a: torch.Tensor, logp_b: torch.Tensor, mask: torch.Tensor,
                          clip_eps: float, workspace: Optional[torch.Tensor] = None):
    """dlogp diagnostics over active tokens; returns (out [9] float64, worst [1] int64), both
    on the device (fields in DIAG_FIELDS order)."""
    mask = _mask_u8(mask)
    N = logp_a.shape[0]
    _vec("logp_a", logp_a, N)
    _vec("logp_b", logp_b, N)
    _vec("mask", mask, N, torch.uint8)
    dev = logp_a.device
    out = torch.empty(9, dtype=torch.float64, device=dev)
    worst = torch.empty(1, dtype=torch.int64, device=dev)
    nb = ctypes.c_size_t(0)
    L.check(L.lib().rlk_dlogp_diagnostics_workspace_size(N, ctypes.byref(nb)),
            "rlk_dlogp_diagnostics_workspace_size")
    ws = _workspace(int(nb.value), dev, workspace)
    L.check(L.lib().rlk_dlogp_diagnostics(_vp(logp_a), _vp(logp_b), _vp(mask), N,
                                          float(clip_eps), _vp(out), _vp(worst), _vp(ws),
                                          ws.numel() * ws.element_size(), _stream(dev)),
            "rlk_dlogp_diagnostics")
    return out, worst


# ---- full-vocabulary KL between two LM heads

def _check_kl(h_s, W_s, h_t, W_t, mask):
    for name, t in (("h_s", h_s), ("W_s", W_s), ("h_t", h_t), ("W_t", W_t), ("mask", mask)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if h_s.dim() != 2 or W_s.dim() != 2 or h_s.shape[1] != W_s.shape[1]:
        raise ValueError("h_s must be [N, H_s] and W_s [V, H_s]")
    if h_t.dim() != 2 or W_t.dim() != 2 or h_t.shape[1] != W_t.shape[1]:
        raise ValueError("h_t must be [N, H_t] and W_t [V, H_t]")
    if h_t.shape[0] != h_s.shape[0] or W_t.shape[0] != W_s.shape[0]:
        raise ValueError("student and teacher must share N and V")
    if len({h_s.dtype, W_s.dtype, h_t.dtype, W_t.dtype}) != 1:
        raise TypeError("all four operands must share a dtype")
    if mask.shape != (h_s.shape[0],):
        raise ValueError("mask must be [N]")


def kl_fwd_workspace_bytes(N: int, H_s: int, H_t: int, V: int, dtype: int,
                           block_tokens: Optional[int] = None) -> int:
    """Workspace bytes of rlk_linear_kl_fwd: the default, or for token blocks of block_tokens (a
    positive multiple of 256)."""
    nb = ctypes.c_size_t(0)
    if block_tokens is None:
        L.check(L.lib().rlk_linear_kl_fwd_workspace_size(N, H_s, H_t, V, dtype, ctypes.byref(nb)),
                "rlk_linear_kl_fwd_workspace_size")
    else:
        L.check(L.lib().rlk_linear_kl_fwd_workspace_size_for_block(N, H_s, H_t, V, dtype,
                                                                   int(block_tokens),
                                                                   ctypes.byref(nb)),
                "rlk_linear_kl_fwd_workspace_size_for_block")
    return int(nb.value)


def rlk_linear_kl_fwd(h_s, W_s, h_t, W_t, mask, temperature: float,
                      workspace: Optional[torch.Tensor] = None,
                      block_tokens: Optional[int] = None):
    """Forward and reverse full-vocabulary KL per token; returns (kl_fwd, kl_rev, lse_s, lse_t),
    each [N] float32.  block_tokens: token blocks of that many tokens (a multiple of 256), in a
    workspace of that size, instead of the default's."""
    mask = _mask_u8(mask)
    _check_kl(h_s, W_s, h_t, W_t, mask)
    N, Hs = h_s.shape
    Ht = h_t.shape[1]
    V = W_s.shape[0]
    dt = _dtype_code(h_s)
    dev = h_s.device
    outs = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(4)]
    nb = kl_fwd_workspace_bytes(N, Hs, Ht, V, dt, block_tokens)
    ws = _workspace(nb, dev, workspace) if block_tokens is not None else \
        _sized_workspace(nb, dev, workspace)
    # the block size follows from the bytes passed: exactly the query's for block_tokens
    wsb = nb if block_tokens is not None else ws.numel() * ws.element_size()
    L.check(L.lib().rlk_linear_kl_fwd(_vp(h_s), _vp(W_s), _vp(h_t), _vp(W_t), _vp(mask), N, Hs,
                                      Ht, V, dt, float(temperature), *(_vp(o) for o in outs),
                                      _vp(ws), wsb, _stream(dev)),
            "rlk_linear_kl_fwd")
    return tuple(outs)


def rlk_linear_kl_bwd(h_s, W_s, h_t, W_t, mask, temperature: float,
                      coef_fwd: Optional[torch.Tensor], coef_rev: Optional[torch.Tensor],
                      lse_s: torch.Tensor, lse_t: torch.Tensor,
                      kl_rev: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """Gradients of L = sum_t mask_t (coef_fwd_t KL_fwd[t] + coef_rev_t KL_rev[t]) into the
    student (either coefficient may be None, not both); returns (dh_s, dW_s)."""
    mask = _mask_u8(mask)
    _check_kl(h_s, W_s, h_t, W_t, mask)
    N, Hs = h_s.shape
    Ht = h_t.shape[1]
    V = W_s.shape[0]
    dt = _dtype_code(h_s)
    dev = h_s.device
    if coef_fwd is None and coef_rev is None:
        raise ValueError("coef_fwd and coef_rev cannot both be None")
    for name, t in (("coef_fwd", coef_fwd), ("coef_rev", coef_rev)):
        if t is not None:
            _vec(name, t, N)
    _vec("lse_s", lse_s, N)
    _vec("lse_t", lse_t, N)
    if coef_rev is not None:
        if kl_rev is None:
            raise ValueError("kl_rev is required with coef_rev")
        _vec("kl_rev", kl_rev, N)
    dh = torch.empty((N, Hs), dtype=torch.float32, device=dev)
    dW = torch.empty((V, Hs), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    L.check(L.lib().rlk_linear_kl_bwd_workspace_size(N, Hs, Ht, V, dt, ctypes.byref(nb)),
            "rlk_linear_kl_bwd_workspace_size")
    ws = _workspace(int(nb.value), dev, workspace)
    L.check(L.lib().rlk_linear_kl_bwd(_vp(h_s), _vp(W_s), _vp(h_t), _vp(W_t), _vp(mask), N, Hs,
                                      Ht, V, dt, float(temperature), _vp(coef_fwd),
                                      _vp(coef_rev), _vp(lse_s), _vp(lse_t), _vp(kl_rev),
                                      _vp(dh), _vp(dW), _vp(ws), ws.numel() * ws.element_size(),
                                      _stream(dev)),
            "rlk_linear_kl_bwd")
    return dh, dW


class LinearKL(torch.autograd.Function):
    """(kl_fwd, kl_rev) = linear_kl(h_s, W_s, h_t, W_t, mask, T); gradients reach the student
    only, through one rlk_linear_kl_bwd call with coef_fwd = dL/dkl_fwd and coef_rev =
    dL/dkl_rev (None for a direction that receives no gradient)."""

    @staticmethod
    def forward(ctx, h_s, W_s, h_t, W_t, mask, temperature):
        kf, kr, ls, lt = rlk_linear_kl_fwd(h_s, W_s, h_t, W_t, mask, temperature)
        ctx.save_for_backward(h_s, W_s, h_t, W_t, mask, ls, lt, kr)
        ctx.temperature = float(temperature)
        return kf, kr

    @staticmethod
    def backward(ctx, grad_fwd, grad_rev):
        h_s, W_s, h_t, W_t, mask, ls, lt, kr = ctx.saved_tensors
        if grad_fwd is None and grad_rev is None:
            return None, None, None, None, None, None
        cf = None if grad_fwd is None else grad_fwd.to(torch.float32).contiguous()
        cr = None if grad_rev is None else grad_rev.to(torch.float32).contiguous()
        dh, dW = rlk_linear_kl_bwd(h_s, W_s, h_t, W_t, mask, ctx.temperature, cf, cr, ls, lt, kr)
        return dh.to(h_s.dtype), dW.to(W_s.dtype), None, None, None, None


def linear_kl(h_s, W_s, h_t, W_t, mask, temperature):
    """Differentiable forward and reverse full-vocabulary KL per token, each [N] (float32);
    the teacher (h_t, W_t) receives no gradient."""
    return LinearKL.apply(h_s, W_s, h_t, W_t, mask, temperature)
