"""ctypes loader of ``librlk.so`` (built in-tree by ``linear_selected_token_amd/build.py``).

There is no fallback: if the library is missing or cannot be loaded, importing the
binding raises, so a run never silently computes on another path."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librlk.so")

RLK_SUCCESS = 0
RLK_ERROR_INVALID_VALUE = 1
RLK_ERROR_UNSUPPORTED = 2
RLK_ERROR_WORKSPACE = 3
RLK_ERROR_DEVICE = 4
RLK_BF16 = 0
RLK_FP32 = 1
RLK_VOCAB_PARTIAL = 128
RLK_NOALLOC_SCRATCH_BYTES = 64 << 20

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes); every symbol include/rlk.h declares
SIGNATURES = {
    "rlk_status_string": (ctypes.c_char_p, [_int]),
    "rlk_build_info": (ctypes.c_char_p, []),
    "rlk_num_vocab_partials": (_i64, [_i64]),
    "rlk_linear_logp_fwd_workspace_size": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_sz)]),
    "rlk_linear_logp_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_sz)]),
    "rlk_linear_logp_fwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p, _p, _sz, _p]),
    "rlk_linear_logp_fwd_noalloc": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p,
                                           _p]),
    "rlk_linear_logp_fwd_entropy_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                                          ctypes.POINTER(_sz)]),
    "rlk_linear_logp_fwd_entropy": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p,
                                           _p, _p, _sz, _p]),
    "rlk_linear_logp_bwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p, _p, _p,
                                   _p, _sz, _p]),
    "rlk_linear_logp_bwd_entropy": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p, _p,
                                           _p, _p, _p, _p, _sz, _p]),
    "rlk_linear_logp_fwd_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                                      ctypes.POINTER(_sz)]),
    "rlk_linear_logp_fwd_bwd_workspace_size_for_block": (_int, [_i64, _i64, _i64, _int, _i64,
                                                                ctypes.POINTER(_sz)]),
    "rlk_linear_logp_fwd_bwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p, _p,
                                       _p, _p, _p, _sz, _p]),
    "rlk_linear_logp_fwd_bwd_entropy_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                                              ctypes.POINTER(_sz)]),
    "rlk_linear_logp_fwd_bwd_entropy": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p,
                                               _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "rlk_linear_ppo_fwd_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                                     ctypes.POINTER(_sz)]),
    "rlk_linear_ppo_fwd_bwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p, _p,
                                      _f, _f, _f, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                                      _p]),
    "rlk_compact_active": (_int, [_p, _i64, _p, _p, _p, _p, _p, _p]),
    "rlk_linear_logp_partials": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _int, _f, _p, _p,
                                        _p, _p]),
    "rlk_linear_logp_partials_shard": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                                              _int, _f, _p, _p, _p, _p]),
    "rlk_linear_logp_merge": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _p, _p, _p]),
    "rlk_linear_kl_fwd_workspace_size": (_int, [_i64, _i64, _i64, _i64, _int,
                                                ctypes.POINTER(_sz)]),
    "rlk_linear_kl_fwd_workspace_size_for_block": (_int, [_i64, _i64, _i64, _i64, _int, _i64,
                                                          ctypes.POINTER(_sz)]),
    "rlk_linear_kl_fwd": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _f, _p, _p, _p,
                                 _p, _p, _sz, _p]),
    "rlk_linear_kl_bwd_workspace_size": (_int, [_i64, _i64, _i64, _i64, _int,
                                                ctypes.POINTER(_sz)]),
    "rlk_linear_kl_bwd": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _f, _p, _p,
                                 _p, _p, _p, _p, _p, _p, _sz, _p]),
    "rlk_ratio_kl_loss_workspace_size": (_int, [_i64, ctypes.POINTER(_sz)]),
    "rlk_ratio_kl_loss": (_int, [_p, _p, _p, _p, _p, _i64, _f, _f, _f, _f, _p, _p, _p, _p, _p,
                                 _sz, _p]),
    "rlk_dlogp_diagnostics_workspace_size": (_int, [_i64, ctypes.POINTER(_sz)]),
    "rlk_dlogp_diagnostics": (_int, [_p, _p, _p, _i64, _f, _p, _p, _p, _sz, _p]),
    "rlk_logp_from_logits_workspace_size": (_int, [_i64, _i64, ctypes.POINTER(_sz)]),
    "rlk_logp_from_logits": (_int, [_p, _i64, _p, _p, _i64, _i64, _int, _f, _p, _p, _p, _sz,
                                    _p]),
}


class RlkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python linear_selected_token_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().rlk_status_string(int(status)).decode()


def build_info() -> str:
    return lib().rlk_build_info().decode()


def check(status: int, where: str) -> None:
    if status != RLK_SUCCESS:
        raise RlkError(status, where)
