"""The forward entry point without a workspace (the library's static scratch serves as its
workspace): called through the C ABI, its outputs are bit-identical to rlk_linear_logp_fwd's
with a caller-provided workspace, on two calls in a row (the second smaller, so it runs over
what the first left in the scratch), and a call whose workspace would not fit the scratch is
refused before anything is written (needs an MI355X)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bits, flush, upload

pytestmark = pytest.mark.gpu


def _noalloc(d, w, logp, lse):
    from linear_selected_token_amd import _lib
    N, H = d["h"].shape
    V = d["W"].shape[0]
    dt = _lib.RLK_BF16 if d["h"].dtype == torch.bfloat16 else _lib.RLK_FP32
    st = _lib.lib().rlk_linear_logp_fwd_noalloc(
        ctypes.c_void_p(d["h"].data_ptr()), ctypes.c_void_p(d["W"].data_ptr()),
        ctypes.c_void_p(d["targets"].data_ptr()), ctypes.c_void_p(d["mask"].data_ptr()),
        N, H, V, dt, w.T, ctypes.c_void_p(logp.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _check_one(w):
    import linear_selected_token_amd as rlk
    d = upload(w)
    N = w.N
    ref_lp, ref_lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    logp = torch.full((N,), 7.0, dtype=torch.float32, device=d["h"].device)
    lse = torch.full((N,), 7.0, dtype=torch.float32, device=d["h"].device)
    st = _noalloc(d, w, logp, lse)
    torch.cuda.synchronize()
    assert st == 0, st
    a, b = logp.cpu().numpy(), ref_lp.cpu().numpy()
    flush(f"  no-alloc forward N={N} H={w.H} V={w.V} ({w.n_active} active): "
          f"{int((bits(a) != bits(b)).sum())} logp bit mismatches")
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(lse.cpu().numpy()), bits(ref_lse.cpu().numpy()))


def test_no_alloc_forward_matches_workspace_forward():
    # the Qwen3-8B head with 4096 tokens (~50% active: ~39 MB of the 64 MiB scratch), then a
    # small head with 600 tokens over what the first call left behind
    _check_one(wl.make(wl.scaled_spec(5, N=4096, n_seq=16, len_lo=64, len_hi=512, seed=171)))
    _check_one(wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                                      seed=172, T=0.7)))


def test_no_alloc_forward_refuses_what_does_not_fit():
    from linear_selected_token_amd import _lib
    # 8192 tokens of the Qwen3-8B vocabulary need ~78 MB of workspace, more than the scratch
    N, H, V = 8192, 256, 151936
    nb = ctypes.c_size_t(0)
    assert _lib.lib().rlk_linear_logp_fwd_workspace_size(N, H, V, _lib.RLK_BF16,
                                                         ctypes.byref(nb)) == 0
    assert nb.value > _lib.RLK_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda", 0)
    h = torch.zeros((N, H), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=dev)
    d = dict(h=h, W=W, targets=torch.zeros(N, dtype=torch.int32, device=dev),
             mask=torch.ones(N, dtype=torch.uint8, device=dev))

    class _W:
        T = 1.0
    logp = torch.full((N,), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((N,), 7.0, dtype=torch.float32, device=dev)
    st = _noalloc(d, _W, logp, lse)
    torch.cuda.synchronize()
    assert st == _lib.RLK_ERROR_WORKSPACE, st
    assert bool((logp == 7.0).all()) and bool((lse == 7.0).all())
