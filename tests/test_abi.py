"""The C-ABI library loads, exports every symbol include/rlk.h declares, and rejects bad
arguments on the host before any device work (no GPU needed: only calls that return
before touching HIP are made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlk.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(os.path.join(ROOT, "linear_selected_token_amd", "librlk.so")):
        import __graft_entry__
        __graft_entry__.build()
    from linear_selected_token_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlk_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("rlk_linear_logp_fwd", "rlk_linear_logp_bwd", "rlk_status_string",
              "rlk_build_info", "rlk_linear_logp_fwd_workspace_size",
              "rlk_linear_logp_bwd_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    names = declared_functions()
    assert set(names) == set(L.SIGNATURES), "binding signatures out of step with the header"
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(rlk_\w+)\b", out))
    assert set(names) <= exported


def test_library_carries_gfx950_code(L):
    # the embedded offload bundle names its target (our own build output)
    data = open(L.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_and_build_info(L):
    lib = L.lib()
    for s in range(5):
        assert lib.rlk_status_string(s).decode().startswith("RLK_")
    assert b"unknown" in lib.rlk_status_string(99)
    info = lib.rlk_build_info().decode()
    assert "gfx950" in info and "vocab partial 128" in info
    assert lib.rlk_num_vocab_partials(151936) == 1187
    assert lib.rlk_num_vocab_partials(1000) == 8
    assert lib.rlk_num_vocab_partials(128) == 1
    assert lib.rlk_num_vocab_partials(0) == 0


def _ws(lib, fn, *args):
    out = ctypes.c_size_t(0)
    st = getattr(lib, fn)(*args, ctypes.byref(out))
    return st, out.value


def test_workspace_queries(L):
    lib = L.lib()
    st, a = _ws(lib, "rlk_linear_logp_fwd_workspace_size", 16384, 4096, 151936, L.RLK_BF16)
    assert st == 0 and a >= 2 * 4 * 16384 * 1187
    st, b = _ws(lib, "rlk_linear_logp_fwd_workspace_size", 8192, 4096, 151936, L.RLK_BF16)
    assert st == 0 and b < a
    st, c = _ws(lib, "rlk_linear_logp_bwd_workspace_size", 4096, 4096, 151936, L.RLK_BF16)
    assert st == 0 and c > 0
    # the backward's buffers hold one token block (11008 tokens at H = 4096): past it only the
    # index grows, and the Qwen3-8B head's backward needs under 1 GB at 16384 tokens (its
    # active tokens' bf16 logits alone would take ~3 GB)
    st, d = _ws(lib, "rlk_linear_logp_bwd_workspace_size", 16384, 4096, 151936, L.RLK_BF16)
    assert st == 0 and d <= 1_000_000_000
    st, e = _ws(lib, "rlk_linear_logp_bwd_workspace_size", (1 << 22) - 256, 256, 151936,
                L.RLK_BF16)
    st2, f = _ws(lib, "rlk_linear_logp_bwd_workspace_size", 65536, 256, 151936, L.RLK_BF16)
    assert st == 0 and st2 == 0 and e - f <= 12 * ((1 << 22) - 256 - 65536) + 1024
    assert f <= 1_000_000_000 + 4 * 65536 + 8192
    assert _ws(lib, "rlk_linear_logp_bwd_workspace_size", 4096, 4096, 151936, L.RLK_FP32)[0] == \
        L.RLK_ERROR_UNSUPPORTED
    assert _ws(lib, "rlk_linear_logp_fwd_workspace_size", 10, 100, 50, L.RLK_BF16)[0] == \
        L.RLK_ERROR_UNSUPPORTED
    assert _ws(lib, "rlk_linear_logp_fwd_workspace_size", -1, 64, 50, L.RLK_BF16)[0] == \
        L.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_linear_logp_fwd_workspace_size(4, 64, 8, 0, None) == L.RLK_ERROR_INVALID_VALUE


FAKE = 1 << 20  # aligned non-null stand-in address: these calls fail validation first


def _fwd(lib, h=FAKE, W=FAKE, tg=FAKE, m=FAKE, N=8, H=64, V=100, dt=0, T=1.0, lp=FAKE,
         lse=FAKE, ws=FAKE, wsb=1 << 30):
    return lib.rlk_linear_logp_fwd(h, W, tg, m, N, H, V, dt, T, lp, lse, ws, wsb, None)


def test_forward_argument_errors(L):
    lib = L.lib()
    E = L
    assert _fwd(lib, N=0) == E.RLK_SUCCESS  # nothing to do, nothing touched
    assert _fwd(lib, h=None) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, W=None) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, tg=None) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, m=None) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, lp=None) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, ws=None) == E.RLK_ERROR_INVALID_VALUE
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert _fwd(lib, T=T) == E.RLK_ERROR_INVALID_VALUE, T
    assert _fwd(lib, N=-1) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, V=0) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, H=0) == E.RLK_ERROR_INVALID_VALUE
    assert _fwd(lib, dt=2) == E.RLK_ERROR_UNSUPPORTED
    assert _fwd(lib, H=96) == E.RLK_ERROR_UNSUPPORTED
    assert _fwd(lib, N=1 << 23) == E.RLK_ERROR_UNSUPPORTED
    # h of 2 GiB: past the 32-bit row offsets of the tile loads
    assert _fwd(lib, N=1 << 18, H=4096) == E.RLK_ERROR_UNSUPPORTED
    # one row less passes the shape checks (and stops at the workspace size, before any launch)
    assert _fwd(lib, N=(1 << 18) - 1, H=4096, wsb=1000) == E.RLK_ERROR_WORKSPACE
    assert _fwd(lib, h=FAKE + 8) == E.RLK_ERROR_UNSUPPORTED
    assert _fwd(lib, W=FAKE + 4) == E.RLK_ERROR_UNSUPPORTED
    assert _fwd(lib, ws=FAKE + 16) == E.RLK_ERROR_UNSUPPORTED
    assert _fwd(lib, wsb=1000) == E.RLK_ERROR_WORKSPACE


def test_backward_argument_errors(L):
    lib = L.lib()
    E = L

    def bwd(h=FAKE, adv=FAKE, lse=FAKE, dh=FAKE, dW=FAKE, N=8, H=256, dt=0, T=1.0, wsb=1 << 30):
        return lib.rlk_linear_logp_bwd(h, FAKE, FAKE, FAKE, N, H, 100, dt, T, adv, lse, dh, dW,
                                       FAKE, wsb, None)

    assert bwd(adv=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(lse=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(dh=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(dW=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(T=0.0) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(dt=1) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(H=192) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(wsb=10) == E.RLK_ERROR_WORKSPACE


def test_fused_workspace_and_argument_errors(L):
    lib = L.lib()
    E = L
    # the fused call's buffers hold one token block (2816 tokens at H = 4096, V = 151936: a
    # row of 152128 two-byte entries per token is most of it); past it only the index grows
    st, a = _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 16384, 4096, 151936, L.RLK_BF16)
    assert st == 0 and a <= 1_000_000_000
    st, b = _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 2816, 4096, 151936, L.RLK_BF16)
    assert st == 0 and 0 <= a - b <= 4 * (16384 - 2816) + 1024
    st, c = _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 2816, 4096, 151936, L.RLK_BF16)
    assert c >= 2816 * (2 * 152128 + 8 * 1187 + 6 * 4096)
    st, d = _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 600, 512, 3000, L.RLK_BF16)
    assert st == 0 and d < b
    assert _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 64, 4096, 151936,
               L.RLK_FP32)[0] == E.RLK_ERROR_UNSUPPORTED
    assert _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 64, 320, 1000,
               L.RLK_BF16)[0] == E.RLK_ERROR_UNSUPPORTED
    # a vocabulary of 2^22 entries leaves room for 256 tokens per block: 2^22 tokens would need
    # more than 1024 blocks
    assert _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", (1 << 22) - 256, 256, 1 << 22,
               L.RLK_BF16)[0] == E.RLK_ERROR_UNSUPPORTED

    # the workspace sets the block size: the size for blocks of block_tokens grows with it (0:
    # the budget's blocks), and stops growing at one block
    sizes = [_ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size_for_block", 16384, 4096, 151936,
                 L.RLK_BF16, bt) for bt in (0, 2816, 2817, 5000, 9831, 16384, 1 << 30, 256, 300)]
    assert all(st == 0 for st, _ in sizes)
    v = [x for _, x in sizes]
    assert v[0] == v[1] == a and a < v[2] <= v[3] < v[4] < v[5] == v[6]
    assert v[7] < v[8] < a  # 256-token blocks, and 300 rounded up to 512
    assert v[4] >= 9984 * (2 * 152128 + 8 * 1187 + 6 * 4096)
    assert _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size_for_block", 16384, 4096, 151936,
               L.RLK_BF16, -1)[0] == E.RLK_ERROR_INVALID_VALUE

    def fused(h=FAKE, adv=FAKE, lp=FAKE, lse=FAKE, dh=FAKE, dW=FAKE, N=8, H=256, dt=0, T=1.0,
              wsb=1 << 30):
        return lib.rlk_linear_logp_fwd_bwd(h, FAKE, FAKE, FAKE, N, H, 100, dt, T, adv, lp, lse,
                                           dh, dW, FAKE, wsb, None)

    assert fused(h=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(adv=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(lp=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(lse=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(dh=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(dW=None) == E.RLK_ERROR_INVALID_VALUE
    assert fused(T=float("nan")) == E.RLK_ERROR_INVALID_VALUE
    assert fused(dt=1) == E.RLK_ERROR_UNSUPPORTED
    assert fused(H=192) == E.RLK_ERROR_UNSUPPORTED
    assert fused(dh=FAKE + 4) == E.RLK_ERROR_UNSUPPORTED  # dh holds 16-byte vectors
    assert fused(lse=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert fused(wsb=10) == E.RLK_ERROR_WORKSPACE


def test_fused_ppo_argument_errors(L):
    lib = L.lib()
    E = L
    st, a = _ws(lib, "rlk_linear_ppo_fwd_bwd_workspace_size", 16384, 4096, 151936, L.RLK_BF16)
    st2, b = _ws(lib, "rlk_linear_logp_fwd_bwd_workspace_size", 16384, 4096, 151936, L.RLK_BF16)
    assert st == 0 and st2 == 0 and b < a <= b + 1024

    def ppo(old=FAKE, adv=FAKE, loss=FAKE, badv=FAKE, ratio=None, sums=None, eps_lo=0.2,
            eps_hi=0.2, beta=0.0, scale=1.0, ws=FAKE, wsb=1 << 30, N=8, H=256, dt=0):
        return lib.rlk_linear_ppo_fwd_bwd(FAKE, FAKE, FAKE, FAKE, N, H, 100, dt, 1.0, old, None,
                                          adv, eps_lo, eps_hi, beta, scale, FAKE, FAKE, loss,
                                          badv, ratio, sums, FAKE, FAKE, ws, wsb, None)

    assert ppo(old=None) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(adv=None) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(loss=None) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(badv=None) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(ws=None) == E.RLK_ERROR_INVALID_VALUE
    for lo in (-0.1, 1.0, float("nan")):
        assert ppo(eps_lo=lo) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(eps_hi=-1.0) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(beta=float("inf")) == E.RLK_ERROR_INVALID_VALUE
    assert ppo(ratio=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert ppo(sums=FAKE + 4) == E.RLK_ERROR_UNSUPPORTED
    assert ppo(dt=1) == E.RLK_ERROR_UNSUPPORTED
    assert ppo(H=192) == E.RLK_ERROR_UNSUPPORTED
    assert ppo(wsb=10) == E.RLK_ERROR_WORKSPACE
    assert ppo(wsb=1024) == E.RLK_ERROR_WORKSPACE  # the loss partials fit, the rest does not


def test_building_block_argument_errors(L):
    lib = L.lib()
    E = L
    assert lib.rlk_compact_active(FAKE, -1, FAKE, FAKE, None, None, None, None) == \
        E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_compact_active(None, 5, FAKE, FAKE, None, None, None, None) == \
        E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_compact_active(FAKE, 5, FAKE, None, None, None, None, None) == \
        E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_linear_logp_partials(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 10, 0, 0.0, FAKE,
                                        FAKE, FAKE, None) == E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_linear_logp_partials(FAKE, FAKE, FAKE, FAKE, None, 4, 64, 10, 0, 1.0, FAKE,
                                        FAKE, FAKE, None) == E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_linear_logp_merge(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, FAKE, None, None) == \
        E.RLK_ERROR_INVALID_VALUE
    assert lib.rlk_linear_logp_merge(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, FAKE, None, None) == \
        E.RLK_SUCCESS


def _shard(lib, V=256, start=0, Vg=1000, N=4, H=64, h=FAKE, idx=FAKE):
    return lib.rlk_linear_logp_partials_shard(h, FAKE, FAKE, idx, FAKE, N, H, V, start, Vg, 0,
                                              1.0, FAKE, FAKE, FAKE, None)


def test_vocabulary_shard_argument_errors(L):
    # every case below is decided on the host, before anything could be launched
    lib = L.lib()
    E = L
    assert _shard(lib, start=-128) == E.RLK_ERROR_INVALID_VALUE       # before the vocabulary
    assert _shard(lib, start=768, V=256) == E.RLK_ERROR_INVALID_VALUE  # past its end
    assert _shard(lib, Vg=0) == E.RLK_ERROR_INVALID_VALUE
    assert _shard(lib, start=64) == E.RLK_ERROR_UNSUPPORTED            # splits a column
    assert _shard(lib, V=200, start=128) == E.RLK_ERROR_UNSUPPORTED    # ends inside a column
    assert _shard(lib, Vg=1 << 23, V=256) == E.RLK_ERROR_UNSUPPORTED
    # a ragged last shard passes the shard checks (and stops at the missing index buffer)
    assert _shard(lib, V=1000 - 896, start=896, idx=None) == E.RLK_ERROR_INVALID_VALUE
    assert _shard(lib, N=0, V=1000 - 896, start=896) == E.RLK_SUCCESS


def _lg(lib, lg=FAKE, ld=1008, N=4, V=1000, dt=0, T=1.0, ws=FAKE, wsb=1 << 30):
    return lib.rlk_logp_from_logits(lg, ld, FAKE, FAKE, N, V, dt, T, FAKE, FAKE, ws, wsb, None)


def test_logits_path_argument_errors(L):
    # every case is decided on the host, before anything could be launched
    lib = L.lib()
    E = L
    assert _lg(lib, N=0) == E.RLK_SUCCESS
    assert _lg(lib, lg=None) == E.RLK_ERROR_INVALID_VALUE
    assert _lg(lib, ld=999) == E.RLK_ERROR_INVALID_VALUE          # row shorter than V
    assert _lg(lib, ld=1004) == E.RLK_ERROR_UNSUPPORTED           # 2008-byte rows
    assert _lg(lib, dt=1, ld=1002) == E.RLK_ERROR_UNSUPPORTED     # 4008-byte rows
    assert _lg(lib, lg=FAKE + 8) == E.RLK_ERROR_UNSUPPORTED
    assert _lg(lib, dt=2) == E.RLK_ERROR_UNSUPPORTED
    assert _lg(lib, T=0.0) == E.RLK_ERROR_INVALID_VALUE
    assert _lg(lib, wsb=100) == E.RLK_ERROR_WORKSPACE
    assert _lg(lib, V=1024001, ld=1024008) == E.RLK_ERROR_UNSUPPORTED  # past the LDS budget
    size = ctypes.c_size_t(0)
    assert lib.rlk_logp_from_logits_workspace_size(4, 1000, ctypes.byref(size)) == E.RLK_SUCCESS
    assert size.value > 0


def _ent(lib, ent=FAKE, N=8, H=64, V=1000, dt=0, T=1.0, ws=FAKE, wsb=1 << 30):
    return lib.rlk_linear_logp_fwd_entropy(FAKE, FAKE, FAKE, FAKE, N, H, V, dt, T, FAKE, FAKE,
                                           ent, ws, wsb, None)


def test_entropy_forward_workspace_and_argument_errors(L):
    # every case is decided on the host, before anything could be launched
    lib = L.lib()
    E = L
    N, H, V = 16384, 4096, 151936
    st, plain = _ws(lib, "rlk_linear_logp_fwd_workspace_size", N, H, V, L.RLK_BF16)
    st2, ent = _ws(lib, "rlk_linear_logp_fwd_entropy_workspace_size", N, H, V, L.RLK_BF16)
    assert st == 0 and st2 == 0
    # one more float per token and 128-entry column
    assert ent - plain == 4 * N * 1187
    assert _ws(lib, "rlk_linear_logp_fwd_entropy_workspace_size", 10, 100, 50, 0)[0] == \
        E.RLK_ERROR_UNSUPPORTED
    _, small = _ws(lib, "rlk_linear_logp_fwd_workspace_size", 8, 64, 1000, 0)
    assert _ent(lib, N=0) == E.RLK_SUCCESS
    assert _ent(lib, wsb=small) == E.RLK_ERROR_WORKSPACE   # the plain forward's is too small
    assert _ent(lib, ent=None) == E.RLK_ERROR_INVALID_VALUE
    assert _ent(lib, ent=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert _ent(lib, T=float("nan")) == E.RLK_ERROR_INVALID_VALUE
    assert _ent(lib, H=96) == E.RLK_ERROR_UNSUPPORTED


def test_entropy_backward_argument_errors(L):
    lib = L.lib()
    E = L

    def bwd(c=FAKE, ent=FAKE, N=8, H=256, dt=0, wsb=1 << 30):
        return lib.rlk_linear_logp_bwd_entropy(FAKE, FAKE, FAKE, FAKE, N, H, 100, dt, 1.0, FAKE,
                                               c, FAKE, ent, FAKE, FAKE, FAKE, wsb, None)

    assert bwd(c=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(ent=None) == E.RLK_ERROR_INVALID_VALUE
    assert bwd(c=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(dt=1) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(H=192) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(wsb=10) == E.RLK_ERROR_WORKSPACE


def test_loss_fragment_argument_errors(L):
    # every case is decided on the host, before anything could be launched
    lib = L.lib()
    E = L

    def loss(N=8, eps_lo=0.2, eps_hi=0.2, beta=0.0, scale=1.0, lp=FAKE, ws=FAKE, wsb=1 << 20):
        return lib.rlk_ratio_kl_loss(lp, FAKE, None, FAKE, FAKE, N, eps_lo, eps_hi, beta, scale,
                                     FAKE, FAKE, None, None, ws, wsb, None)

    assert loss(N=-1) == E.RLK_ERROR_INVALID_VALUE
    assert loss(N=1 << 23) == E.RLK_ERROR_UNSUPPORTED
    assert loss(eps_lo=1.0) == E.RLK_ERROR_INVALID_VALUE
    assert loss(eps_lo=-0.1) == E.RLK_ERROR_INVALID_VALUE
    assert loss(eps_hi=float("nan")) == E.RLK_ERROR_INVALID_VALUE
    assert loss(beta=float("inf")) == E.RLK_ERROR_INVALID_VALUE
    assert loss(scale=float("nan")) == E.RLK_ERROR_INVALID_VALUE
    assert loss(lp=None) == E.RLK_ERROR_INVALID_VALUE
    assert loss(ws=None) == E.RLK_ERROR_INVALID_VALUE
    assert loss(lp=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert loss(ws=FAKE + 64) == E.RLK_ERROR_UNSUPPORTED
    assert loss(wsb=16) == E.RLK_ERROR_WORKSPACE
    st, b1 = _ws(lib, "rlk_ratio_kl_loss_workspace_size", 1 << 20)
    assert st == 0 and b1 >= 32 * 1024

    def diag(N=8, eps=0.2, a=FAKE, out=FAKE, worst=FAKE, wsb=1 << 20):
        return lib.rlk_dlogp_diagnostics(a, FAKE, FAKE, N, eps, out, worst, FAKE, wsb, None)

    assert diag(N=-1) == E.RLK_ERROR_INVALID_VALUE
    assert diag(eps=-1.0) == E.RLK_ERROR_INVALID_VALUE
    assert diag(out=None) == E.RLK_ERROR_INVALID_VALUE
    assert diag(worst=None) == E.RLK_ERROR_INVALID_VALUE
    assert diag(a=None) == E.RLK_ERROR_INVALID_VALUE
    assert diag(out=FAKE + 4) == E.RLK_ERROR_UNSUPPORTED
    assert diag(wsb=100) == E.RLK_ERROR_WORKSPACE
    st, b2 = _ws(lib, "rlk_dlogp_diagnostics_workspace_size", 1 << 20)
    assert st == 0 and b2 >= 12 * (1 << 20)


def test_kl_argument_errors(L):
    # every case is decided on the host, before anything could be launched
    lib = L.lib()
    E = L

    def fwd(N=8, Hs=64, Ht=128, V=1000, dt=0, T=1.0, hs=FAKE, ht=FAKE, kf=FAKE, wsb=1 << 40):
        return lib.rlk_linear_kl_fwd(hs, FAKE, ht, FAKE, FAKE, N, Hs, Ht, V, dt, T, kf, FAKE, None,
                                     None, FAKE, wsb, None)

    assert fwd(N=0) == E.RLK_SUCCESS
    assert fwd(hs=None) == E.RLK_ERROR_INVALID_VALUE
    assert fwd(ht=None) == E.RLK_ERROR_INVALID_VALUE
    assert fwd(kf=None) == E.RLK_ERROR_INVALID_VALUE
    assert fwd(Ht=96) == E.RLK_ERROR_UNSUPPORTED
    assert fwd(ht=FAKE + 8) == E.RLK_ERROR_UNSUPPORTED
    assert fwd(T=0.0) == E.RLK_ERROR_INVALID_VALUE
    assert fwd(wsb=1000) == E.RLK_ERROR_WORKSPACE
    st, b = _ws(lib, "rlk_linear_kl_fwd_workspace_size", 16384, 4096, 2048, 151936, 0)
    # six [J][Npad] statistics for one token block (all 16384 tokens fit the forward's own
    # capacity of 32512 at V = 151936) and the 64 MiB scratch of the tile kernel: under 1e9 bytes
    assert st == 0 and b >= 6 * 4 * 16384 * 1187 + (64 << 20)
    assert b <= 1_000_000_000
    # past one token block only the index grows with N
    st1, b1 = _ws(lib, "rlk_linear_kl_fwd_workspace_size", 65536, 4096, 2048, 151936, 0)
    st2, b2 = _ws(lib, "rlk_linear_kl_fwd_workspace_size", 131072, 4096, 2048, 151936, 0)
    assert st1 == st2 == 0 and b1 <= 1_000_000_000 + 4 * 65536 + 8192
    assert b2 - b1 <= 4 * 65536 + 512
    # a workspace sized for 3584-token blocks (six at N = 20000, V = 2000) is smaller than the
    # default's one block; block sizes are positive multiples of 256, at most 1024 blocks
    sd = _ws(lib, "rlk_linear_kl_fwd_workspace_size", 20000, 256, 128, 2000, 0)
    sb = _ws(lib, "rlk_linear_kl_fwd_workspace_size_for_block", 20000, 256, 128, 2000, 0, 3584)
    assert sd[0] == sb[0] == 0 and sb[1] < sd[1]
    assert sb[1] >= 6 * 4 * 3584 * 16 + (64 << 20)
    for bad in (0, -256, 300):
        assert _ws(lib, "rlk_linear_kl_fwd_workspace_size_for_block", 20000, 256, 128, 2000, 0,
                   bad)[0] == E.RLK_ERROR_INVALID_VALUE
    assert _ws(lib, "rlk_linear_kl_fwd_workspace_size_for_block", 1 << 20, 256, 256, 2000, 0,
               256)[0] == E.RLK_ERROR_UNSUPPORTED
    # a workspace below the smallest blocks' is refused before anything is launched
    assert fwd(wsb=sb[1] // 4) == E.RLK_ERROR_WORKSPACE
    # a vocabulary of 2^22 entries leaves 256 tokens per block: 2^22 tokens would need more than
    # 1024 blocks
    assert _ws(lib, "rlk_linear_kl_fwd_workspace_size", (1 << 22) - 256, 256, 256, 1 << 22,
               0)[0] == E.RLK_ERROR_UNSUPPORTED

    def bwd(Hs=256, dt=0, cf=FAKE, cr=None, kr=FAKE, wsb=1 << 40, dh=FAKE):
        return lib.rlk_linear_kl_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, 8, Hs, 64, 1000, dt, 1.0, cf, cr,
                                     FAKE, FAKE, kr, dh, FAKE, FAKE, wsb, None)

    assert bwd(Hs=64) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(dt=1) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(cf=None) == E.RLK_ERROR_INVALID_VALUE            # no coefficient at all
    assert bwd(cf=None, cr=FAKE, kr=None) == E.RLK_ERROR_INVALID_VALUE  # reverse needs kl_rev
    assert bwd(cr=FAKE + 2) == E.RLK_ERROR_UNSUPPORTED
    assert bwd(dh=FAKE + 4) == E.RLK_ERROR_UNSUPPORTED          # dh_s: 16 bytes
    assert bwd(wsb=1000) == E.RLK_ERROR_WORKSPACE
    assert bwd(cf=None, cr=FAKE, wsb=1000) == E.RLK_ERROR_WORKSPACE
    assert _ws(lib, "rlk_linear_kl_bwd_workspace_size", 8, 64, 64, 1000, 0)[0] == \
        E.RLK_ERROR_UNSUPPORTED
    # the backward's buffers for blocks of 10240 tokens (H_s = 4096) and the scratch: within
    # 1e9 bytes but for the index, and no growth past one block but the index
    st, b = _ws(lib, "rlk_linear_kl_bwd_workspace_size", 16384, 4096, 4096, 151936, 0)
    assert st == 0 and b <= 1_000_000_000 + 4 * 16384 + 8192
    st2, b2 = _ws(lib, "rlk_linear_kl_bwd_workspace_size", 65536, 4096, 4096, 151936, 0)
    assert st2 == 0 and b2 - b <= 4 * (65536 - 16384) + 8 * 8 + 512
