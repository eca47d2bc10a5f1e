"""Backward parity of the HIP path against the float64 oracle (needs an MI355X).

L = -sum_t mask_t adv_t logp_t; gates: rel-L2 of dL/dh and dL/dW <= 1e-2.  A token's dL/dh
row is bit-identical across batch layouts; dL/dW is deterministic run to run."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (MAX_ABS_DLOGP, assert_rows, assert_tiles, bits, edge_rows,
                      device, flush, oracle_inputs, run_bwd, upload)

pytestmark = pytest.mark.gpu

SMALL = wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300, seed=95)


def _full_compare(w):
    """Every active dL/dh row and every dL/dW row on its own rel-L2, every 256 x 256 block of
    dL/dW too; inactive dL/dh rows exactly 0."""
    _, _, dh, dW = run_bwd(w)
    dh = dh.cpu().numpy()
    dW = dW.cpu().numpy()
    h64, W64 = oracle_inputs(w)
    odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, w.adv)
    act = np.nonzero(w.mask)[0]
    flush(f"  {w.spec.name} N={w.N} H={w.H} V={w.V} active={act.size}")
    assert_rows("dh (every active row)", dh[act], odh[act], act)
    assert_rows("dW (every vocabulary row)", dW, odW)
    assert_tiles("dW", dW, odW)
    assert not dh[w.mask == 0].any()
    return dh, dW


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_small_full(T):
    _full_compare(wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64,
                                         len_hi=300, seed=95, T=T)))


def _chunking():
    """(vocabulary entries per backward chunk, split point of dL/dh) of the loaded build."""
    import re
    import linear_selected_token_amd as rlk
    m = re.search(r"bwd chunk (\d+), dh split at (\d+)", rlk.build_info())
    assert m, rlk.build_info()
    return int(m.group(1)), int(m.group(2))


def test_two_chunks_ragged():
    # the vocabulary spans two backward chunks, both with entries past the dL/dh split point,
    # the second with a ragged tail; a ragged token tile
    chunk, split = _chunking()
    _full_compare(wl.make(wl.scaled_spec(5, N=300, H=256, V=chunk + split + 300, n_seq=2,
                                         len_lo=100, len_hi=200, seed=96)))


@pytest.mark.parametrize("dv", [0, 64, 3616])
def test_one_chunk_around_dh_split(dv):
    # one backward chunk whose vocabulary ends exactly at the dL/dh split point (one K half:
    # the second-half buffer is never written), one 64-entry stage past it, and well past it
    # (both halves stored by the first chunk's tiles)
    _, split = _chunking()
    _full_compare(wl.make(wl.scaled_spec(5, N=300, H=256, V=split + dv, n_seq=2, len_lo=100,
                                         len_hi=200, seed=97)))


@pytest.mark.parametrize("H", [256, 4096])
def test_schedules_agree_across_4096_tokens(H):
    # Batches of up to 4096 tokens run dL/dh and dL/dW of a chunk as one launch with claimed
    # tiles, larger ones as two launches in a fixed order.  The same tokens with 8 inactive
    # padding rows appended (4104 tokens) take the other schedule; every active dL/dh row and
    # all of dL/dW keep their bits (dL/dW sums the active tokens in the same order).  At
    # H = 4096 (the Qwen3-8B head) a chunk has 16 rounds of dL/dW claims and a partial last
    # round of dL/dh tiles dealt out over the XCDs before the claims start.
    import dataclasses
    w = wl.make(wl.scaled_spec(5, N=4096, H=H, V=70000, n_seq=16, len_lo=64, len_hi=512,
                               seed=131))
    pad = 8
    w2 = dataclasses.replace(
        w, h=np.concatenate([w.h, w.h[:pad]]),
        targets=np.concatenate([w.targets, np.zeros(pad, np.int32)]),
        mask=np.concatenate([w.mask, np.zeros(pad, np.uint8)]),
        adv=np.concatenate([w.adv, np.zeros(pad, np.float32)]),
        u=np.concatenate([w.u, np.zeros(pad)]),
        seq_id=np.concatenate([w.seq_id, np.full(pad, -1, np.int32)]),
        pos=np.concatenate([w.pos, np.zeros(pad, np.int32)]))
    act = torch.from_numpy(w.mask.astype(bool)).to(device())
    flush(f"  N={w.N} vs {w2.N}, H={H}, {int(act.sum())} active, V={w.V}")
    _, _, dh1, dW1 = run_bwd(w)
    _, _, dh2, dW2 = run_bwd(w2)
    assert torch.equal(dh1[act].view(torch.int32), dh2[:w.N][act].view(torch.int32))
    assert not dh2[:w.N][~act].any()
    assert torch.equal(dW1.view(torch.int32), dW2.view(torch.int32))


def _token_cap(H):
    """Token capacity of the backward's block buffers, by the rule the build states: the largest
    multiple of 256 tokens whose buffers (131200 + 14 H bytes per token) fit 1e9 bytes."""
    import re
    import linear_selected_token_amd as rlk
    m = re.search(r"multiple of 256 tokens whose buffers \((\d+) \+ (\d+) H bytes per token\) "
                  r"fit (\d+) bytes", rlk.build_info())
    assert m, rlk.build_info()
    a, b, budget = (int(x) for x in m.groups())
    return budget // (a + b * H) // 256 * 256


# ~60% active of 40000 tokens at H = 256 (blocks of at most 14848 tokens): two equal blocks of
# the backward and a third that holds no active token
MULTI = wl.scaled_spec(3, N=40000, H=256, V=3000, n_seq=110, len_lo=128, len_hi=512, seed=141,
                       targets="uniform", backward=True)


def test_token_blocks_full():
    # every active dL/dh row and every dL/dW row against the oracle when the active tokens
    # span more than one token block of the backward, with an empty last block
    w = wl.make(MULTI)
    cap = _token_cap(w.H)
    flush(f"  {w.n_active} active of {w.N}: token blocks of at most {cap}")
    assert cap < w.n_active < 2 * cap and w.N > 2 * cap
    _full_compare(w)


def test_token_blocks_dh_invariance_and_dw():
    # a token's dL/dh row keeps its bits whichever token block it falls in (alone, shuffled,
    # padded, all tokens active: 40000 active, three blocks); dL/dW is deterministic and does not
    # depend on padding or inactive rows (they never enter the compacted order)
    fam = wl.Family(MULTI)
    base = fam.batch()
    _, _, dh, dW = run_bwd(base)
    dh = dh.cpu().numpy()
    ref = {k: dh[i] for i, k in enumerate(base.key()) if base.mask[i]}
    for w in (fam.alone(17), fam.shuffled(7), fam.padded(8), fam.all_active()):
        _, _, dh2, _ = run_bwd(w)
        dh2 = dh2.cpu().numpy()
        n = 0
        for i, k in enumerate(w.key()):
            if k[0] >= 0 and w.mask[i] and k in ref:
                assert np.array_equal(bits(dh2[i]), bits(ref[k])), k
                n += 1
        flush(f"  {w.N} tokens, {w.n_active} active: {n} dh rows bit-identical")
    _, _, _, dW2 = run_bwd(base)
    assert torch.equal(dW.view(torch.int32), dW2.view(torch.int32))
    _, _, _, dW3 = run_bwd(fam.padded(9))
    assert torch.equal(dW.view(torch.int32), dW3.view(torch.int32))


def test_all_masked_backward():
    import linear_selected_token_amd as rlk
    w = wl.make(SMALL)
    d = upload(w)
    d["mask"].zero_()
    lse = torch.zeros(w.N, dtype=torch.float32, device=d["h"].device)
    dh, dW = rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], 1.0, d["adv"], lse)
    torch.cuda.synchronize()
    assert not dh.any() and not dW.any()


def test_dh_invariance_and_dw_determinism():
    fam = wl.Family(SMALL)
    base = fam.batch()
    _, _, dh, dW = run_bwd(base)
    dh = dh.cpu().numpy()
    ref = {k: dh[i] for i, k in enumerate(base.key()) if base.mask[i]}
    for w in (fam.alone(1), fam.shuffled(7), fam.padded(8)):
        _, _, dh2, _ = run_bwd(w)
        dh2 = dh2.cpu().numpy()
        for i, k in enumerate(w.key()):
            if k[0] >= 0 and w.mask[i]:
                assert np.array_equal(bits(dh2[i]), bits(ref[k])), k
    _, _, _, dW2 = run_bwd(base)
    assert np.array_equal(bits(dW.cpu().numpy()), bits(dW2.cpu().numpy()))
    # padding and inactive rows do not change dW either
    _, _, _, dW3 = run_bwd(fam.padded(9))
    assert np.array_equal(bits(dW.cpu().numpy()), bits(dW3.cpu().numpy()))


def test_autograd_matches_direct_call():
    import linear_selected_token_amd as rlk
    w = wl.make(SMALL)
    d = upload(w)
    h = d["h"].clone().requires_grad_(True)
    W = d["W"].clone().requires_grad_(True)
    lp = rlk.linear_logp(h, W, d["targets"], d["mask"], w.T)
    loss = -(d["mask"].float() * d["adv"] * lp).sum()
    loss.backward()
    _, _, dh, dW = run_bwd(w, d)
    assert torch.equal(h.grad, dh.to(torch.bfloat16))
    assert torch.equal(W.grad, dW.to(torch.bfloat16))


def _edge_vocab_rows(V, r, n_random):
    """dL/dW rows on the boundaries the backward cuts the vocabulary at: every dL/dh piece
    and chunk (multiples of 16384 and of the chunk size, two rows each side), a spread of the 256-entry
    tile boundaries, the ragged tail, plus random rows."""
    _, split = _chunking()
    piece = edge_rows(V, split, 2)
    tiles = edge_rows(V, 256, 1)[::9]
    return np.unique(np.concatenate([piece, tiles, [V - 2, V - 1], r.integers(0, V, n_random)]))


def _edge_token_rows(act, r, n_random):
    """Active tokens at the 256-token tile boundaries of the compacted order, the first and
    last active tokens, plus random ones."""
    ci = edge_rows(act.size, 256, 1)
    return np.unique(np.concatenate([act[ci], r.choice(act, n_random, replace=False)]))


def test_config5_full_size_sampled():
    flush("config 5: generating inputs")
    w = wl.make(5)
    logp_gpu, lse_gpu, dh, dW = run_bwd(w)
    h64, W64 = oracle_inputs(w)
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(5)
    flush("  config5: oracle logp and lse over all active tokens")
    ologp, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    dl = np.abs(logp_gpu.cpu().numpy()[act].astype(np.float64) - ologp[act]).max()
    ds = np.abs(lse_gpu.cpu().numpy()[act].astype(np.float64) - olse[act]).max()
    flush(f"  config5 forward over {act.size} active tokens: max|dlogp|={dl:.3e} "
          f"max|dlse|={ds:.3e}")
    assert dl <= MAX_ABS_DLOGP and ds <= MAX_ABS_DLOGP
    rows = _edge_token_rows(act, r, 24)
    odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows)
    assert_rows("config5 dh (sampled rows)",
                dh[torch.from_numpy(rows).to(dh.device)].cpu().numpy(), odh, rows)
    vr = np.unique(np.concatenate([w.targets[act[:8]], _edge_vocab_rows(w.V, r, 24)]))
    odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, w.adv, vr, lse=olse)
    assert_rows("config5 dW (sampled rows)",
                dW[torch.from_numpy(vr).to(dW.device)].cpu().numpy(), odW, vr)
    # every row of dL/dz sums to zero, so the columns of dW sum to ~0
    colsum = dW.double().sum(0).abs().max().item()
    scale = dW.double().abs().sum(0).max().item()
    flush(f"  config5 |sum_v dW_v|max={colsum:.3e} (column abs-sum {scale:.3e})")
    assert colsum <= 1e-3 * scale


def test_large_hidden_head_sampled():
    # the large-hidden head (H = 7168, V = 129280): 28 hidden tiles, W rows of 14 KiB
    w = wl.make(wl.scaled_spec(4, N=512, n_seq=2, len_lo=200, len_hi=300, prompt="floor_half",
                               seed=150, backward=True))
    _, _, dh, dW = run_bwd(w)
    h64, W64 = oracle_inputs(w)
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(151)
    rows = _edge_token_rows(act, r, 12)
    odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows)
    _, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    vr = np.unique(np.concatenate([w.targets[act[:8]], _edge_vocab_rows(w.V, r, 12)]))
    odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, w.adv, vr, lse=olse)
    flush(f"  large-hidden head N={w.N} H={w.H} V={w.V}")
    assert_rows("dh (sampled rows)", dh[torch.from_numpy(rows).to(dh.device)].cpu().numpy(),
                odh, rows)
    assert_rows("dW (sampled rows)", dW[torch.from_numpy(vr).to(dW.device)].cpu().numpy(),
                odW, vr)
