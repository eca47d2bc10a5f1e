"""Parity of the fused forward + backward (rlk_linear_logp_fwd_bwd) against the float64 oracle
(needs an MI355X).

logp and lse are the forward's own bits; dL/dh and dL/dW of L = -sum_t mask_t adv_t logp_t are
gated per row at rel-L2 <= 1e-2 like the two-call backward.  The fused call forms dL/dz from the
forward's d = x - (column max), kept as a 16-bit code in steps of 2^-9, instead of recomputing
the logits, so its gradients differ from the two-call backward's by that rounding only; a
token's dL/dh row is still bit-identical across batch layouts and token blocks."""
import re

import numpy as np
import pytest
import torch

import oracle
import oracle.rl_loss as orl
import workloads as wl
from gpu_util import (MAX_ABS_DLOGP, assert_rows, assert_tiles, bits, device, edge_rows, flush,
                      oracle_inputs, rel_l2, run_fwd, upload)

pytestmark = pytest.mark.gpu


def run_fused(w, d=None):
    import linear_selected_token_amd as rlk
    d = d or upload(w)
    logp, lse, dh, dW = rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                                    d["adv"])
    torch.cuda.synchronize()
    return logp, lse, dh, dW


def _chunking():
    import linear_selected_token_amd as rlk
    m = re.search(r"bwd chunk (\d+), dh split at (\d+)", rlk.build_info())
    assert m, rlk.build_info()
    return int(m.group(1)), int(m.group(2))


def _fused_cap(H, V):
    """Token capacity of the fused call's block buffers, by the rule include/rlk.h states: the
    largest multiple of 256 tokens whose buffers (a row of roundup(V, 256) + 64 two-byte
    entries, 8 bytes per 128-entry column, 6 H + 12 bytes) fit 1e9 bytes."""
    pitch = (V + 255) // 256 * 256 + 64
    per = 2 * pitch + 8 * ((V + 127) // 128) + 6 * H + 12
    return max(256, 10**9 // per // 256 * 256)


def _same_forward(w, d, logp, lse):
    """logp and lse of the fused call carry the forward's bits at every token."""
    flogp, flse = run_fwd(w, d)
    assert np.array_equal(bits(logp.cpu().numpy()), bits(flogp))
    assert np.array_equal(bits(lse.cpu().numpy()), bits(flse))


def _full_compare(w):
    d = upload(w)
    logp, lse, dh, dW = run_fused(w, d)
    _same_forward(w, d, logp, lse)
    dh = dh.cpu().numpy()
    dW = dW.cpu().numpy()
    h64, W64 = oracle_inputs(w)
    odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, w.adv)
    act = np.nonzero(w.mask)[0]
    flush(f"  {w.spec.name} N={w.N} H={w.H} V={w.V} active={act.size}")
    assert_rows("fused dh (every active row)", dh[act], odh[act], act)
    assert_rows("fused dW (every vocabulary row)", dW, odW)
    assert_tiles("fused dW", dW, odW)
    assert not dh[w.mask == 0].any()
    return dh, dW


def _sweep_specs(n, seed):
    """Seeded shapes across tile, column, piece and chunk edges: N in [1, 900], H in {256, 512,
    768}, V in [1, 40000] (log-uniform), T in [0.5, 1.5]; one to three packed sequences."""
    r = np.random.default_rng(seed)
    out = []
    for k in range(n):
        N = int(r.integers(1, 901))
        n_seq = int(min(N, r.integers(1, 4)))
        V = int(np.exp(r.uniform(0.0, np.log(40000.0)))) + 1
        out.append(wl.scaled_spec(5, N=N, H=int(r.choice([256, 512, 768])), V=V, n_seq=n_seq,
                                  len_lo=1, len_hi=N, seed=700 + k, T=float(r.uniform(0.5, 1.5))))
    return out


@pytest.mark.parametrize("spec", _sweep_specs(16, 211), ids=lambda s: f"N{s.N}-H{s.H}-V{s.V}")
def test_random_shapes_sweep(spec):
    # the fused call in full against the oracle (every active dh row, every dW row and tile),
    # and the two calls' gradients beside it
    from gpu_util import run_bwd
    w = wl.make(spec)
    dh, dW = _full_compare(w)
    _, _, dh2, dW2 = run_bwd(w)
    act = np.nonzero(w.mask)[0]
    h64, W64 = oracle_inputs(w)
    odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, w.adv)
    assert_rows("two calls dh (every active row)", dh2.cpu().numpy()[act], odh[act], act)
    assert_rows("two calls dW (every vocabulary row)", dW2.cpu().numpy(), odW)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_small_full(T):
    _full_compare(wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64,
                                         len_hi=300, seed=95, T=T)))


def test_two_chunks_ragged():
    # a vocabulary of two backward chunks of the two-call path plus a ragged tail; the fused
    # call's dL/dh splits it into its two halves (the split at 24768 of 49472 columns, inside a
    # 256-entry vocabulary tile) and its dL/dW tiles end in the ragged last tile
    chunk, split = _chunking()
    _full_compare(wl.make(wl.scaled_spec(5, N=300, H=256, V=chunk + split + 300, n_seq=2,
                                         len_lo=100, len_hi=200, seed=96)))


@pytest.mark.parametrize("V", [1, 129, 255, 257])
def test_tiny_vocabularies(V):
    # one tile or a few entries past one: the stored rows end inside the first vocabulary tile
    _full_compare(wl.make(wl.scaled_spec(5, N=300, H=256, V=V, n_seq=2, len_lo=100,
                                         len_hi=200, seed=98)))


@pytest.mark.parametrize("scale", [4.0, 24.0])
def test_peaked_softmax(scale):
    # h scaled up: most of each token's probability sits on a few entries, where the stored d
    # (distance to the column maximum) is small; the rest of the row spans tens of log2 units
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=100, T=0.7))
    w.h = wl.bf16_bits(wl.bf16_to_f32(w.h) * np.float32(scale))
    _full_compare(w)


def test_agrees_with_two_call_backward():
    # the same gradients as rlk_linear_logp_fwd + rlk_linear_logp_bwd up to the rounding of d
    from gpu_util import run_bwd
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=99, T=0.7))
    d = upload(w)
    _, _, dh1, dW1 = run_bwd(w, d)
    _, _, dh2, dW2 = run_fused(w, d)
    eh = rel_l2(dh2.cpu().numpy(), dh1.cpu().numpy())
    ew = rel_l2(dW2.cpu().numpy(), dW1.cpu().numpy())
    flush(f"  fused vs two-call: dh relL2 {eh:.3e}, dW relL2 {ew:.3e}")
    assert eh <= 5e-3 and ew <= 5e-3


def test_out_of_range_targets_both_forms():
    # an active token whose target is outside [0, V): logp NaN, lse unchanged, and dL/dz without
    # the target term (-g_t p[t, v]) in the fused call and in the two calls alike.  Expected
    # values: the oracle's gradients with those tokens' targets set to 0, minus the target
    # term it then adds, g_t e_0, carried through dh_t = G_t W / T and dW_0 += G[t, 0] h_t / T.
    from gpu_util import run_bwd
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=191, T=0.7))
    act = np.nonzero(w.mask)[0]
    bad = np.array([int(act[3]), int(act[40])])
    _, lse_ok, _, _ = run_fused(w)
    w.targets[bad[0]] = w.V
    w.targets[bad[1]] = -5
    d = upload(w)
    lp, lse, dh, dW = run_fused(w, d)
    lp2, lse2, dh2, dW2 = run_bwd(w, d)
    lp, lse, lp2 = lp.cpu().numpy(), lse.cpu().numpy(), lp2.cpu().numpy()
    assert np.all(np.isnan(lp[bad])) and np.all(np.isnan(lp2[bad]))
    assert np.array_equal(bits(lse), bits(lse_ok.cpu().numpy()))
    keep = np.setdiff1d(act, bad)
    assert not np.isnan(lp[keep]).any()
    h64, W64 = oracle_inputs(w)
    y0 = w.targets.copy()
    y0[bad] = 0
    odh, odW = oracle.linear_logp_grads(h64, W64, y0, w.mask, w.T, w.adv)
    g = -w.adv[bad].astype(np.float64)
    odh[bad] -= g[:, None] * W64[0][None, :] / w.T
    odW[0] -= (g[:, None] * h64[bad]).sum(0) / w.T
    for name, gh, gw in (("fused", dh, dW), ("two calls", dh2, dW2)):
        gh = gh.cpu().numpy()
        assert_rows(f"{name} dh (active rows, two without a target)", gh[act], odh[act], act)
        assert_rows(f"{name} dW (every vocabulary row)", gw.cpu().numpy(), odW)


def test_inactive_rows_may_hold_anything():
    # inactive tokens are never read into the products: NaN and infinite h rows and
    # out-of-range targets there change no bit of logp, lse, dh or dW (forward, two calls and
    # the fused call)
    from gpu_util import run_bwd
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=192, T=0.9))
    ref = [t.cpu() for t in run_bwd(w) + run_fused(w)]
    off = np.nonzero(w.mask == 0)[0]
    assert off.size > 0
    r = np.random.default_rng(193)
    poison = np.array([0x7FC0, 0x7F80, 0xFF80, 0x7F7F], dtype=np.uint16)  # NaN, +inf, -inf, max
    w.h[off] = poison[r.integers(0, poison.size, (off.size, w.H))]
    w.targets[off] = r.choice([-7, w.V, w.V + 1000], off.size)
    got = [t.cpu() for t in run_bwd(w) + run_fused(w)]
    names = ("logp", "lse", "dh", "dW", "fused logp", "fused lse", "fused dh", "fused dW")
    for name, a, b in zip(names, got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    flush(f"  {off.size} inactive rows poisoned: every output keeps its bits")


def test_all_masked():
    import linear_selected_token_amd as rlk
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=95))
    d = upload(w)
    d["mask"].zero_()
    logp, lse, dh, dW = rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], 1.0,
                                                    d["adv"])
    torch.cuda.synchronize()
    assert not logp.any() and not lse.any() and not dh.any() and not dW.any()


def test_invariance_and_determinism():
    fam = wl.Family(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                                   seed=95))
    base = fam.batch()
    logp, lse, dh, dW = run_fused(base)
    dh = dh.cpu().numpy()
    logp = logp.cpu().numpy()
    ref = {k: (dh[i], logp[i]) for i, k in enumerate(base.key()) if base.mask[i]}
    for w in (fam.alone(1), fam.shuffled(7), fam.padded(8)):
        lp2, _, dh2, _ = run_fused(w)
        dh2 = dh2.cpu().numpy()
        lp2 = lp2.cpu().numpy()
        for i, k in enumerate(w.key()):
            if k[0] >= 0 and w.mask[i]:
                assert np.array_equal(bits(dh2[i]), bits(ref[k][0])), k
                assert np.array_equal(bits(lp2[i]), bits(ref[k][1])), k
    _, _, _, dW2 = run_fused(base)
    assert np.array_equal(bits(dW.cpu().numpy()), bits(dW2.cpu().numpy()))
    _, _, _, dW3 = run_fused(fam.padded(9))
    assert np.array_equal(bits(dW.cpu().numpy()), bits(dW3.cpu().numpy()))


# The full Qwen3-8B vocabulary at H = 256: blocks of at most 3072 tokens, so ~60% active of
# 8000 tokens take two blocks; sampled rows against the oracle
BLOCKS = wl.scaled_spec(3, N=8000, H=256, n_seq=24, len_lo=128, len_hi=512, seed=161,
                        targets="uniform", backward=True)


def _sampled_compare(w, logp, lse, dh, dW, seed, n_tok=24, n_voc=24):
    h64, W64 = oracle_inputs(w)
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(seed)
    flush(f"  oracle logp and lse over all {act.size} active tokens")
    ologp, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    dl = np.abs(logp.cpu().numpy()[act].astype(np.float64) - ologp[act]).max()
    ds = np.abs(lse.cpu().numpy()[act].astype(np.float64) - olse[act]).max()
    flush(f"  max|dlogp|={dl:.3e} max|dlse|={ds:.3e}")
    assert dl <= MAX_ABS_DLOGP and ds <= MAX_ABS_DLOGP
    ci = edge_rows(act.size, 256, 1)
    rows = np.unique(np.concatenate([act[ci], r.choice(act, n_tok, replace=False)]))
    odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows)
    assert_rows("fused dh (sampled rows)",
                dh[torch.from_numpy(rows).to(dh.device)].cpu().numpy(), odh, rows)
    _, split = _chunking()
    vr = np.unique(np.concatenate([w.targets[act[:8]], edge_rows(w.V, split, 2),
                                   [w.V - 2, w.V - 1], r.integers(0, w.V, n_voc)]))
    odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, w.adv, vr, lse=olse)
    assert_rows("fused dW (sampled rows)",
                dW[torch.from_numpy(vr).to(dW.device)].cpu().numpy(), odW, vr)


def test_token_blocks_sampled():
    w = wl.make(BLOCKS)
    cap = _fused_cap(w.H, w.V)
    flush(f"  {w.n_active} active of {w.N}: fused blocks of at most {cap}")
    assert cap < w.n_active < 2 * cap
    d = upload(w)
    logp, lse, dh, dW = run_fused(w, d)
    _same_forward(w, d, logp, lse)
    assert not dh[torch.from_numpy(w.mask == 0).to(dh.device)].any()
    _sampled_compare(w, logp, lse, dh, dW, 162)


def test_token_blocks_dh_invariance():
    # a token's logp and dL/dh row keep their bits whichever block it falls in
    fam = wl.Family(BLOCKS)
    base = fam.batch()
    logp, _, dh, _ = run_fused(base)
    dh = dh.cpu().numpy()
    logp = logp.cpu().numpy()
    ref = {k: (dh[i], logp[i]) for i, k in enumerate(base.key()) if base.mask[i]}
    for w in (fam.alone(5), fam.shuffled(3), fam.all_active()):
        lp2, _, dh2, _ = run_fused(w)
        dh2 = dh2.cpu().numpy()
        lp2 = lp2.cpu().numpy()
        n = 0
        for i, k in enumerate(w.key()):
            if k[0] >= 0 and w.mask[i] and k in ref:
                assert np.array_equal(bits(dh2[i]), bits(ref[k][0])), k
                assert np.array_equal(bits(lp2[i]), bits(ref[k][1])), k
                n += 1
        flush(f"  {w.N} tokens, {w.n_active} active: {n} rows bit-identical")


def test_larger_workspace_one_block():
    # a workspace sized for one block of every active token: logp, lse and each dL/dh row keep
    # their bits; dL/dW (one block's sum instead of two) agrees with the oracle and, to rounding,
    # with the two-block result
    import linear_selected_token_amd as rlk
    w = wl.make(BLOCKS)
    d = upload(w)
    lp1, ls1, dh1, dW1 = run_fused(w, d)
    nb = rlk.fwd_bwd_workspace_bytes_for_block(w.N, w.H, w.V, 0, w.n_active)
    assert nb > rlk.fwd_bwd_workspace_bytes(w.N, w.H, w.V, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=d["h"].device)
    lp2, ls2, dh2, dW2 = rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                                     d["adv"], workspace=ws)
    torch.cuda.synchronize()
    flush(f"  {w.n_active} active: one block with {nb / 1e9:.2f} GB against two")
    assert torch.equal(lp1.view(torch.int32), lp2.view(torch.int32))
    assert torch.equal(ls1.view(torch.int32), ls2.view(torch.int32))
    assert torch.equal(dh1.view(torch.int32), dh2.view(torch.int32))
    e = rel_l2(dW2.cpu().numpy(), dW1.cpu().numpy())
    flush(f"  dW one block vs two: relL2 {e:.3e}")
    assert e <= 1e-5
    _sampled_compare(w, lp2, ls2, dh2, dW2, 164, n_tok=8)


MANY = wl.scaled_spec(5, N=3200, H=256, V=1000, n_seq=8, len_lo=200, len_hi=600, seed=175, T=0.8)


def test_many_small_blocks():
    # a workspace for 256-token blocks (seven blocks here, against one by default): logp, lse and
    # every dL/dh row keep their bits, dL/dW (a sum over the blocks) agrees with the one-block
    # result to rounding and with the oracle row by row
    import linear_selected_token_amd as rlk
    w = wl.make(MANY)
    d = upload(w)
    lp1, ls1, dh1, dW1 = run_fused(w, d)
    nb = rlk.fwd_bwd_workspace_bytes_for_block(w.N, w.H, w.V, 0, 256)
    assert nb < rlk.fwd_bwd_workspace_bytes(w.N, w.H, w.V, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=d["h"].device)
    lp2, ls2, dh2, dW2 = rlk.rlk_linear_logp_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                                     d["adv"], workspace=ws)
    torch.cuda.synchronize()
    nblk = -(-w.n_active // 256)
    flush(f"  {w.n_active} active: {nblk} blocks of 256 tokens in {nb / 1e6:.1f} MB against one")
    assert nblk >= 7
    assert torch.equal(lp1.view(torch.int32), lp2.view(torch.int32))
    assert torch.equal(ls1.view(torch.int32), ls2.view(torch.int32))
    assert torch.equal(dh1.view(torch.int32), dh2.view(torch.int32))
    e = rel_l2(dW2.cpu().numpy(), dW1.cpu().numpy())
    flush(f"  dW {nblk} blocks vs one: relL2 {e:.3e}")
    assert e <= 1e-5
    h64, W64 = oracle_inputs(w)
    odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, w.adv)
    assert_rows("fused dW over many blocks (every vocabulary row)", dW2.cpu().numpy(), odW)
    assert_tiles("fused dW over many blocks", dW2.cpu().numpy(), odW)


def test_config5_full_size_sampled():
    flush("config 5 fused: generating inputs")
    w = wl.make(5)
    d = upload(w)
    logp, lse, dh, dW = run_fused(w, d)
    _same_forward(w, d, logp, lse)
    _sampled_compare(w, logp, lse, dh, dW, 163)
    colsum = dW.double().sum(0).abs().max().item()
    scale = dW.double().abs().sum(0).max().item()
    flush(f"  config5 fused |sum_v dW_v|max={colsum:.3e} (column abs-sum {scale:.3e})")
    assert colsum <= 1e-3 * scale


def test_large_hidden_head_fused_sampled():
    # the large-hidden head (H = 7168, V = 129280) through the fused call: 28 hidden tiles per
    # dL/dh row block, dL/dW tiles of every vocabulary row in the one whole-vocabulary launch
    w = wl.make(wl.scaled_spec(4, N=512, n_seq=2, len_lo=200, len_hi=300, prompt="floor_half",
                               seed=152, backward=True))
    flush(f"  large-hidden head N={w.N} H={w.H} V={w.V}, {w.n_active} active")
    d = upload(w)
    logp, lse, dh, dW = run_fused(w, d)
    _same_forward(w, d, logp, lse)
    _sampled_compare(w, logp, lse, dh, dW, 153, n_tok=12, n_voc=16)


def test_autograd_loss():
    import linear_selected_token_amd as rlk
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=95))
    d = upload(w)
    h = d["h"].clone().requires_grad_(True)
    W = d["W"].clone().requires_grad_(True)
    loss, lp = rlk.linear_logp_pg_loss(h, W, d["targets"], d["mask"], w.T, d["adv"])
    (2.0 * loss).backward()
    logp, _, dh, dW = run_fused(w, d)
    assert torch.equal(lp, logp)
    assert torch.equal(h.grad, (2.0 * dh).to(torch.bfloat16))
    assert torch.equal(W.grad, (2.0 * dW).to(torch.bfloat16))
    ref = -(d["mask"].float() * d["adv"] * logp).sum()
    assert torch.equal(loss.detach(), ref)


# ------------------------------------------------------------------ the fused PPO step

def _ppo_inputs(w, d, seed):
    """old and reference log-probs: the forward's logp plus seeded noise (tokens whose ratio
    would sit within 1e-4 of a clip edge keep old = logp, so no decision is a rounding tie)."""
    logp, _ = run_fwd(w, d)
    r = np.random.default_rng(seed)
    old = (logp + r.normal(0, 0.2, w.N)).astype(np.float32)
    ref = (logp + r.normal(0, 0.2, w.N)).astype(np.float32)
    ratio = np.exp(logp.astype(np.float64) - old)
    near = (np.abs(ratio - 0.8) < 1e-4) | (np.abs(ratio - 1.2) < 1e-4)
    old[near] = logp[near]
    return old, ref


def _ppo_chain(w, d, old_t, ref_t, scale):
    """The same step through the separate calls: forward, loss fragment, backward."""
    import linear_selected_token_amd as rlk
    logp, lse = rlk.rlk_linear_logp_fwd(d["h"], d["W"], d["targets"], d["mask"], w.T)
    loss, badv, ratio, sums = rlk.rlk_ratio_kl_loss(logp, old_t, ref_t, d["adv"], d["mask"], 0.2,
                                                    0.2, 0.05, scale, want_ratio=True)
    dh, dW = rlk.rlk_linear_logp_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, badv, lse)
    torch.cuda.synchronize()
    return logp, lse, loss, badv, ratio, sums, dh, dW


def _check_ppo(w, seed, oracle_rows=None):
    import linear_selected_token_amd as rlk
    d = upload(w)
    dev = d["h"].device
    old, ref = _ppo_inputs(w, d, seed)
    old_t, ref_t = torch.from_numpy(old).to(dev), torch.from_numpy(ref).to(dev)
    scale = 1.0 / int(w.mask.sum())
    chain = _ppo_chain(w, d, old_t, ref_t, scale)
    fused = rlk.rlk_linear_ppo_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], w.T, old_t, ref_t,
                                       d["adv"], 0.2, 0.2, 0.05, scale)
    torch.cuda.synchronize()
    # logp, lse, loss, -dloss/dlogp, ratio and the fixed-order sums: the chain's bits
    for name, a, b in zip(("logp", "lse", "loss", "bwd_adv", "ratio", "sums"), fused[:6], chain[:6]):
        ai = a.view(torch.int64) if a.dtype == torch.float64 else a.view(torch.int32)
        bi = b.view(torch.int64) if b.dtype == torch.float64 else b.view(torch.int32)
        assert torch.equal(ai, bi), name
    act = np.nonzero(w.mask)[0]
    eh = rel_l2(fused[6].cpu().numpy()[act], chain[6].cpu().numpy()[act])
    ew = rel_l2(fused[7].cpu().numpy(), chain[7].cpu().numpy())
    flush(f"  fused PPO vs the chain of calls: dh relL2 {eh:.3e}, dW relL2 {ew:.3e}")
    assert eh <= 5e-3 and ew <= 5e-3
    assert not fused[6][torch.from_numpy(w.mask == 0).to(dev)].any()
    # against the oracle's chain rule on the oracle's own logp
    h64, W64 = oracle_inputs(w)
    olp, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
    _, og, _, _, _ = orl.ratio_kl_loss(olp, old, ref, w.adv, w.mask, 0.2, 0.2, 0.05, scale)
    dh, dW = fused[6].cpu().numpy(), fused[7].cpu().numpy()
    if oracle_rows is None:
        odh, odW = oracle.linear_logp_grads(h64, W64, w.targets, w.mask, w.T, -og)
        assert_rows("fused PPO dh (every active row)", dh[act], odh[act], act)
        assert_rows("fused PPO dW (every vocabulary row)", dW, odW)
    else:
        rows, vr = oracle_rows
        odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, -og, rows)
        assert_rows("fused PPO dh (sampled rows)", dh[rows], odh, rows)
        odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, -og, vr, lse=olse)
        assert_rows("fused PPO dW (sampled rows)", dW[vr], odW, vr)


def test_ppo_fused_matches_chain_and_oracle():
    _check_ppo(wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                                      seed=101, T=0.9)), 102)


@pytest.mark.parametrize("spec", _sweep_specs(6, 213), ids=lambda s: f"N{s.N}-H{s.H}-V{s.V}")
def test_ppo_fused_sweep(spec):
    # the fused PPO step over seeded random shapes: per-token outputs bitwise the chain of
    # calls, gradients against the oracle's chain rule in full
    _check_ppo(wl.make(spec), spec.seed + 1)


def test_ppo_fused_token_blocks():
    # two token blocks over the Qwen3-8B vocabulary: each block's loss fragment sees its own
    # tokens' final logp
    w = wl.make(BLOCKS)
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(171)
    rows = np.unique(np.concatenate([act[edge_rows(act.size, 256, 1)], r.choice(act, 8, False)]))
    vr = np.unique(np.concatenate([w.targets[act[:4]], r.integers(0, w.V, 12)]))
    _check_ppo(w, 172, oracle_rows=(rows, vr))


def test_ppo_fused_many_small_blocks():
    # 256-token blocks: each block's loss fragment runs on its own tokens, so every per-token
    # output and dL/dh row keeps the one-block call's bits; dL/dW agrees to rounding
    import linear_selected_token_amd as rlk
    w = wl.make(MANY)
    d = upload(w)
    dev = d["h"].device
    old, ref = _ppo_inputs(w, d, 176)
    old_t, ref_t = torch.from_numpy(old).to(dev), torch.from_numpy(ref).to(dev)
    scale = 1.0 / int(w.mask.sum())
    args = (d["h"], d["W"], d["targets"], d["mask"], w.T, old_t, ref_t, d["adv"], 0.2, 0.2, 0.05,
            scale)
    one = rlk.rlk_linear_ppo_fwd_bwd(*args)
    loss_bytes = (rlk.ppo_fwd_bwd_workspace_bytes(w.N, w.H, w.V, 0) -
                  rlk.fwd_bwd_workspace_bytes(w.N, w.H, w.V, 0))
    nb = loss_bytes + rlk.fwd_bwd_workspace_bytes_for_block(w.N, w.H, w.V, 0, 256)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    many = rlk.rlk_linear_ppo_fwd_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("logp", "lse", "loss", "bwd_adv", "ratio", "sums", "dh"), many[:7],
                          one[:7]):
        ai = a.view(torch.int64) if a.dtype == torch.float64 else a.view(torch.int32)
        bi = b.view(torch.int64) if b.dtype == torch.float64 else b.view(torch.int32)
        assert torch.equal(ai, bi), name
    e = rel_l2(many[7].cpu().numpy(), one[7].cpu().numpy())
    flush(f"  fused PPO, 256-token blocks vs one block: dW relL2 {e:.3e}")
    assert e <= 1e-5


def test_ppo_fused_all_masked():
    import linear_selected_token_amd as rlk
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=95))
    d = upload(w)
    d["mask"].zero_()
    z = torch.zeros(w.N, dtype=torch.float32, device=d["h"].device)
    out = rlk.rlk_linear_ppo_fwd_bwd(d["h"], d["W"], d["targets"], d["mask"], 1.0, z, z, d["adv"],
                                     0.2, 0.2, 0.05, 1.0)
    torch.cuda.synchronize()
    assert all(not t.any() for t in out)


# ------------------------------------------------------------------ the fused entropy bonus

def _check_entropy(w, seed, oracle_rows=None):
    import linear_selected_token_amd as rlk
    d = upload(w)
    dev = d["h"].device
    c = np.random.default_rng(seed).uniform(0.0, 0.5, w.N).astype(np.float32)
    ct = torch.from_numpy(c).to(dev)
    lp1, ls1, en1 = rlk.rlk_linear_logp_fwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T)
    dh1, dW1 = rlk.rlk_linear_logp_bwd_entropy(d["h"], d["W"], d["targets"], d["mask"], w.T,
                                               d["adv"], ct, ls1, en1)
    lp2, ls2, en2, dh2, dW2 = rlk.rlk_linear_logp_fwd_bwd_entropy(d["h"], d["W"], d["targets"],
                                                                  d["mask"], w.T, d["adv"], ct)
    torch.cuda.synchronize()
    for name, a, b in (("logp", lp2, lp1), ("lse", ls2, ls1), ("entropy", en2, en1)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    act = np.nonzero(w.mask)[0]
    eh = rel_l2(dh2.cpu().numpy()[act], dh1.cpu().numpy()[act])
    ew = rel_l2(dW2.cpu().numpy(), dW1.cpu().numpy())
    flush(f"  fused entropy bonus vs the two calls: dh relL2 {eh:.3e}, dW relL2 {ew:.3e}")
    assert eh <= 5e-3 and ew <= 5e-3
    h64, W64 = oracle_inputs(w)
    dh, dW = dh2.cpu().numpy(), dW2.cpu().numpy()
    if oracle_rows is None:
        odh, odW = oracle.linear_logp_entropy_grads(h64, W64, w.targets, w.mask, w.T, w.adv, c)
        assert_rows("fused entropy dh (every active row)", dh[act], odh[act], act)
        assert_rows("fused entropy dW (every vocabulary row)", dW, odW)
    else:
        rows, vr = oracle_rows
        odh = oracle.grad_h_rows(h64, W64, w.targets, w.mask, w.T, w.adv, rows, ent_coef=c)
        assert_rows("fused entropy dh (sampled rows)", dh[rows], odh, rows)
        _, olse = oracle.linear_logp(h64, W64, w.targets, w.mask, w.T)
        odW = oracle.grad_W_rows(h64, W64, w.targets, w.mask, w.T, w.adv, vr, lse=olse,
                                 ent_coef=c)
        assert_rows("fused entropy dW (sampled rows)", dW[vr], odW, vr)


def test_entropy_bonus_fused():
    _check_entropy(wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64,
                                          len_hi=300, seed=103, T=0.8)), 104)


@pytest.mark.parametrize("spec", _sweep_specs(8, 212), ids=lambda s: f"N{s.N}-H{s.H}-V{s.V}")
def test_entropy_bonus_fused_sweep(spec):
    # the fused call with an entropy bonus over seeded random shapes: logp, lse and entropy
    # bitwise the entropy forward's, gradients against the oracle in full
    _check_entropy(wl.make(spec), spec.seed + 1)


def test_entropy_bonus_fused_peaked():
    # h x 8: peaked softmaxes, where p ln p of the tail entries is tiny but their codes are far
    # from 0
    w = wl.make(wl.scaled_spec(5, N=600, H=512, V=3000, n_seq=4, len_lo=64, len_hi=300,
                               seed=105, T=0.8))
    w.h = wl.bf16_bits(wl.bf16_to_f32(w.h) * np.float32(8.0))
    _check_entropy(w, 106)


def test_entropy_bonus_fused_token_blocks():
    w = wl.make(BLOCKS)
    act = np.nonzero(w.mask)[0]
    r = np.random.default_rng(173)
    rows = np.unique(np.concatenate([act[edge_rows(act.size, 256, 1)], r.choice(act, 6, False)]))
    vr = np.unique(np.concatenate([w.targets[act[:4]], r.integers(0, w.V, 10)]))
    _check_entropy(w, 174, oracle_rows=(rows, vr))
