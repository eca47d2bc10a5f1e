"""The forward at the largest sizes the library accepts (needs an MI355X).

  - h of 2^31 - 1 bytes or just under (the tile loads address token rows of h with 31-bit
    offsets): the last rows of h are scored correctly;
  - N = 2^22 tokens (the compaction walks 1024 blocks of 4096);
  - V = 2^22 entries (32768 partial columns per token in the merge);
  - the logits path at its largest vocabulary, 1,024,000 entries (a row's column statistics,
    8 bytes per 128-entry column, fill 64 KB of LDS);
  - the fused forward + backward at V = 2^22 (logp and lse over all active rows, sampled
    dL/dh and dL/dW rows), and the two calls' backward on the same inputs;
  - both backward forms at N = 2^22 - 1 tokens (dozens of token blocks).
Inputs are seeded normal draws made on the device; the oracle scores sampled rows from exact
copies of them, within the 1e-3 gate."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import MAX_ABS_DLOGP, device, flush

pytestmark = pytest.mark.gpu


def _draw(shape, seed, scale=1.0):
    g = torch.Generator(device=device())
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device())
    rows = max(1, (1 << 26) // shape[1])
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        out[r0:r1] = (torch.randn((r1 - r0, shape[1]), generator=g, device=device()) *
                      scale).to(torch.bfloat16)
    return out


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(N, H, V, T, seed, rows_extra=16):
    import linear_selected_token_amd as rlk
    r = np.random.default_rng(seed)
    h = _draw((N, H), seed)
    W = _draw((V, H), seed + 1, 1.0 / np.sqrt(H))
    y = r.integers(0, V, N).astype(np.int32)
    m = np.ones(N, np.uint8)
    m[::7] = 0
    logp, lse = rlk.rlk_linear_logp_fwd(h, W, torch.from_numpy(y).to(h.device),
                                        torch.from_numpy(m).to(h.device), T)
    torch.cuda.synchronize()
    act = np.nonzero(m)[0]
    rows = np.unique(np.concatenate([act[:2], act[-3:], r.choice(act, rows_extra)]))
    W64 = _f64(W)
    h64 = _f64(h[torch.from_numpy(rows).to(h.device)])
    olp, olse = oracle.linear_logp(h64, W64, y[rows], np.ones(rows.size, np.uint8), T)
    lp = logp.cpu().numpy()
    ls = lse.cpu().numpy()
    err = float(np.abs(lp[rows] - olp).max())
    flush(f"  N={N} H={H} V={V}: max_abs_dlogp={err:.3e} over {rows.size} sampled rows "
          f"(last row {rows[-1]})")
    assert err <= MAX_ABS_DLOGP
    assert float(np.abs(ls[rows] - olse).max()) <= MAX_ABS_DLOGP
    inact = np.nonzero(m == 0)[0]
    assert not lp[inact].any() and not ls[inact].any()


def test_hidden_states_at_the_byte_limit():
    H = 4096
    N = ((1 << 31) - 1) // (2 * H)   # 262143 rows: 2^31 - 8192 bytes
    _run(N, H, 1000, 0.9, 41)


def test_most_tokens():
    _run(1 << 22, 64, 1000, 1.0, 42)


def test_largest_vocabulary():
    _run(300, 64, 1 << 22, 1.0, 43, rows_extra=6)


def test_backward_largest_vocabulary():
    # the fused forward + backward at V = 2^22: 8 MiB of codes per token (256-token blocks, a
    # 2.2 GB workspace), dL/dh tiles whose K is a whole half of the vocabulary (2^21 entries,
    # 32768 K stages, W offsets past 2^31 bytes), 16384 vocabulary tiles of dL/dW
    import linear_selected_token_amd as rlk
    from gpu_util import assert_rows
    N, H, V, T = 64, 256, 1 << 22, 1.0
    r = np.random.default_rng(45)
    h = _draw((N, H), 45)
    W = _draw((V, H), 46, 1.0 / np.sqrt(H))
    y = r.integers(0, V, N).astype(np.int32)
    m = np.ones(N, np.uint8)
    m[::5] = 0
    adv = r.normal(0, 1, N).astype(np.float32)
    dev = h.device
    logp, lse, dh, dW = rlk.rlk_linear_logp_fwd_bwd(h, W, torch.from_numpy(y).to(dev),
                                                    torch.from_numpy(m).to(dev), T,
                                                    torch.from_numpy(adv).to(dev))
    torch.cuda.synchronize()
    act = np.nonzero(m)[0]
    h64, W64 = _f64(h), _f64(W)
    olp, olse = oracle.linear_logp(h64, W64, y, m, T)
    err = float(np.abs(logp.cpu().numpy()[act] - olp[act]).max())
    flush(f"  fused N={N} H={H} V={V}: max_abs_dlogp={err:.3e} over all {act.size} active rows")
    assert err <= MAX_ABS_DLOGP
    assert float(np.abs(lse.cpu().numpy()[act] - olse[act]).max()) <= MAX_ABS_DLOGP
    rows = np.unique(np.concatenate([act[:2], act[-2:], r.choice(act, 4)]))
    odh = oracle.grad_h_rows(h64, W64, y, m, T, adv, rows)
    assert_rows("fused dh (sampled rows)", dh[torch.from_numpy(rows).to(dev)].cpu().numpy(),
                odh, rows)
    half = 1 << 21
    vr = np.unique(np.concatenate([y[act[:4]], [0, 1, half - 1, half, V - 2, V - 1],
                                   r.integers(0, V, 10)]))
    odW = oracle.grad_W_rows(h64, W64, y, m, T, adv, vr, lse=olse)
    assert_rows("fused dW (sampled rows)", dW[torch.from_numpy(vr).to(dev)].cpu().numpy(), odW,
                vr)
    # the two calls on the same inputs: 128 vocabulary chunks of 32768 entries
    yt, mt, at = (torch.from_numpy(x).to(dev) for x in (y, m, adv))
    _, lse2 = rlk.rlk_linear_logp_fwd(h, W, yt, mt, T)
    dh2, dW2 = rlk.rlk_linear_logp_bwd(h, W, yt, mt, T, at, lse2)
    torch.cuda.synchronize()
    assert_rows("two calls dh (sampled rows)",
                dh2[torch.from_numpy(rows).to(dev)].cpu().numpy(), odh, rows)
    assert_rows("two calls dW (sampled rows)",
                dW2[torch.from_numpy(vr).to(dev)].cpu().numpy(), odW, vr)


def test_backward_most_tokens():
    # both backward forms at N = 2^22 - 1 tokens (h just under 2^31 bytes at H = 256), in
    # dozens of token blocks each
    import linear_selected_token_amd as rlk
    from gpu_util import assert_rows
    N, H, V, T = (1 << 22) - 1, 256, 1000, 1.1
    r = np.random.default_rng(47)
    h = _draw((N, H), 47)
    W = _draw((V, H), 48, 1.0 / np.sqrt(H))
    y = r.integers(0, V, N).astype(np.int32)
    m = np.ones(N, np.uint8)
    m[::7] = 0
    adv = r.normal(0, 1, N).astype(np.float32)
    dev = h.device
    yt, mt, at = (torch.from_numpy(x).to(dev) for x in (y, m, adv))
    logp, lse, dh, dW = rlk.rlk_linear_logp_fwd_bwd(h, W, yt, mt, T, at)
    _, lse2 = rlk.rlk_linear_logp_fwd(h, W, yt, mt, T)
    dh2, dW2 = rlk.rlk_linear_logp_bwd(h, W, yt, mt, T, at, lse2)
    torch.cuda.synchronize()
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    act = np.nonzero(m)[0]
    rows = np.unique(np.concatenate([act[:2], act[-3:], r.choice(act, 12),
                                     act[65536 * np.arange(1, 4) - 1], act[65536 * np.arange(1, 4)]]))
    h64, W64 = _f64(h), _f64(W)
    olp, olse = oracle.linear_logp(h64, W64, y, m, T)
    err = float(np.abs(logp.cpu().numpy()[act] - olp[act]).max())
    flush(f"  N={N} H={H} V={V}: max_abs_dlogp={err:.3e} over all {act.size} active rows")
    assert err <= MAX_ABS_DLOGP
    odh = oracle.grad_h_rows(h64, W64, y, m, T, adv, rows)
    vr = np.unique(np.concatenate([[0, 255, 256, V - 1], r.integers(0, V, 12)]))
    odW = oracle.grad_W_rows(h64, W64, y, m, T, adv, vr, lse=olse)
    for name, gh, gw in (("fused", dh, dW), ("two calls", dh2, dW2)):
        assert_rows(f"{name} dh (sampled rows)",
                    gh[torch.from_numpy(rows).to(dev)].cpu().numpy(), odh, rows)
        assert_rows(f"{name} dW (sampled rows)",
                    gw[torch.from_numpy(vr).to(dev)].cpu().numpy(), odW, vr)


def test_logits_path_largest_vocabulary():
    import linear_selected_token_amd as rlk
    N, V, T = 40, 1024000, 0.8
    z = _draw((N, V), 44, 3.0)
    r = np.random.default_rng(44)
    y = r.integers(0, V, N).astype(np.int32)
    m = np.ones(N, np.uint8)
    logp, lse = rlk.rlk_logp_from_logits(z, torch.from_numpy(y).to(z.device),
                                         torch.from_numpy(m).to(z.device), T)
    torch.cuda.synchronize()
    rows = np.array([0, 17, N - 1])
    olp, olse = oracle.logp_from_logits(_f64(z[torch.from_numpy(rows).to(z.device)]), y[rows],
                                        np.ones(rows.size, np.uint8), T)
    err = float(np.abs(logp.cpu().numpy()[rows] - olp).max())
    flush(f"  logits path V={V}: max_abs_dlogp={err:.3e}")
    assert err <= MAX_ABS_DLOGP
    assert float(np.abs(lse.cpu().numpy()[rows] - olse).max()) <= MAX_ABS_DLOGP
