"""The seeded input generator: reproducibility, layout recipe, bf16 rounding (no GPU)."""
import hashlib

import numpy as np
import torch

import workloads as wl


def _digest(w):
    m = hashlib.sha256()
    for a in (w.h, w.W, w.targets, w.mask, w.adv, w.u):
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()


SMALL = wl.scaled_spec(2, N=700, H=128, V=900, n_seq=5, len_lo=64, len_hi=300)


def test_same_seed_same_bytes():
    assert _digest(wl.make(SMALL)) == _digest(wl.make(SMALL))
    other = wl.scaled_spec(2, N=700, H=128, V=900, n_seq=5, len_lo=64, len_hi=300, seed=7)
    assert _digest(wl.make(other)) != _digest(wl.make(SMALL))


def test_weight_blocks_independent_of_threads(monkeypatch):
    a = wl.weight_matrix(5, 9000, 64, "bf16")
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.weight_matrix(5, 9000, 64, "bf16")
    np.testing.assert_array_equal(a, b)


def test_lengths_and_prompts():
    for cfg in (2, 3, 5):
        s = wl.CONFIGS[cfg]
        lens = wl.pack_lengths(s.seed, s.n_seq, s.len_lo, s.len_hi, s.N)
        assert lens.sum() == s.N and lens.min() >= s.len_lo and lens.max() <= s.len_hi
    assert wl.prompt_length("floor_half", 301) == 150
    assert wl.prompt_length("round_40pct", 301) == 120
    assert wl.prompt_length("round_40pct", 128) == 51
    w = wl.make(SMALL)
    assert w.N == 700 and w.mask.dtype == np.uint8
    for s in range(5):
        m = w.mask[w.seq_id == s]
        L = m.size
        assert m[:L // 2].sum() == 0 and m[L // 2:].all()


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-7, -(1 + 2**-8), 3.0e38, 1e-40],
                 dtype=np.float32)
    got = wl.bf16_to_f32(wl.bf16_bits(x))
    exp = np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -1.0], dtype=np.float32)
    np.testing.assert_array_equal(got[:5], exp)
    # library rounding (torch, round-to-nearest-even) on random values
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    ref = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(wl.bf16_bits(r), ref)
    np.testing.assert_array_equal(wl.as_f64(wl.bf16_bits(r)),
                                  torch.from_numpy(r).to(torch.bfloat16).double().numpy())


def test_value_distributions():
    w = wl.make(SMALL)
    Wf = wl.as_f64(w.W)
    hf = wl.as_f64(w.h)
    assert abs(Wf.var() * 128 - 1) < 0.02 and abs(Wf.mean()) < 0.01
    assert abs(hf.var() - 1) < 0.02
    assert w.targets.min() >= 0 and w.targets.max() < 900
    assert np.all((w.u >= 0) & (w.u < 1))
    for s in range(5):
        assert np.unique(w.adv[w.seq_id == s]).size == 1


def test_layout_variants_keep_token_rows():
    fam = wl.Family(SMALL)
    base = fam.batch()
    ref = {k: i for i, k in enumerate(base.key())}
    for v in (fam.alone(3), fam.shuffled(11), fam.padded(12), fam.subset([4, 0])):
        for i, (s, p) in enumerate(v.key()):
            if s < 0:
                assert v.mask[i] == 0
                continue
            j = ref[(s, p)]
            assert np.array_equal(v.h[i], base.h[j])
            assert v.targets[i] == base.targets[j] and v.mask[i] == base.mask[j]
    pad = fam.padded(12)
    assert pad.N > base.N and (pad.seq_id < 0).sum() == pad.N - base.N
    dense = fam.all_active()
    assert dense.mask.all() and np.array_equal(dense.h, base.h)


def test_fp32_config():
    w = wl.make(1)
    assert w.h.dtype == np.float32 and w.W.dtype == np.float32
    assert w.h.shape == (64, 256) and w.W.shape == (1000, 256) and w.mask.all()
