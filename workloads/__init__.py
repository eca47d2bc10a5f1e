"""Seeded synthetic inputs for the fused linear log-prob.

The pages describe the operator's inputs as hidden states, target token ids, an active
response mask, the LM-head weight and the rollout temperature (RL-Kernel integration
roadmap for vime, "Operator Integration Plan", linear_logp "vime hook"), and score only
active response tokens (same page, "Consistency Contract").  The workloads here reproduce
the shapes of a Qwen3-8B-sized LM head (the model the pages run) and of a larger-hidden
head, with h ~ N(0, 1) and W ~ N(0, 1/H).  Tokens are packed as variable-length
sequences whose leading part is a masked prompt and whose remainder is the active
response.  No model weights, tokenizer or prompt set are involved: every value is drawn
from a seeded PCG64 generator.

This module only draws random numbers, rounds them to bf16 and lays tokens out.  It holds
none of the method's arithmetic.  Both the oracle-side checks and the GPU path consume
what it returns; neither is imported here.

Every random quantity has its own stream, keyed ``SeedSequence([seed, stream, index])``,
so a sequence's rows are the same bytes whichever batch, order or padding it is placed in.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

# Independent random streams.
STREAM_LENGTHS = 0
STREAM_H = 1
STREAM_W = 2
STREAM_TARGETS = 3
STREAM_UNIFORM = 4
STREAM_ADV = 5
STREAM_PAD = 6
STREAM_PAD_H = 7
STREAM_LOGITS = 8

W_BLOCK_ROWS = 4096  # rows of W drawn per independent sub-stream


# --------------------------------------------------------------------------- bf16 bits

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 copy of bf16 bits (uint16) or of float32 values."""
    if x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_rows(seed: int, stream: int, index: int, rows: int, cols: int, scale: float,
                dtype: str) -> np.ndarray:
    """rows x cols draws of N(0, scale^2) from one sub-stream, as bf16 bits or float32."""
    x = _rng(seed, stream, index).standard_normal((rows, cols), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_bits(x) if dtype == "bf16" else x


def logits_rows(seed: int, rows: int, V: int, scale: float, dtype: str,
                ld: Optional[int] = None) -> np.ndarray:
    """rows x V logits drawn N(0, scale^2), one sub-stream per row (so a row is the same bytes
    in any batch), as bf16 bits or float32; with ld > V each row is padded to ld entries
    (padding holds a large value that must never be read)."""
    ld = V if ld is None else ld
    out = np.empty((rows, ld), dtype=np.uint16 if dtype == "bf16" else np.float32)
    pad = bf16_bits(np.array([1e30], np.float32))[0] if dtype == "bf16" else np.float32(1e30)
    for r in range(rows):
        out[r, :V] = normal_rows(seed, STREAM_LOGITS, r, 1, V, scale, dtype)[0]
        out[r, V:] = pad
    return out


def weight_matrix(seed: int, V: int, H: int, dtype: str) -> np.ndarray:
    """W[V, H] ~ N(0, 1/H), drawn in fixed blocks of rows on worker threads.

    The block partition is fixed, so the bytes do not depend on the thread count."""
    out = np.empty((V, H), dtype=np.uint16 if dtype == "bf16" else np.float32)
    scale = 1.0 / np.sqrt(H)
    nblk = (V + W_BLOCK_ROWS - 1) // W_BLOCK_ROWS

    def fill(b: int) -> None:
        r0 = b * W_BLOCK_ROWS
        r1 = min(V, r0 + W_BLOCK_ROWS)
        out[r0:r1] = normal_rows(seed, STREAM_W, b, r1 - r0, H, scale, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def pack_lengths(seed: int, n_seq: int, lo: int, hi: int, total: int) -> np.ndarray:
    """Seeded sequence lengths in [lo, hi] that sum exactly to ``total``.

    Draw integers uniformly in [lo, hi], scale them to the total, clamp to [lo, hi] and
    settle the remainder one token at a time, round-robin in sequence order."""
    if not (n_seq * lo <= total <= n_seq * hi):
        raise ValueError("lengths cannot pack to the requested total")
    raw = _rng(seed, STREAM_LENGTHS).integers(lo, hi + 1, size=n_seq)
    lens = np.clip(np.floor(raw * total / raw.sum()).astype(np.int64), lo, hi)
    diff = int(total - lens.sum())
    i = 0
    while diff != 0:
        step = 1 if diff > 0 else -1
        if lo <= lens[i] + step <= hi:
            lens[i] += step
            diff -= step
        i = (i + 1) % n_seq
    return lens


# --------------------------------------------------------------------------- specs

@dataclasses.dataclass(frozen=True)
class Spec:
    """Recipe of one workload."""
    name: str
    N: int
    H: int
    V: int
    dtype: str            # "bf16" or "fp32"
    T: float
    n_seq: int
    len_lo: int
    len_hi: int
    prompt: str           # "none", "floor_half" or "round_40pct"
    targets: str          # "uniform" or "sampled" (sampled ones come from the oracle softmax)
    seed: int
    backward: bool = False


CONFIGS: Dict[int, Spec] = {
    1: Spec("tiny-fp32 N=64 H=256 V=1000", 64, 256, 1000, "fp32", 1.0,
            1, 64, 64, "none", "uniform", 1001),
    2: Spec("qwen3-8b-head N=2048 fwd", 2048, 4096, 151936, "bf16", 1.0,
            8, 64, 512, "floor_half", "uniform", 1002),
    3: Spec("qwen3-8b-head N=16384 T=0.7 fwd", 16384, 4096, 151936, "bf16", 0.7,
            64, 128, 512, "round_40pct", "sampled", 1003),
    4: Spec("large-hidden-head N=8192 H=7168 V=129280 fwd", 8192, 7168, 129280, "bf16", 1.0,
            16, 512, 512, "none", "uniform", 1004),
    5: Spec("qwen3-8b-head N=4096 fwd+bwd", 4096, 4096, 151936, "bf16", 1.0,
            16, 64, 512, "floor_half", "uniform", 1005, backward=True),
}


def prompt_length(kind: str, length: int) -> int:
    if kind == "none":
        return 0
    if kind == "floor_half":
        return length // 2
    if kind == "round_40pct":
        return int(np.floor(0.4 * length + 0.5))
    raise ValueError(kind)


# --------------------------------------------------------------------------- workload

@dataclasses.dataclass
class Workload:
    """One batch of inputs plus the identity of every token.

    ``h`` and ``W`` hold bf16 bits (uint16) or float32 values.  ``seq_id`` is -1 for
    padding tokens.  ``u`` holds the per-token uniforms that drive target sampling."""
    spec: Spec
    h: np.ndarray
    W: np.ndarray
    targets: np.ndarray   # int32 [N]
    mask: np.ndarray      # uint8 [N]
    adv: np.ndarray       # float32 [N], the per-sequence advantage broadcast to its tokens
    u: np.ndarray         # float64 [N] in [0, 1)
    seq_id: np.ndarray    # int32 [N]
    pos: np.ndarray       # int32 [N]

    @property
    def N(self) -> int:
        return int(self.h.shape[0])

    @property
    def H(self) -> int:
        return self.spec.H

    @property
    def V(self) -> int:
        return self.spec.V

    @property
    def T(self) -> float:
        return self.spec.T

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def n_active(self) -> int:
        return int(self.mask.astype(bool).sum())

    def key(self) -> List[tuple]:
        """(sequence, position) of every token, the identity kept across layouts."""
        return list(zip(self.seq_id.tolist(), self.pos.tolist()))


@dataclasses.dataclass
class _Sequences:
    spec: Spec
    W: np.ndarray
    h: List[np.ndarray]
    targets: List[np.ndarray]
    mask: List[np.ndarray]
    adv: List[np.ndarray]
    u: List[np.ndarray]


def _sequences(spec: Spec, W: Optional[np.ndarray]) -> _Sequences:
    if spec.n_seq == 1:
        lens = np.array([spec.N], dtype=np.int64)
    else:
        lens = pack_lengths(spec.seed, spec.n_seq, spec.len_lo, spec.len_hi, spec.N)
    if W is None:
        W = weight_matrix(spec.seed, spec.V, spec.H, spec.dtype)

    def one(s: int):
        L = int(lens[s])
        h = normal_rows(spec.seed, STREAM_H, s, L, spec.H, 1.0, spec.dtype)
        tg = _rng(spec.seed, STREAM_TARGETS, s).integers(0, spec.V, size=L).astype(np.int32)
        p = prompt_length(spec.prompt, L)
        m = np.zeros(L, dtype=np.uint8)
        m[p:] = 1
        adv = np.full(L, _rng(spec.seed, STREAM_ADV, s).standard_normal(), dtype=np.float32)
        u = _rng(spec.seed, STREAM_UNIFORM, s).random(L)
        return h, tg, m, adv, u

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(one, range(len(lens))))
    return _Sequences(spec, W, [p[0] for p in parts], [p[1] for p in parts],
                      [p[2] for p in parts], [p[3] for p in parts], [p[4] for p in parts])


def _assemble(sq: _Sequences, order: Sequence[int], pads: Optional[Sequence[int]] = None,
              pad_seed: int = 0, all_active: bool = False) -> Workload:
    """Concatenate sequences in ``order``; ``pads[k]`` padding tokens go before the k-th
    placed sequence and ``pads[-1]`` after the last one."""
    spec = sq.spec
    hs, ts, ms, advs, us, sid, pos = [], [], [], [], [], [], []
    rng_pad = _rng(pad_seed, STREAM_PAD, 1)

    def add_pad(n: int, k: int) -> None:
        if n <= 0:
            return
        hs.append(normal_rows(pad_seed, STREAM_PAD_H, k, n, spec.H, 1.0, spec.dtype))
        ts.append(rng_pad.integers(0, spec.V, size=n).astype(np.int32))
        ms.append(np.zeros(n, dtype=np.uint8))
        advs.append(np.zeros(n, dtype=np.float32))
        us.append(np.zeros(n))
        sid.append(np.full(n, -1, dtype=np.int32))
        pos.append(np.arange(n, dtype=np.int32))

    for k, s in enumerate(order):
        if pads is not None:
            add_pad(int(pads[k]), k)
        L = sq.h[s].shape[0]
        hs.append(sq.h[s])
        ts.append(sq.targets[s])
        ms.append(np.ones(L, dtype=np.uint8) if all_active else sq.mask[s])
        advs.append(sq.adv[s])
        us.append(sq.u[s])
        sid.append(np.full(L, s, dtype=np.int32))
        pos.append(np.arange(L, dtype=np.int32))
    if pads is not None:
        add_pad(int(pads[len(order)]), len(order))

    cat = np.concatenate
    return Workload(spec, np.ascontiguousarray(cat(hs, axis=0)), sq.W, cat(ts), cat(ms),
                    cat(advs), cat(us), cat(sid), cat(pos))


class Family:
    """A workload and the layout variants of the same sequences (scored alone, shuffled,
    padded, all tokens active), for the batch-invariance sweep."""

    def __init__(self, spec: Spec, W: Optional[np.ndarray] = None):
        self.spec = spec
        self._sq = _sequences(spec, W)

    @property
    def W(self) -> np.ndarray:
        return self._sq.W

    @property
    def n_seq(self) -> int:
        return len(self._sq.h)

    def batch(self) -> Workload:
        return _assemble(self._sq, range(self.n_seq))

    def alone(self, s: int) -> Workload:
        return _assemble(self._sq, [s])

    def subset(self, seqs: Sequence[int]) -> Workload:
        return _assemble(self._sq, list(seqs))

    def shuffled(self, shuffle_seed: int) -> Workload:
        order = _rng(shuffle_seed, STREAM_PAD, 0).permutation(self.n_seq)
        return _assemble(self._sq, order.tolist())

    def padded(self, pad_seed: int, max_pad: int = 64) -> Workload:
        pads = _rng(pad_seed, STREAM_PAD, 2).integers(0, max_pad + 1, size=self.n_seq + 1)
        return _assemble(self._sq, range(self.n_seq), pads=pads.tolist(), pad_seed=pad_seed)

    def all_active(self) -> Workload:
        return _assemble(self._sq, range(self.n_seq), all_active=True)

    def use_targets(self, batch_targets: np.ndarray) -> None:
        """Replace every sequence's targets by ``batch_targets``, given in the token order
        of ``batch()``; later layouts carry them along."""
        off = 0
        for s in range(self.n_seq):
            L = self._sq.h[s].shape[0]
            self._sq.targets[s] = np.asarray(batch_targets[off:off + L], dtype=np.int32)
            off += L
        if off != len(batch_targets):
            raise ValueError("target count does not match the batch")


def make(config: int | Spec, W: Optional[np.ndarray] = None) -> Workload:
    spec = CONFIGS[config] if isinstance(config, int) else config
    return Family(spec, W).batch()


def scaled_spec(config: int, **changes) -> Spec:
    """A copy of a config's recipe with some fields changed (reduced sizes for tests)."""
    return dataclasses.replace(CONFIGS[config], **changes)


def with_targets(w: Workload, targets: np.ndarray) -> Workload:
    return dataclasses.replace(w, targets=np.ascontiguousarray(targets, dtype=np.int32))
