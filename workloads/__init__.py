"""Seeded synthetic inputs for the fused LM-head log-prob / entropy op.

This module only draws random inputs and rounds them to bfloat16. It holds no
arithmetic of the op itself, so both the CPU oracle and the GPU path can take
their inputs from it without sharing any of the method's code.

Shapes and distributions follow the workloads the pages discuss:

* prime-rl PR #3326 ("Don't compute the logprobs and their gradients for tokens
  no loss com..."), author comment and Overview: the LM-head matmul is
  [N, 4096] @ [4096, 151936] on a Qwen model; a keep mask selects the positions
  some loss term reads.
* SkyRL PR #2374 ("feat(megatron): fuse LM-head entropy for RL"), Performance
  table: H=4096, V=131072, 16K tokens, active-row fractions 100/95/73/64/23 %.
* twinkle PR #283 ("Fix three memory defects in the Megatron path"), PR
  information and Experiment results: Qwen3-4B GRPO at 16384 tokens, vocab
  151936.

Random numbers come from numpy's PCG64 seeded through ``SeedSequence``. Each
input tensor has its own stream, and large tensors are drawn in fixed row
blocks, each block from its own child seed, so the bits do not depend on the
number of threads used to draw them.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Stream order is fixed: hidden, weight, targets, keep, g_logp, g_entropy, extra.
_STREAMS = ("hidden", "weight", "targets", "keep", "g_logp", "g_entropy", "extra")
_BLOCK_ROWS = 1024
_THREADS = 8

# Active-row fractions of the SkyRL PR #2374 Performance table.
KEEP_SWEEP = (1.00, 0.95, 0.73, 0.64, 0.23)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int) -> dict:
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, kids))


def _normal_bf16(ss: np.random.SeedSequence, rows: int, cols: int, std,
                 out_f32_hook=None) -> np.ndarray:
    """Draw a [rows, cols] N(0, std) matrix in float32 and round it to bf16.

    ``std`` is a scalar or a per-row float32 vector. ``out_f32_hook`` may edit a
    float32 block in place before rounding (used for the +3 sigma bias).
    """
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS
    kids = ss.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.uint16)
    std_arr = np.asarray(std, dtype=np.float32)

    def one(b):
        r0 = b * _BLOCK_ROWS
        r1 = min(rows, r0 + _BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(kids[b]))
        blk = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std_arr.ndim == 0:
            blk *= std_arr
        else:
            blk *= std_arr[r0:r1, None]
        if out_f32_hook is not None:
            out_f32_hook(r0, r1, blk)
        out[r0:r1] = f32_to_bf16_bits(blk)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, range(nblk)))
    return out


def _gen(ss):
    return np.random.Generator(np.random.PCG64(ss))


@dataclass
class Workload:
    """One synthetic batch: bf16 bit patterns, int32 targets, u8 keep mask."""

    name: str
    hidden: np.ndarray          # uint16 [N, H]  (bf16 bits)
    weight: np.ndarray          # uint16 [V, H]  (bf16 bits)
    targets: np.ndarray         # int32  [N]
    keep: np.ndarray | None     # uint8  [N], or None = keep every row
    g_logp: np.ndarray          # float32 [N]
    g_entropy: np.ndarray       # float32 [N]
    return_entropy: bool = True
    entropy_requires_grad: bool = True
    backward: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def N(self):
        return self.hidden.shape[0]

    @property
    def H(self):
        return self.hidden.shape[1]

    @property
    def V(self):
        return self.weight.shape[0]

    def kept_rows(self) -> np.ndarray:
        if self.keep is None:
            return np.arange(self.N, dtype=np.int64)
        return np.flatnonzero(self.keep)


def _upstream(st, N):
    g_lp = _gen(st["g_logp"]).standard_normal(N, dtype=np.float32)
    g_h = _gen(st["g_entropy"]).standard_normal(N, dtype=np.float32)
    return g_lp, g_h


def tiny_batch(seed: int = 1) -> Workload:
    """Tiny forward+backward: N=128, H=512, V=8192, keep ~ Bernoulli(0.7).

    hidden ~ N(0, 1); weight ~ N(0, std 1/sqrt(H)), giving unit-std logits.
    """
    N, H, V = 128, 512, 8192
    st = _streams(seed)
    X = _normal_bf16(st["hidden"], N, H, 1.0)
    W = _normal_bf16(st["weight"], V, H, 1.0 / math.sqrt(H))
    t = _gen(st["targets"]).integers(0, V, N, dtype=np.int32)
    keep = (_gen(st["keep"]).random(N) < 0.7).astype(np.uint8)
    g_lp, g_h = _upstream(st, N)
    return Workload("tiny N128 H512 V8192", X, W, t, keep, g_lp, g_h,
                    meta=dict(workload="tiny_batch", seed=seed, keep_fraction=0.7))


def dense_rl(keep_fraction: float = 1.0, seed: int = 2, N: int = 16384,
            H: int = 4096, V: int = 131072, mask: bool = True) -> Workload:
    """Dense RL shape: N=16384, H=4096, V=131072, Bernoulli keep mask.

    One draw of X, W, targets and upstream grads serves the whole keep-fraction
    sweep; the mask is ``u < f`` for one shared uniform draw ``u``, so masks of
    lower fractions are subsets of higher ones. ``mask=False`` passes no mask.
    """
    st = _streams(seed)
    X = _normal_bf16(st["hidden"], N, H, 1.0)
    W = _normal_bf16(st["weight"], V, H, 0.02)
    t = _gen(st["targets"]).integers(0, V, N, dtype=np.int32)
    u = _gen(st["keep"]).random(N)
    keep = (u < keep_fraction).astype(np.uint8) if mask else None
    g_lp, g_h = _upstream(st, N)
    return Workload(f"dense RL N{N} H{H} V{V} keep{keep_fraction:.2f}", X, W, t,
                    keep, g_lp, g_h,
                    meta=dict(workload="dense_rl", seed=seed, keep_fraction=keep_fraction))


def dense_rl_masks(fractions=KEEP_SWEEP, seed: int = 2, N: int = 16384) -> dict:
    """The keep masks ``dense_rl(f).keep`` for each fraction f, from the same
    uniform draw, without generating X and W again."""
    u = _gen(_streams(seed)["keep"]).random(N)
    return {f: (u < f).astype(np.uint8) for f in fractions}


def packed_grpo_layout(N: int, V: int, nseq: int, rng: np.random.Generator):
    """Packed sequences with prompt/completion split and next-token targets.

    Returns (tokens, targets, keep, seq_starts). ``keep[i]`` is 1 iff position
    i+1 is a completion token of the same sequence (the next-token shift); the
    last position of each sequence has keep 0 and target 0.
    """
    cuts = np.sort(rng.choice(np.arange(1, N), size=nseq - 1, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int64)
    ends = np.concatenate([cuts, [N]]).astype(np.int64)
    frac = rng.uniform(0.2, 0.6, size=nseq)
    tokens = rng.integers(0, V, N, dtype=np.int32)
    targets = np.zeros(N, dtype=np.int32)
    keep = np.zeros(N, dtype=np.uint8)
    for s, e, f in zip(starts, ends, frac):
        L = int(e - s)
        plen = int(round(f * L))
        targets[s:e - 1] = tokens[s + 1:e]
        lo = s + max(plen, 1) - 1
        keep[lo:e - 1] = 1
    return tokens, targets, keep, starts


def packed_grpo(seed: int = 3, N: int = 16384, H: int = 4096, V: int = 151936) -> Workload:
    """Packed GRPO batch: 16 sequences, prompt 20-60 % of each (keep 0),
    completion kept, next-token targets, and a +3 sigma bias on the weight row
    of each kept target so the logits are peaked. Entropy is metric-only.
    """
    st = _streams(seed)
    rng = _gen(st["extra"])
    _, t, keep, starts = packed_grpo_layout(N, V, 16, rng)
    X = _normal_bf16(st["hidden"], N, H, 1.0)
    Xf = bf16_bits_to_f32(X)
    sigma = math.sqrt(H) * 0.02
    kept = np.flatnonzero(keep)
    # first kept row (ascending) for each distinct kept target
    uniq_t, first = np.unique(t[kept], return_index=True)
    src_rows = kept[first]
    bias_for = {}
    for v, r in zip(uniq_t.tolist(), src_rows.tolist()):
        x = Xf[r].astype(np.float64)
        bias_for[v] = (3.0 * sigma * x / float(x @ x)).astype(np.float32)
    biased = np.array(sorted(bias_for), dtype=np.int64)

    def hook(r0, r1, blk):
        lo = np.searchsorted(biased, r0)
        hi = np.searchsorted(biased, r1)
        for v in biased[lo:hi].tolist():
            blk[v - r0] += bias_for[v]

    W = _normal_bf16(st["weight"], V, H, 0.02, out_f32_hook=hook)
    g_lp, g_h = _upstream(st, N)
    return Workload(f"packed GRPO N{N} H{H} V{V}", X, W, t, keep, g_lp, g_h,
                    return_entropy=True, entropy_requires_grad=False,
                    meta=dict(workload="packed_grpo", seed=seed, seq_starts=starts,
                              keep_fraction=float(keep.mean())))


def fp32_stress(seed: int = 4, N: int = 16384, H: int = 2560, V: int = 151936) -> Workload:
    """fp32-accuracy stress: per-row scale s_i ~ LogUniform(0.5, 8) on the
    hidden state before bf16 rounding; every row kept; entropy grad on."""
    st = _streams(seed)
    s = np.exp(_gen(st["extra"]).uniform(math.log(0.5), math.log(8.0), N)).astype(np.float32)
    X = _normal_bf16(st["hidden"], N, H, s)
    W = _normal_bf16(st["weight"], V, H, 0.02)
    t = _gen(st["targets"]).integers(0, V, N, dtype=np.int32)
    keep = np.ones(N, dtype=np.uint8)
    g_lp, g_h = _upstream(st, N)
    return Workload(f"fp32 stress N{N} H{H} V{V}", X, W, t, keep, g_lp, g_h,
                    meta=dict(workload="fp32_stress", seed=seed, keep_fraction=1.0, row_scale=s))


def span_keep(N: int, rng: np.random.Generator, lo: int = 64, hi: int = 2048,
              p: float = 0.5) -> np.ndarray:
    """Keep mask in contiguous spans of U{lo..hi} tokens, each kept with prob p."""
    keep = np.zeros(N, dtype=np.uint8)
    i = 0
    while i < N:
        L = int(rng.integers(lo, hi + 1))
        if rng.random() < p:
            keep[i:min(N, i + L)] = 1
        i += L
    return keep


def scoring(seed: int = 5, N: int = 262144, H: int = 5120, V: int = 152064) -> Workload:
    """Reference-model scoring, forward only: keep mask in contiguous spans."""
    st = _streams(seed)
    X = _normal_bf16(st["hidden"], N, H, 1.0)
    W = _normal_bf16(st["weight"], V, H, 0.02)
    t = _gen(st["targets"]).integers(0, V, N, dtype=np.int32)
    keep = span_keep(N, _gen(st["keep"]))
    g_lp, g_h = _upstream(st, N)
    return Workload(f"scoring N{N} H{H} V{V}", X, W, t, keep, g_lp, g_h,
                    return_entropy=True, entropy_requires_grad=False, backward=False,
                    meta=dict(workload="scoring", seed=seed, keep_fraction=float(keep.mean())))


def small(N: int, H: int, V: int, seed: int = 0, keep_fraction: float = 0.7,
          x_std: float = 1.0, w_std: float | None = None, mask: bool = True,
          return_entropy: bool = True, entropy_requires_grad: bool = True) -> Workload:
    """Arbitrary small shape with the tiny batch's distributions (for edge cases)."""
    st = _streams(seed)
    if w_std is None:
        w_std = 1.0 / math.sqrt(H)
    X = _normal_bf16(st["hidden"], N, H, x_std)
    W = _normal_bf16(st["weight"], V, H, w_std)
    t = _gen(st["targets"]).integers(0, V, N, dtype=np.int32) if V > 0 else np.zeros(N, np.int32)
    keep = (_gen(st["keep"]).random(N) < keep_fraction).astype(np.uint8) if mask else None
    g_lp, g_h = _upstream(st, N)
    return Workload(f"small N{N} H{H} V{V}", X, W, t, keep, g_lp, g_h,
                    return_entropy=return_entropy,
                    entropy_requires_grad=entropy_requires_grad,
                    meta=dict(seed=seed, keep_fraction=keep_fraction))


def sample_rows(rows: np.ndarray, n: int, seed: int) -> np.ndarray:
    """Seeded, sorted subsample of ``n`` entries of ``rows`` (all if fewer)."""
    rows = np.asarray(rows)
    if rows.size <= n:
        return np.sort(rows)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919])))
    return np.sort(g.choice(rows, size=n, replace=False))


def row_mask(N: int, rows: np.ndarray) -> np.ndarray:
    """u8 keep mask of length N with ones exactly at ``rows``."""
    m = np.zeros(N, dtype=np.uint8)
    m[np.asarray(rows, dtype=np.int64)] = 1
    return m


WORKLOADS = {"tiny": tiny_batch, "dense_rl": dense_rl, "packed_grpo": packed_grpo,
             "fp32_stress": fp32_stress, "scoring": scoring}
