"""CPU float64 oracle for the fused LM-head log-prob / entropy op.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The GPU library never calls it
and shares no code with it.

What it computes is the plain, materialised-logit definition, in float64:

* Logits of kept rows: Z = X[kept] @ W^T. The logit projection is the expensive
  matmul of prime-rl PR #3326 ("Don't compute the logprobs and their gradients
  for tokens no loss com..."), author comment.
* Selected-target log-probability: logp_i = Z[i, t_i] - logsumexp(Z[i, :]).
* Policy entropy in nats over the full vocabulary: H_i = -sum_v p_iv log p_iv
  with log p_iv = Z[i, v] - logsumexp(Z[i, :]); SkyRL PR #2374 ("feat(megatron):
  fuse LM-head entropy for RL"), gemini-code-assist suggested change (entropy as
  minus the sum of exp(logp) * logp).
* Rows the keep mask drops get log-prob 0, entropy 0 and no gradient; prime-rl
  PR #3326, Overview (skipped positions are filled with zeros after the
  compact / compute / expand-back sequence).
* Outputs are float precision or better for bf16 inputs; twinkle PR #283 ("Fix
  three memory defects in the Megatron path"), section 1 (float32 compute and
  float32 log-probs and entropies for a bfloat16 input). This oracle keeps
  float64 throughout.
* Gradients: the pages print no backward formula. The oracle takes the
  derivative of L = sum_i g_lp[i] * logp_i + [entropy grad] * g_H[i] * H_i with
  respect to the logits,
      dZ_i = g_lp[i] * (onehot(t_i) - p_i) - g_H[i] * p_i * (log p_i + H_i),
  and then dX[i] = dZ_i @ W, dW = sum_i outer(dZ_i, X[i]). The entropy term is
  present only when entropy gradients are requested; SkyRL PR #2374, "How it
  works" (metric-only entropy adds no gradient work, entropy-loss mode keeps
  the entropy derivative). The formula is pinned by finite differences and by
  torch autograd in the tests.

Inputs are bf16 bit patterns (uint16) decoded exactly to float64, int32 targets
and a uint8 keep mask (nonzero = keep; None = keep every row).
"""

from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns: the 16 bits are the top half of
    an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compact(keep_mask, N: int | None = None) -> np.ndarray:
    """Ascending int32 positions of the kept rows (prime-rl PR #3326, Overview:
    compaction of the masked positions before the chunked computation)."""
    if keep_mask is None:
        return np.arange(N, dtype=np.int32)
    m = np.asarray(keep_mask)
    return np.flatnonzero(m != 0).astype(np.int32)


def _logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def row_stats(X: np.ndarray, W: np.ndarray, targets: np.ndarray):
    """Materialised logits and their per-row statistics, all float64.

    X [R, H], W [V, H], targets [R]. Returns (Z, lse, logp, entropy, logP) where
    logP = Z - lse is the full-vocabulary log-softmax.
    """
    Z = X @ W.T
    lse = _logsumexp_rows(Z)
    logP = Z - lse[:, None]
    P = np.exp(logP)
    logp = logP[np.arange(Z.shape[0]), targets]
    ent = -(P * logP).sum(axis=1)
    return Z, lse, logp, ent, logP


def logit_grad(logP: np.ndarray, ent: np.ndarray, targets: np.ndarray,
               g_logp: np.ndarray, g_entropy: np.ndarray | None,
               entropy_requires_grad: bool) -> np.ndarray:
    """dL/dZ for L = sum g_lp * logp + [entropy grad] * g_H * entropy."""
    P = np.exp(logP)
    R = P.shape[0]
    onehot = np.zeros_like(P)
    onehot[np.arange(R), targets] = 1.0
    dZ = g_logp[:, None] * (onehot - P)
    if entropy_requires_grad:
        dZ = dZ - g_entropy[:, None] * P * (logP + ent[:, None])
    return dZ


def forward_f64(X, W, targets, keep_mask=None):
    """Forward on float64 arrays. Returns dict with full-length [N] arrays
    ``logp``, ``entropy``, ``lse`` (zeros at skipped rows) and ``kept_idx``."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    targets = np.asarray(targets, dtype=np.int64)
    N = X.shape[0]
    idx = compact(keep_mask, N)
    logp = np.zeros(N)
    ent = np.zeros(N)
    lse = np.zeros(N)
    if idx.size:
        _, l, lp, h, _ = row_stats(X[idx], W, targets[idx])
        logp[idx] = lp
        ent[idx] = h
        lse[idx] = l
    return dict(logp=logp, entropy=ent, lse=lse, kept_idx=idx)


def backward_f64(X, W, targets, keep_mask, g_logp, g_entropy,
                 entropy_requires_grad: bool):
    """Backward on float64 arrays. Returns (dX [N, H], dW [V, H]); rows the mask
    drops get exactly zero in dX and contribute nothing to dW."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    targets = np.asarray(targets, dtype=np.int64)
    g_logp = np.asarray(g_logp, dtype=np.float64)
    g_ent = None if g_entropy is None else np.asarray(g_entropy, dtype=np.float64)
    N = X.shape[0]
    idx = compact(keep_mask, N)
    dX = np.zeros_like(X)
    dW = np.zeros_like(W)
    if idx.size:
        _, _, _, h, logP = row_stats(X[idx], W, targets[idx])
        dZ = logit_grad(logP, h, targets[idx], g_logp[idx],
                        None if g_ent is None else g_ent[idx], entropy_requires_grad)
        dX[idx] = dZ @ W
        dW = dZ.T @ X[idx]
    return dX, dW


def forward(hidden_bits, weight_bits, targets, keep_mask=None):
    """Forward from bf16 bit patterns (see ``forward_f64``)."""
    return forward_f64(bf16_to_f64(hidden_bits), bf16_to_f64(weight_bits), targets, keep_mask)


def backward(hidden_bits, weight_bits, targets, keep_mask, g_logp, g_entropy,
             entropy_requires_grad: bool):
    """Backward from bf16 bit patterns (see ``backward_f64``)."""
    return backward_f64(bf16_to_f64(hidden_bits), bf16_to_f64(weight_bits), targets,
                        keep_mask, g_logp, g_entropy, entropy_requires_grad)


def rows_fwd_bwd(hidden_bits, weight_bits, targets, rows, g_logp, g_entropy,
                 entropy_requires_grad: bool, W64: np.ndarray | None = None,
                 want_dw: bool = True):
    """Forward and backward restricted to the given (kept) rows.

    Rows are independent in the forward and in dX, so this gives exactly the
    values the full problem has at those rows. dW returned here is the
    contribution of these rows only, which equals the full op's dW when the
    keep mask selects exactly these rows.

    Returns dict(logp, entropy, lse, dX [len(rows), H], dW [V, H] or None).
    """
    rows = np.asarray(rows, dtype=np.int64)
    Wd = bf16_to_f64(weight_bits) if W64 is None else W64
    Xr = bf16_to_f64(np.asarray(hidden_bits)[rows])
    tr = np.asarray(targets, dtype=np.int64)[rows]
    _, lse, lp, h, logP = row_stats(Xr, Wd, tr)
    gl = np.asarray(g_logp, dtype=np.float64)[rows]
    gh = None if g_entropy is None else np.asarray(g_entropy, dtype=np.float64)[rows]
    dZ = logit_grad(logP, h, tr, gl, gh, entropy_requires_grad)
    dX = dZ @ Wd
    dW = dZ.T @ Xr if want_dw else None
    return dict(logp=lp, entropy=h, lse=lse, dX=dX, dW=dW)


def logits_input_fwd_bwd(logits, targets, g_logp, g_entropy, entropy_requires_grad):
    """Log-prob, entropy and dL/dlogits from already materialised logits [R, V]
    (the twinkle PR #283 ``selective_log_softmax`` contract, section 1), in
    float64."""
    Z = np.asarray(logits, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    lse = _logsumexp_rows(Z)
    logP = Z - lse[:, None]
    P = np.exp(logP)
    lp = logP[np.arange(Z.shape[0]), t]
    h = -(P * logP).sum(axis=1)
    dZ = logit_grad(logP, h, t, np.asarray(g_logp, np.float64),
                    None if g_entropy is None else np.asarray(g_entropy, np.float64),
                    entropy_requires_grad)
    return dict(logp=lp, entropy=h, lse=lse, dlogits=dZ)


# --------------------------------------------------------------------------
# Vocabulary shards (tensor parallelism over the weight rows)
# --------------------------------------------------------------------------
# SkyRL PR #2374 ("feat(megatron): fuse LM-head entropy for RL") splits the
# weight rows over tensor-parallel ranks: each rank reduces over its own
# vocabulary range and the ranks combine their results with collectives
# (gemini-code-assist review); the hidden gradient a rank computes from its
# shard is its local share, reduced by the caller, while the weight gradient
# is exactly the shard's rows (cursor and greptile reviews). The functions
# below state those per-shard quantities and their combination in float64.

def shard_partials_f64(X, W_shard, targets, keep_mask, vocab_start: int) -> np.ndarray:
    """Per-row statistics of the logits over the vocabulary range
    [vocab_start, vocab_start + V_shard) that W_shard holds.

    Returns float64 [N, 4]: m = max_v z_v, s = sum_v exp(z_v - m),
    b = sum_v exp(z_v - m) (z_v - m), and z_t, the target's logit when the
    target lies in the range (NaN otherwise). Skipped rows get
    (-inf, 0, 0, NaN), the statistics of an empty set.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W_shard, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    N = X.shape[0]
    out = np.empty((N, 4))
    out[:] = (-np.inf, 0.0, 0.0, np.nan)
    idx = compact(keep_mask, N)
    if idx.size:
        Z = X[idx] @ W.T
        m = Z.max(axis=1)
        D = Z - m[:, None]
        E = np.exp(D)
        local = t[idx] - vocab_start
        inside = (local >= 0) & (local < W.shape[0])
        z = np.full(idx.size, np.nan)
        rows = np.flatnonzero(inside)
        z[rows] = Z[rows, local[rows]]
        out[idx, 0] = m
        out[idx, 1] = E.sum(axis=1)
        out[idx, 2] = (E * D).sum(axis=1)
        out[idx, 3] = z
    return out


def merge_shard_partials(parts, keep_mask, N: int):
    """Combines the statistics of disjoint vocabulary ranges, in the order
    given, into the whole vocabulary's: with M = max_p m_p and
    a_p = exp(m_p - M),
        s = sum_p a_p s_p,   b = sum_p a_p (b_p + (m_p - M) s_p),
    so that LSE = M + ln s and entropy = ln s - b / s (both follow from
    sum_v exp(z_v - M) = s and sum_v exp(z_v - M)(z_v - M) = b). The
    log-probability takes z_t from the range that holds the target.
    Returns dict(logp, entropy, lse) with zeros at skipped rows.
    """
    parts = np.asarray(parts, dtype=np.float64)
    idx = compact(keep_mask, N)
    logp = np.zeros(N)
    ent = np.zeros(N)
    lse = np.zeros(N)
    for i in idx:
        M = -np.inf
        for p in range(parts.shape[0]):
            M = max(M, parts[p, i, 0])
        s = 0.0
        b = 0.0
        z = np.nan
        for p in range(parts.shape[0]):
            mp, sp, bp, zp = parts[p, i]
            if mp == -np.inf:
                continue
            a = math.exp(mp - M)
            s += a * sp
            b += a * (bp + (mp - M) * sp)
            if not np.isnan(zp):
                z = zp
        lse[i] = M + math.log(s)
        ent[i] = math.log(s) - b / s
        logp[i] = z - lse[i]
    return dict(logp=logp, entropy=ent, lse=lse)


def backward_shard_f64(X, W_shard, targets, keep_mask, vocab_start: int, lse, ent,
                       g_logp, g_entropy, entropy_requires_grad: bool):
    """One vocabulary shard's backward with the whole vocabulary's LSE and
    entropy (full-length [N] arrays, as merge_shard_partials returns them):
    dZ over the shard's columns by the same formula as logit_grad, then
    (dX_share [N, H] = dZ W_shard on the kept rows, zero elsewhere;
    dW_shard [V_shard, H] = dZ^T X_kept)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W_shard, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    N = X.shape[0]
    idx = compact(keep_mask, N)
    dX = np.zeros_like(X)
    dW = np.zeros_like(W)
    if idx.size:
        Z = X[idx] @ W.T
        logP = Z - np.asarray(lse, np.float64)[idx][:, None]
        P = np.exp(logP)
        local = t[idx] - vocab_start
        onehot = np.zeros_like(P)
        rows = np.flatnonzero((local >= 0) & (local < W.shape[0]))
        onehot[rows, local[rows]] = 1.0
        g = np.asarray(g_logp, np.float64)[idx]
        dZ = g[:, None] * (onehot - P)
        if entropy_requires_grad:
            gh = np.asarray(g_entropy, np.float64)[idx]
            h = np.asarray(ent, np.float64)[idx]
            dZ = dZ - gh[:, None] * P * (logP + h[:, None])
        dX[idx] = dZ @ W
        dW = dZ.T @ X[idx]
    return dX, dW
