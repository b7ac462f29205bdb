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
