"""Pins of the CPU float64 oracle against facts other than itself.

Each test fixes the oracle by something the pages or the mathematics determine:
closed forms, central finite differences, torch's own log-softmax / entropy /
autograd in float64, invariants, brute force. The mutation tests at the end
plant plausible mistakes in a copy of the oracle's arithmetic and check that
at least one pin catches each.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import lmhead_ref as ref
from workloads import f32_to_bf16_bits


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# --------------------------------------------------------------------------
# compaction: brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bernoulli", "ones", "zeros", "alternating",
                                  "first", "last", "spans"])
def test_compaction_brute_force(kind):
    N = 1000
    rng = np.random.default_rng(3)
    if kind == "bernoulli":
        m = (rng.random(N) < 0.37).astype(np.uint8) * rng.integers(1, 255, N).astype(np.uint8)
    elif kind == "ones":
        m = np.ones(N, np.uint8)
    elif kind == "zeros":
        m = np.zeros(N, np.uint8)
    elif kind == "alternating":
        m = (np.arange(N) % 2).astype(np.uint8)
    elif kind == "first":
        m = np.zeros(N, np.uint8); m[0] = 1
    elif kind == "last":
        m = np.zeros(N, np.uint8); m[-1] = 1
    else:
        m = np.zeros(N, np.uint8); m[100:300] = 7; m[900:] = 1
    brute = []
    for i in range(N):
        if m[i] != 0:
            brute.append(i)
    got = oracle.compact(m)
    assert got.dtype == np.int32
    assert got.tolist() == brute
    assert oracle.compact(None, 5).tolist() == [0, 1, 2, 3, 4]


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_uniform_logits_closed_form():
    """W = 0 gives equal logits: logp = -ln V, entropy = ln V, the entropy
    gradient vanishes and dZ = g_lp * (onehot - 1/V)."""
    V, H, N = 131072, 8, 6
    rng = np.random.default_rng(0)
    Xb = _bf16(rng.standard_normal((N, H)))
    Wb = np.zeros((V, H), np.uint16)
    t = rng.integers(0, V, N).astype(np.int32)
    keep = np.array([1, 0, 1, 1, 0, 1], np.uint8)
    out = oracle.forward(Xb, Wb, t, keep)
    lnV = 17.0 * math.log(2.0)  # V = 2**17
    kept = keep != 0
    np.testing.assert_allclose(out["logp"][kept], -lnV, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["entropy"][kept], lnV, rtol=0, atol=1e-13)
    assert np.all(out["logp"][~kept] == 0) and np.all(out["entropy"][~kept] == 0)

    g_lp = rng.standard_normal(N)
    g_h = rng.standard_normal(N)
    dX, dW = oracle.backward(Xb, Wb, t, keep, g_lp, g_h, True)
    assert np.all(dX == 0)  # dX = dZ @ W with W = 0
    X = oracle.bf16_to_f64(Xb)
    expect = np.zeros((V, H))
    for i in np.flatnonzero(kept):
        expect -= g_lp[i] / V * X[i][None, :]
        expect[t[i]] += g_lp[i] * X[i]
    np.testing.assert_allclose(dW, expect, rtol=0, atol=1e-12)


def test_two_level_logits_closed_form():
    """X row = e0, W[:, 0] = 0 except W[t*, 0] = a. Then the hot token has
    p = 1 / (1 + (V-1) e^-a) and every other token e^-a times that."""
    V, H, a, hot = 131072, 4, 40.0, 1234
    Wf = np.zeros((V, H), np.float32)
    Wf[hot, 0] = a
    Wb = _bf16(Wf)
    Xb = _bf16(np.tile(np.eye(1, H, 0, dtype=np.float32), (3, 1)))
    t = np.array([hot, 7, V - 1], np.int32)
    out = oracle.forward(Xb, Wb, t)
    eps = (V - 1) * math.exp(-a)
    log_pt = -math.log1p(eps)
    ent = math.log1p(eps) + a * eps / (1.0 + eps)
    # float64 summation of 1 + (V-1) e^-a loses a few 1e-15 (the hot term is 1)
    np.testing.assert_allclose(out["logp"][0], log_pt, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["logp"][1:], -a + log_pt, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["entropy"], ent, rtol=0, atol=1e-14)
    assert out["entropy"].max() < 1e-10  # one-hot dominant row: entropy ~ 0
    np.testing.assert_allclose(out["lse"], a - log_pt, rtol=0, atol=1e-12)


def test_two_point_vocab_closed_form():
    """V = 2 with logits (0, d): logp_1 = -log1p(e^-d), entropy is the binary
    entropy of sigmoid(d), and d entropy/d d = -d * p0 * p1."""
    d = 1.5
    Xb = _bf16([[1.0, 0.0]])
    Wb = _bf16([[0.0, 0.0], [d, 0.0]])
    out = oracle.forward(Xb, Wb, np.array([1], np.int32))
    p1 = 1.0 / (1.0 + math.exp(-d))
    p0 = 1.0 - p1
    np.testing.assert_allclose(out["logp"][0], math.log(p1), atol=1e-15)
    np.testing.assert_allclose(out["entropy"][0], -(p0 * math.log(p0) + p1 * math.log(p1)),
                               atol=1e-15)
    # only the entropy gradient: dL/dW[1,0] = dH/dd * x0 = -d p0 p1
    _, dW = oracle.backward(Xb, Wb, np.array([1], np.int32), None, np.zeros(1),
                            np.ones(1), True)
    np.testing.assert_allclose(dW[1, 0], -d * p0 * p1, atol=1e-15)
    np.testing.assert_allclose(dW[0, 0], d * p0 * p1, atol=1e-15)


# --------------------------------------------------------------------------
# finite differences
# --------------------------------------------------------------------------

def _loss(X, W, t, keep, g_lp, g_h, erg):
    out = oracle.forward_f64(X, W, t, keep)
    L = float((g_lp * out["logp"]).sum())
    if erg:
        L += float((g_h * out["entropy"]).sum())
    return L


@pytest.mark.parametrize("erg", [True, False])
def test_gradients_central_differences(erg):
    rng = np.random.default_rng(11)
    N, H, V = 5, 3, 7
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    t = rng.integers(0, V, N)
    keep = np.array([1, 0, 1, 1, 0], np.uint8)
    g_lp = rng.standard_normal(N)
    g_h = rng.standard_normal(N)
    dX, dW = oracle.backward_f64(X, W, t, keep, g_lp, g_h, erg)
    h = 1e-6
    fdX = np.zeros_like(X)
    for i in range(N):
        for j in range(H):
            Xp = X.copy(); Xp[i, j] += h
            Xm = X.copy(); Xm[i, j] -= h
            fdX[i, j] = (_loss(Xp, W, t, keep, g_lp, g_h, erg) -
                         _loss(Xm, W, t, keep, g_lp, g_h, erg)) / (2 * h)
    fdW = np.zeros_like(W)
    for v in range(V):
        for j in range(H):
            Wp = W.copy(); Wp[v, j] += h
            Wm = W.copy(); Wm[v, j] -= h
            fdW[v, j] = (_loss(X, Wp, t, keep, g_lp, g_h, erg) -
                         _loss(X, Wm, t, keep, g_lp, g_h, erg)) / (2 * h)
    assert np.abs(dX - fdX).max() < 1e-7
    assert np.abs(dW - fdW).max() < 1e-7
    # masked rows: exactly zero gradient
    assert np.all(dX[keep == 0] == 0.0)


# --------------------------------------------------------------------------
# torch float64 cross-check (different library routines, autograd gradients)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("erg", [True, False])
def test_torch_float64_cross_check(erg):
    rng = np.random.default_rng(5)
    N, H, V = 24, 16, 97
    X = rng.standard_normal((N, H)) * 2.0
    W = rng.standard_normal((V, H)) * 0.7
    t = rng.integers(0, V, N)
    keep = (rng.random(N) < 0.6).astype(np.uint8)
    g_lp = rng.standard_normal(N)
    g_h = rng.standard_normal(N)

    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    kt = torch.tensor(keep.astype(bool))
    logits = Xt[kt] @ Wt.T
    lp = torch.log_softmax(logits, dim=-1).gather(1, torch.tensor(t)[kt][:, None])[:, 0]
    ent = torch.distributions.Categorical(logits=logits).entropy()
    L = (torch.tensor(g_lp)[kt] * lp).sum()
    if erg:
        L = L + (torch.tensor(g_h)[kt] * ent).sum()
    L.backward()

    out = oracle.forward_f64(X, W, t, keep)
    np.testing.assert_allclose(out["logp"][keep != 0], lp.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["entropy"][keep != 0], ent.detach().numpy(), rtol=0, atol=1e-12)
    dX, dW = oracle.backward_f64(X, W, t, keep, g_lp, g_h, erg)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=0, atol=1e-12)


def test_logits_input_variant_matches_torch():
    rng = np.random.default_rng(9)
    R, V = 7, 33
    Z = rng.standard_normal((R, V)) * 5
    t = rng.integers(0, V, R)
    g_lp = rng.standard_normal(R)
    g_h = rng.standard_normal(R)
    Zt = torch.tensor(Z, requires_grad=True)
    lp = torch.log_softmax(Zt, -1).gather(1, torch.tensor(t)[:, None])[:, 0]
    ent = torch.distributions.Categorical(logits=Zt).entropy()
    ((torch.tensor(g_lp) * lp).sum() + (torch.tensor(g_h) * ent).sum()).backward()
    out = oracle.logits_input_fwd_bwd(Z, t, g_lp, g_h, True)
    np.testing.assert_allclose(out["logp"], lp.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(out["entropy"], ent.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(out["dlogits"], Zt.grad.numpy(), atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def _rand_case(seed, N=16, H=12, V=50, scale=3.0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H)) * scale
    W = rng.standard_normal((V, H))
    t = rng.integers(0, V, N)
    keep = (rng.random(N) < 0.7).astype(np.uint8)
    g_lp = rng.standard_normal(N)
    g_h = rng.standard_normal(N)
    return X, W, t, keep, g_lp, g_h


def test_invariants_bounds_and_dw_column_sums():
    X, W, t, keep, g_lp, g_h = _rand_case(1)
    out = oracle.forward_f64(X, W, t, keep)
    k = keep != 0
    assert np.all(out["logp"][k] <= 0)
    assert np.all(out["entropy"][k] >= 0)
    assert np.all(out["entropy"][k] <= math.log(W.shape[0]) + 1e-12)
    _, dW = oracle.backward_f64(X, W, t, keep, g_lp, g_h, True)
    # each dZ row sums to zero, so the vocab-sum of dW vanishes
    assert np.abs(dW.sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(dW).max())


def test_invariant_vocab_permutation():
    X, W, t, keep, g_lp, g_h = _rand_case(2)
    perm = np.random.default_rng(7).permutation(W.shape[0])
    inv = np.argsort(perm)
    Wp = W[perm]          # new row r holds old row perm[r]
    tp = inv[t]           # old target v now lives at row inv[v]
    a = oracle.forward_f64(X, W, t, keep)
    b = oracle.forward_f64(X, Wp, tp, keep)
    np.testing.assert_allclose(a["logp"], b["logp"], atol=1e-12)
    np.testing.assert_allclose(a["entropy"], b["entropy"], atol=1e-12)
    dXa, dWa = oracle.backward_f64(X, W, t, keep, g_lp, g_h, True)
    dXb, dWb = oracle.backward_f64(X, Wp, tp, keep, g_lp, g_h, True)
    np.testing.assert_allclose(dXa, dXb, atol=1e-12)
    np.testing.assert_allclose(dWa[perm], dWb, atol=1e-12)


def test_invariant_constant_logit_shift():
    """Appending a hidden column of ones with a constant weight column c shifts
    every logit of a row by c: log-probs, entropies and dX on the original
    columns do not change."""
    X, W, t, keep, g_lp, g_h = _rand_case(3)
    c = 2.75
    X2 = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    W2 = np.concatenate([W, np.full((W.shape[0], 1), c)], axis=1)
    a = oracle.forward_f64(X, W, t, keep)
    b = oracle.forward_f64(X2, W2, t, keep)
    np.testing.assert_allclose(a["logp"], b["logp"], atol=1e-12)
    np.testing.assert_allclose(a["entropy"], b["entropy"], atol=1e-12)
    dXa, dWa = oracle.backward_f64(X, W, t, keep, g_lp, g_h, True)
    dXb, dWb = oracle.backward_f64(X2, W2, t, keep, g_lp, g_h, True)
    np.testing.assert_allclose(dXa, dXb[:, :-1], atol=1e-12)
    np.testing.assert_allclose(dWa, dWb[:, :-1], atol=1e-12)
    # the constant column's dX entry is sum_v dZ_v * c = 0
    assert np.abs(dXb[:, -1]).max() < 1e-12


def test_mask_semantics_equal_dense_on_kept_rows():
    X, W, t, keep, g_lp, g_h = _rand_case(4)
    k = np.flatnonzero(keep)
    a = oracle.forward_f64(X, W, t, keep)
    b = oracle.forward_f64(X[k], W, t[k], None)
    np.testing.assert_array_equal(a["logp"][k], b["logp"])
    np.testing.assert_array_equal(a["entropy"][k], b["entropy"])
    skipped = keep == 0
    assert np.all(a["logp"][skipped] == 0) and np.all(a["entropy"][skipped] == 0)
    # +0.0, not -0.0
    assert not np.any(np.signbit(a["logp"][skipped]))
    dXa, dWa = oracle.backward_f64(X, W, t, keep, g_lp, g_h, True)
    dXb, dWb = oracle.backward_f64(X[k], W, t[k], None, g_lp[k], g_h[k], True)
    np.testing.assert_array_equal(dXa[k], dXb)
    np.testing.assert_array_equal(dWa, dWb)
    assert np.all(dXa[skipped] == 0) and not np.any(np.signbit(dXa[skipped]))


def test_rows_helper_equals_full_problem():
    X, W, t, keep, g_lp, g_h = _rand_case(6)
    Xb, Wb = _bf16(X), _bf16(W)
    rows = np.flatnonzero(keep)[::2]
    r = oracle.rows_fwd_bwd(Xb, Wb, t, rows, g_lp, g_h, True)
    mask = np.zeros(len(t), np.uint8); mask[rows] = 1
    full = oracle.forward(Xb, Wb, t, mask)
    dX, dW = oracle.backward(Xb, Wb, t, mask, g_lp, g_h, True)
    np.testing.assert_allclose(r["logp"], full["logp"][rows], atol=1e-13)
    np.testing.assert_allclose(r["entropy"], full["entropy"][rows], atol=1e-13)
    np.testing.assert_allclose(r["dX"], dX[rows], atol=1e-13)
    np.testing.assert_allclose(r["dW"], dW, atol=1e-13)


def test_bf16_decode_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 1e-30, -65504.0, 2.0 ** -133], np.float32)
    bits = _bf16(vals)
    dec = oracle.bf16_to_f64(bits)
    # each value above is exactly representable in bf16 except pi-ish and 1e-30,
    # which must decode to the float32 whose low 16 bits are zero
    assert dec[0] == 0.0 and dec[1] == 1.0 and dec[2] == -2.5 and dec[3] == 3.140625
    assert dec[5] == -65536.0  # -65504 rounds to nearest-even bf16 = -65536
    assert dec[6] == 2.0 ** -133
    assert (np.float32(dec[4]).view(np.uint32) & 0xFFFF) == 0


# --------------------------------------------------------------------------
# planted mistakes: each plausible error must fail at least one pin
# --------------------------------------------------------------------------

def _mut_drop_entropy_term(logP, ent, targets, g_lp, g_h, erg):
    return _orig_logit_grad(logP, ent, targets, g_lp, g_h, False)


def _mut_entropy_sign(logP, ent, targets, g_lp, g_h, erg):
    P = np.exp(logP)
    d = _orig_logit_grad(logP, ent, targets, g_lp, g_h, False)
    if erg:
        d = d + g_h[:, None] * P * (logP + ent[:, None])
    return d


def _mut_entropy_missing_H(logP, ent, targets, g_lp, g_h, erg):
    P = np.exp(logP)
    d = _orig_logit_grad(logP, ent, targets, g_lp, g_h, False)
    if erg:
        d = d - g_h[:, None] * P * logP
    return d


def _mut_target_off_by_one(logP, ent, targets, g_lp, g_h, erg):
    return _orig_logit_grad(logP, ent, (targets + 1) % logP.shape[1], g_lp, g_h, erg)


_orig_logit_grad = ref.logit_grad


def _pins_backward():
    """Run the gradient pins; return True iff all pass."""
    try:
        test_gradients_central_differences(True)
        test_torch_float64_cross_check(True)
        test_two_point_vocab_closed_form()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", [_mut_drop_entropy_term, _mut_entropy_sign,
                                    _mut_entropy_missing_H, _mut_target_off_by_one])
def test_planted_gradient_mistakes_are_caught(monkeypatch, mutant):
    assert _pins_backward()
    monkeypatch.setattr(ref, "logit_grad", mutant)
    assert not _pins_backward()


def _mut_stats_entropy_sign(X, W, targets):
    Z, lse, logp, ent, logP = _orig_row_stats(X, W, targets)
    return Z, lse, logp, -ent, logP


def _mut_stats_lse_max_only(X, W, targets):
    Z = X @ W.T
    lse = Z.max(axis=1)
    logP = Z - lse[:, None]
    P = np.exp(logP)
    return Z, lse, logP[np.arange(Z.shape[0]), targets], -(P * logP).sum(1), logP


def _mut_stats_transposed_target(X, W, targets):
    Z, lse, logp, ent, logP = _orig_row_stats(X, W, targets)
    r = np.arange(Z.shape[0])
    return Z, lse, logP[r, (targets[::-1])], ent, logP


_orig_row_stats = ref.row_stats


def _pins_forward():
    try:
        test_uniform_logits_closed_form()
        test_two_level_logits_closed_form()
        test_torch_float64_cross_check(False)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", [_mut_stats_entropy_sign, _mut_stats_lse_max_only,
                                    _mut_stats_transposed_target])
def test_planted_forward_mistakes_are_caught(monkeypatch, mutant):
    assert _pins_forward()
    monkeypatch.setattr(ref, "row_stats", mutant)
    assert not _pins_forward()


def test_planted_mask_mistake_is_caught(monkeypatch):
    """A backward that ignores the mask for dW must fail the mask pin."""
    def bad_backward(X, W, targets, keep_mask, g_logp, g_entropy, erg):
        dX, _ = _orig_backward(X, W, targets, keep_mask, g_logp, g_entropy, erg)
        _, dW_all = _orig_backward(X, W, targets, None, g_logp, g_entropy, erg)
        return dX, dW_all
    _orig_backward = ref.backward_f64
    test_mask_semantics_equal_dense_on_kept_rows()
    monkeypatch.setattr(oracle, "backward_f64", bad_backward)
    with pytest.raises(AssertionError):
        test_mask_semantics_equal_dense_on_kept_rows()


# --------------------------------------------------------------------------
# vocabulary shards: the per-range statistics and their combination must give
# exactly the whole-vocabulary result of the direct definition above
# --------------------------------------------------------------------------

def _shard_problem(seed=21, N=40, H=24, V=53):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    t = rng.integers(0, V, N)
    keep = (rng.random(N) < 0.7).astype(np.uint8)
    g_lp = rng.standard_normal(N)
    g_h = rng.standard_normal(N)
    return X, W, t, keep, g_lp, g_h


# uneven ranges, listed out of vocabulary order, one of a single row
_CUTS = [(30, 53), (0, 17), (17, 18), (18, 30)]


def test_single_shard_statistics_are_the_definition():
    X, W, t, keep, _, _ = _shard_problem()
    part = oracle.shard_partials_f64(X, W, t, keep, 0)
    full = oracle.forward_f64(X, W, t, keep)
    idx = full["kept_idx"]
    Z = X[idx] @ W.T
    np.testing.assert_allclose(part[idx, 0], Z.max(axis=1), rtol=0, atol=0)
    np.testing.assert_allclose(part[idx, 0] + np.log(part[idx, 1]), full["lse"][idx], rtol=1e-13)
    np.testing.assert_allclose(part[idx, 3], Z[np.arange(idx.size), t[idx]], rtol=0, atol=0)
    skipped = np.flatnonzero(keep == 0)
    assert np.all(part[skipped, 0] == -np.inf) and np.all(part[skipped, 1:3] == 0)
    assert np.all(np.isnan(part[skipped, 3]))


def test_shard_merge_equals_whole_vocabulary():
    X, W, t, keep, _, _ = _shard_problem()
    N = X.shape[0]
    parts = np.stack([oracle.shard_partials_f64(X, W[a:b], t, keep, a) for a, b in _CUTS])
    got = oracle.merge_shard_partials(parts, keep, N)
    full = oracle.forward_f64(X, W, t, keep)
    for k in ("logp", "entropy", "lse"):
        np.testing.assert_allclose(got[k], full[k], rtol=1e-12, atol=1e-12, err_msg=k)
    # exactly one range holds each kept target
    idx = full["kept_idx"]
    assert np.all((~np.isnan(parts[:, idx, 3])).sum(axis=0) == 1)


def test_shard_merge_target_outside_every_range_is_nan():
    X, W, t, keep, _, _ = _shard_problem()
    N = X.shape[0]
    parts = np.stack([oracle.shard_partials_f64(X, W[a:b], t, keep, a) for a, b in _CUTS[:2]])
    got = oracle.merge_shard_partials(parts, keep, N)
    idx = oracle.compact(keep, N)
    covered = ((t[idx] >= 30) & (t[idx] < 53)) | (t[idx] < 17)
    assert np.all(np.isnan(got["logp"][idx[~covered]]))
    assert np.all(np.isfinite(got["logp"][idx[covered]]))


@pytest.mark.parametrize("erg", [False, True])
def test_shard_backward_sums_to_whole_vocabulary(erg):
    X, W, t, keep, g_lp, g_h = _shard_problem(seed=22)
    N = X.shape[0]
    full = oracle.forward_f64(X, W, t, keep)
    dX_ref, dW_ref = oracle.backward_f64(X, W, t, keep, g_lp, g_h, erg)
    dX = np.zeros_like(dX_ref)
    for a, b in _CUTS:
        dXs, dWs = oracle.backward_shard_f64(X, W[a:b], t, keep, a, full["lse"], full["entropy"],
                                             g_lp, g_h, erg)
        dX += dXs
        np.testing.assert_allclose(dWs, dW_ref[a:b], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dX, dX_ref, rtol=1e-11, atol=1e-12)


def _merge_without_shift_correction(parts, keep_mask, N):
    """A plausible mistake: b combined without the (m_p - M) s_p term."""
    parts = np.asarray(parts, dtype=np.float64)
    idx = oracle.compact(keep_mask, N)
    out = dict(logp=np.zeros(N), entropy=np.zeros(N), lse=np.zeros(N))
    for i in idx:
        M = parts[:, i, 0].max()
        a = np.exp(parts[:, i, 0] - M)
        s = (a * parts[:, i, 1]).sum()
        b = (a * parts[:, i, 2]).sum()
        out["lse"][i] = M + math.log(s)
        out["entropy"][i] = math.log(s) - b / s
    return out


def test_planted_shard_merge_mistake_is_caught():
    X, W, t, keep, _, _ = _shard_problem()
    N = X.shape[0]
    parts = np.stack([oracle.shard_partials_f64(X, W[a:b], t, keep, a) for a, b in _CUTS])
    bad = _merge_without_shift_correction(parts, keep, N)
    full = oracle.forward_f64(X, W, t, keep)
    idx = full["kept_idx"]
    assert np.abs(bad["entropy"][idx] - full["entropy"][idx]).max() > 1e-3
