"""The backward's check of the saved state against its own arguments.

lmhead_bwd / lmhead_bwd_partial read the state lmhead_fwd saved; the saved
header records the forward's N, H, V and flags (SkyRL PR #2374,
gemini-code-assist review: the forward's entropy_requires_grad travels with
the saved tensors). The check runs on the device, since the library does not
synchronise: a backward whose N, H or V differ from the forward's, whose
entropy-gradient flag differs, or whose state is a shard forward's that
lmhead_merge_partials never completed, computes nothing from the state. It
writes +0.0 to every element of dX and dW, and lmhead_check_status then
reports LMHEAD_ERR_INVALID_ARG (1). A later consistent backward on the same
state clears the status and matches the oracle.
"""

import numpy as np
import pytest
import torch

import lm_head_log_amd as lmh
import oracle
import workloads as wl
from tests.gpu_helpers import TOL_GRAD_REL, assert_pos_zero, dev_tensors, rel_fro, say

pytestmark = pytest.mark.gpu

N, H, V = 300, 128, 1000


def _nan_grads(n, h, v):
    gX = torch.full((n, h), float("nan"), dtype=torch.float32, device="cuda:0")
    gW = torch.full((v, h), float("nan"), dtype=torch.float32, device="cuda:0")
    return gX, gW


def _assert_rejected(saved, gX, gW, what):
    torch.cuda.synchronize()
    st = lmh.lmhead_check_status(saved)
    say(f"{what}: status {st}")
    assert st == 1, f"{what}: status {st}"
    assert_pos_zero(gX.cpu().numpy(), f"{what} dX")
    assert_pos_zero(gW.cpu().numpy(), f"{what} dW")


@pytest.fixture(scope="module")
def batch():
    w = wl.small(N, H, V, seed=41, keep_fraction=0.6)
    return w, dev_tensors(w)


def test_mismatched_hidden_size(batch):
    say("case: saved state, backward with another H")
    w, (X, W, t, km, glp, gh) = batch
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, True)
    w2 = wl.small(N, 192, V, seed=42)
    X2, W2, *_ = dev_tensors(w2)
    gX, gW = _nan_grads(N, 192, V)
    lmh.lmhead_bwd(X2, W2, t, saved, glp, gh, True, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "H 192 vs 128")


def test_mismatched_vocabulary(batch):
    say("case: saved state, backward with another V")
    w, (X, W, t, km, glp, gh) = batch
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, True)
    W2 = W[:999].contiguous()
    gX, gW = _nan_grads(N, H, 999)
    lmh.lmhead_bwd(X, W2, t, saved, glp, gh, True, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "V 999 vs 1000")


def test_mismatched_row_count(batch):
    say("case: saved state, backward with another N")
    w, (X, W, t, km, glp, gh) = batch
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, True)
    n = N - 1
    gX, gW = _nan_grads(n, H, V)
    lmh.lmhead_bwd(X[:n].contiguous(), W, t[:n].contiguous(), saved, glp[:n].contiguous(),
                   gh[:n].contiguous(), True, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "N 299 vs 300")


def test_mismatched_entropy_flag(batch):
    say("case: saved state, entropy gradient flag differs from the forward's")
    w, (X, W, t, km, glp, gh) = batch
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, True)
    gX, gW = _nan_grads(N, H, V)
    lmh.lmhead_bwd(X, W, t, saved, glp, None, False, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "entropy grad 0 after a forward with 1")
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, False)
    gX, gW = _nan_grads(N, H, V)
    lmh.lmhead_bwd(X, W, t, saved, glp, gh, True, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "entropy grad 1 after a forward with 0")


def test_unmerged_shard_state(batch):
    say("case: saved state of a shard forward that was never merged")
    w, (X, W, t, km, glp, gh) = batch
    part, saved = lmh.lmhead_fwd_partial(X, W[:600].contiguous(), t, 0, V, km)
    gX, gW = _nan_grads(N, H, 600)
    lmh.lmhead_bwd_partial(X, W[:600].contiguous(), t, 0, saved, glp, None, False,
                           grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "shard state without lmhead_merge_partials")
    # a whole-vocabulary backward on a shard forward's state is rejected too
    gX, gW = _nan_grads(N, H, V)
    lmh.lmhead_bwd(X, W, t, saved, glp, None, False, grad_hidden=gX, grad_weight=gW)
    _assert_rejected(saved, gX, gW, "whole-vocabulary backward on a shard state")


def test_consistent_backward_after_a_rejected_one(batch):
    say("case: saved state, rejected backward then a consistent one")
    w, (X, W, t, km, glp, gh) = batch
    _, _, saved = lmh.lmhead_fwd(X, W, t, km, True, True)
    gX, gW = _nan_grads(N, H, 999)
    lmh.lmhead_bwd(X, W[:999].contiguous(), t, saved, glp, gh, True, grad_hidden=gX,
                   grad_weight=gW)
    _assert_rejected(saved, gX, gW, "V 999")
    gX, gW = lmh.lmhead_bwd(X, W, t, saved, glp, gh, True)
    torch.cuda.synchronize()
    assert lmh.lmhead_check_status(saved) == 0
    dX, dW = oracle.backward(w.hidden, w.weight, w.targets, w.keep, w.g_logp, w.g_entropy, True)
    kept = w.kept_rows()
    ex = rel_fro(gX.cpu().numpy()[kept], dX[kept])
    ew = rel_fro(gW.cpu().numpy(), dW)
    say(f"after the rejected call: dX {ex:.2e} dW {ew:.2e}")
    assert ex <= TOL_GRAD_REL and ew <= TOL_GRAD_REL
    skipped = np.setdiff1d(np.arange(N), kept)
    assert_pos_zero(gX.cpu().numpy()[skipped], "dX skipped rows")
