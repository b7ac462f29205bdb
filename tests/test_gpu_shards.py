"""GPU parity of the vocabulary-shard entry points (lmhead_fwd_partial,
lmhead_merge_partials, lmhead_bwd_partial) against the CPU float64 oracle's
shard statistics, their combination and the shard backward, on ragged,
uneven shards listed out of vocabulary order.

Bars: as for the whole op (log-prob / entropy 2e-3 absolute; summed dX and
each shard's dW within 1e-2 relative Frobenius error; skipped rows +0.0);
per-shard statistics: max logit and target logit 2e-3 absolute, sum-exp and
its first moment 1e-3 relative.
"""

import numpy as np
import pytest
import torch

import lm_head_log_amd as lmh
import oracle
import workloads as wl
from tests.gpu_helpers import (TOL_ENT, TOL_GRAD_REL, TOL_LOGP, assert_pos_zero, dev_tensors,
                               rel_fro, say)

pytestmark = pytest.mark.gpu


CASES = [
    # N, H, V, shards (start, end) in call order, seed
    (300, 192, 3000, [(0, 1000), (1000, 2256), (2256, 3000)], 31),
    (257, 256, 2049, [(1024, 2049), (0, 1024)], 32),
    (130, 704, 700, [(600, 700), (0, 1), (1, 600)], 33),
    # slices of at least 16384 rows: each shard backward splits its dX tail
    # (8 pieces for the 16384-row slice, 4 for the 23617-row one)
    (300, 128, 40001, [(16384, 40001), (0, 16384)], 34),
]


@pytest.mark.parametrize("N,H,V,cuts,seed", CASES)
def test_shard_forward_merge_backward(N, H, V, cuts, seed):
    say(f"case: shards N{N} H{H} V{V} cuts {cuts}")
    w = wl.small(N, H, V, seed=seed, keep_fraction=0.6)
    X, W, t, km, glp, gh = dev_tensors(w)
    Xd = oracle.bf16_to_f64(w.hidden)
    Wd = oracle.bf16_to_f64(w.weight)
    kept = oracle.compact(w.keep, N)
    skipped = np.setdiff1d(np.arange(N), kept)

    parts, saveds = [], []
    for a, b in cuts:
        part, saved = lmh.lmhead_fwd_partial(X, W[a:b].contiguous(), t, a, V, km)
        parts.append(part)
        saveds.append(saved)
    for (a, b), part in zip(cuts, parts):
        ref = oracle.shard_partials_f64(Xd, Wd[a:b], w.targets, w.keep, a)
        got = part.cpu().numpy().astype(np.float64)
        em = np.abs(got[kept, 0] - ref[kept, 0]).max()
        assert em <= TOL_LOGP, f"shard {a}:{b} max-logit err {em}"
        es = (np.abs(got[kept, 1] - ref[kept, 1]) / ref[kept, 1]).max()
        assert es <= 1e-3, f"shard {a}:{b} sum-exp rel err {es}"
        eb = (np.abs(got[kept, 2] - ref[kept, 2]) / np.maximum(np.abs(ref[kept, 2]), 1.0)).max()
        assert eb <= 1e-3, f"shard {a}:{b} first-moment rel err {eb}"
        has = ~np.isnan(ref[kept, 3])
        np.testing.assert_array_equal(~np.isnan(got[kept, 3]), has, err_msg=f"shard {a}:{b} z_t")
        if has.any():
            ez = np.abs(got[kept, 3][has] - ref[kept, 3][has]).max()
            assert ez <= TOL_LOGP, f"shard {a}:{b} target-logit err {ez}"
        assert np.all(got[skipped, 0] == -np.inf) and np.all(got[skipped, 1:3] == 0)
        assert np.all(np.isnan(got[skipped, 3]))

    saved = saveds[0]
    logp, ent = lmh.lmhead_merge_partials(torch.stack(parts), saved, True, True)
    ref = oracle.forward(w.hidden, w.weight, w.targets, w.keep)
    lp = logp.cpu().numpy()
    h = ent.cpu().numpy()
    e_lp = np.abs(lp[kept] - ref["logp"][kept]).max()
    e_h = np.abs(h[kept] - ref["entropy"][kept]).max()
    say(f"merged logp err {e_lp:.2e} entropy err {e_h:.2e}")
    assert e_lp <= TOL_LOGP and e_h <= TOL_ENT
    assert_pos_zero(lp[skipped], "merged logp skipped")
    assert_pos_zero(h[skipped], "merged entropy skipped")
    # the whole-vocabulary call on the same inputs agrees to fp32 rounding
    lp_full, h_full, _ = lmh.lmhead_fwd(X, W, t, km, True, True)
    assert np.abs(lp_full.cpu().numpy()[kept] - lp[kept]).max() <= 1e-4
    assert np.abs(h_full.cpu().numpy()[kept] - h[kept]).max() <= 1e-4

    dX_ref, dW_ref = oracle.backward(w.hidden, w.weight, w.targets, w.keep, w.g_logp,
                                     w.g_entropy, True)
    dX = np.zeros((N, H))
    for a, b in cuts:
        gX, gW = lmh.lmhead_bwd_partial(X, W[a:b].contiguous(), t, a, saved, glp, gh, True)
        gX = gX.cpu().numpy()
        assert_pos_zero(gX[skipped], f"shard {a}:{b} dX skipped rows")
        dX += gX
        ew = rel_fro(gW.cpu().numpy(), dW_ref[a:b])
        assert ew <= TOL_GRAD_REL, f"shard {a}:{b} dW rel err {ew}"
    ex = rel_fro(dX[kept], dX_ref[kept])
    say(f"summed dX rel err {ex:.2e}")
    assert ex <= TOL_GRAD_REL
    torch.cuda.synchronize()


def test_shards_without_mask_and_with_token_chunks():
    """Every row kept (no mask) and a backward in 256-row chunks."""
    N, H, V = 600, 256, 1300
    cuts = [(0, 700), (700, 1300)]
    say(f"case: shards no mask, chunked backward N{N} H{H} V{V}")
    w = wl.small(N, H, V, seed=34, keep_fraction=1.0)
    X, W, t, _, glp, gh = dev_tensors(w)
    parts, saveds = [], []
    for a, b in cuts:
        part, saved = lmh.lmhead_fwd_partial(X, W[a:b].contiguous(), t, a, V, None)
        parts.append(part)
        saveds.append(saved)
    saved = saveds[0]
    logp, ent = lmh.lmhead_merge_partials(torch.stack(parts), saved, True, True)
    ref = oracle.forward(w.hidden, w.weight, w.targets, None)
    assert np.abs(logp.cpu().numpy() - ref["logp"]).max() <= TOL_LOGP
    assert np.abs(ent.cpu().numpy() - ref["entropy"]).max() <= TOL_ENT
    dX_ref, dW_ref = oracle.backward(w.hidden, w.weight, w.targets, None, w.g_logp,
                                     w.g_entropy, True)
    dX = np.zeros((N, H))
    for a, b in cuts:
        gX, gW = lmh.lmhead_bwd_partial(X, W[a:b].contiguous(), t, a, saved, glp, gh, True, 256)
        dX += gX.cpu().numpy()
        assert rel_fro(gW.cpu().numpy(), dW_ref[a:b]) <= TOL_GRAD_REL
    assert rel_fro(dX, dX_ref) <= TOL_GRAD_REL
    torch.cuda.synchronize()


def test_single_shard_merge_matches_whole_vocabulary_call():
    N, H, V = 257, 128, 999
    say(f"case: one shard N{N} H{H} V{V}")
    w = wl.small(N, H, V, seed=35, keep_fraction=0.5)
    X, W, t, km, _, _ = dev_tensors(w)
    part, saved = lmh.lmhead_fwd_partial(X, W, t, 0, V, km)
    lp, h = lmh.lmhead_merge_partials(part[None], saved, True, False)
    lp_full, h_full, _ = lmh.lmhead_fwd(X, W, t, km, True, False)
    assert np.abs(lp.cpu().numpy() - lp_full.cpu().numpy()).max() <= 1e-5
    assert np.abs(h.cpu().numpy() - h_full.cpu().numpy()).max() <= 1e-5
    torch.cuda.synchronize()
