"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default token chunk, persistent grids over the whole batch).

Rows are independent in the forward and in dX, so a seeded sample of kept rows
is checked against the oracle row by row; dW is checked by a second GPU call
whose keep mask selects exactly the sampled rows, which the oracle can compute.
Properties that hold at any size (kept positions, +0.0 at skipped rows, the
log-prob / entropy bounds) are checked over every row.
"""

import gc
import math

import numpy as np
import pytest
import torch

import lm_head_log_amd as lmh
import oracle
import workloads as wl
from tests.gpu_helpers import (TOL_ENT, TOL_GRAD_REL, TOL_LOGP, assert_pos_zero, rel_fro,
                               run, say)

pytestmark = pytest.mark.gpu

SAMPLE = 512


def _full_check(w, sample_seed, backward=True, blocksparse=False, token_chunk=0):
    g = run(w, backward=backward, token_chunk=token_chunk)
    if blocksparse:
        _blocksparse_check(w, g)
    kept = w.kept_rows()
    np.testing.assert_array_equal(g["kept_idx"], kept)
    assert g["status"] == 0
    skipped = np.setdiff1d(np.arange(w.N), kept)
    assert_pos_zero(g["logp"][skipped], "logp skipped")
    assert_pos_zero(g["entropy"][skipped], "entropy skipped")
    # bounds over every kept row: logp <= 0, 0 <= entropy <= ln V
    assert np.all(g["logp"][kept] <= 1e-5)
    assert np.all(g["entropy"][kept] >= -1e-5)
    assert np.all(g["entropy"][kept] <= math.log(w.V) + 1e-5)
    if backward:
        assert_pos_zero(g["dX"][skipped], "dX skipped")
    rows = wl.sample_rows(kept, SAMPLE, sample_seed)
    W64 = oracle.bf16_to_f64(w.weight)
    ref = oracle.rows_fwd_bwd(w.hidden, w.weight, w.targets, rows, w.g_logp, w.g_entropy,
                              w.entropy_requires_grad, W64=W64, want_dw=backward)
    e_lp = np.abs(g["logp"][rows] - ref["logp"]).max()
    e_h = np.abs(g["entropy"][rows] - ref["entropy"]).max()
    say(f"{w.name}: logp err {e_lp:.3e} entropy err {e_h:.3e}")
    assert e_lp <= TOL_LOGP and e_h <= TOL_ENT
    if backward:
        ex = rel_fro(g["dX"][rows], ref["dX"])
        say(f"{w.name}: dX rel err {ex:.3e}")
        assert ex <= TOL_GRAD_REL
        # the dW of this very launch (every kept row, this token chunk): its
        # column sums vanish, since each dZ row sums to zero, up to the bf16
        # rounding of dZ
        colsum = float(np.abs(g["dW"].sum(axis=0, dtype=np.float64)).max())
        nrm = float(np.linalg.norm(g["dW"]))
        say(f"{w.name}: main-call dW column sums {colsum:.3e} vs norm {nrm:.3e}")
        assert colsum <= 1e-2 * nrm
        del g
        gc.collect()
        # dW against the oracle: a second call whose mask keeps exactly the
        # sampled rows; with an explicit token chunk it runs 256-row chunks,
        # so its dW is added over chunks as the main call's is
        g2 = run(w, keep=wl.row_mask(w.N, rows), token_chunk=256 if token_chunk else 0)
        ew = rel_fro(g2["dW"], ref["dW"])
        # the same rows give the same dX whether or not other rows are kept
        ex2 = rel_fro(g2["dX"][rows], ref["dX"])
        say(f"{w.name}: dW rel err {ew:.3e} (sampled-rows call), dX {ex2:.3e}")
        assert ew <= TOL_GRAD_REL and ex2 <= TOL_GRAD_REL
        # column sums of dW vanish (each dZ row sums to zero), up to bf16 dZ rounding
        colsum = np.abs(g2["dW"].astype(np.float64).sum(axis=0)).max()
        assert colsum <= 1e-2 * np.linalg.norm(g2["dW"])
    torch.cuda.empty_cache()


@pytest.mark.parametrize("frac,chunk", [(1.0, 0), (0.23, 0), (1.0, 8192)])
def test_dense_rl_full_size(frac, chunk):
    # chunk 8192: the pages' default token chunk, two chunks with dW added in
    # order (the main call); its sampled-rows dW call runs two 256-row chunks
    say(f"case: dense_rl N16384 H4096 V131072 keep {frac} token chunk {chunk or 'default'}")
    _full_check(wl.dense_rl(frac), 2, token_chunk=chunk)


@pytest.mark.parametrize("chunk", [0, 8192])
def test_full_k_weight_gradient(chunk):
    """dW over K = 16384 kept rows, the bench batch's row count, checked whole
    against the oracle: every row kept (H 256, V 4096), in one chunk (the
    benchmark's launch) and in two chunks of 8192 (the pages' token chunk,
    prime-rl PR #3326 Overview), whose dW the second chunk adds to. SkyRL PR
    #2374 "Test coverage" compares weight gradients with materialised-logit
    references the same way."""
    say(f"case: full-K dW N16384 H256 V4096 all kept, token chunk {chunk or 'default'}")
    w = wl.small(16384, 256, 4096, seed=81, keep_fraction=1.0)
    assert int(w.keep.sum()) == 16384
    g = run(w, token_chunk=chunk)
    assert g["status"] == 0 and g["n_kept"] == 16384
    ref = oracle.forward(w.hidden, w.weight, w.targets, w.keep)
    dX, dW = oracle.backward(w.hidden, w.weight, w.targets, w.keep, w.g_logp, w.g_entropy, True)
    e_lp = np.abs(g["logp"] - ref["logp"]).max()
    e_h = np.abs(g["entropy"] - ref["entropy"]).max()
    ex, ew = rel_fro(g["dX"], dX), rel_fro(g["dW"], dW)
    say(f"full-K chunk {chunk}: logp {e_lp:.2e} entropy {e_h:.2e} dX {ex:.2e} dW {ew:.2e}")
    assert e_lp <= TOL_LOGP and e_h <= TOL_ENT
    assert ex <= TOL_GRAD_REL and ew <= TOL_GRAD_REL


def test_largest_n_with_backward():
    """N = 2^24, the largest row count the library accepts, forward and
    backward (H 256, V 1000: four default 2^22-row chunks). At this N the
    kept rows' transposed copy has a row pitch of 2^24 elements, past the
    2^22 at which a whole-tile operand descriptor would wrap. X is drawn on
    the device (torch's seeded normal generator, bf16); W, targets and upstream
    grads come from the seeded workload generator. Checked: every row listed,
    512 sampled rows' log-prob / entropy / dX against the oracle, the dW column
    sums of the main call, and a second call that keeps only the sampled rows,
    whose dW is checked whole against the oracle and whose other rows are
    +0.0."""
    N, H, V = 1 << 24, 256, 1000
    say(f"case: largest N {N} H{H} V{V} fwd+bwd")
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(91)
    X = torch.empty(N, H, dtype=torch.bfloat16, device=dev)
    blk = 1 << 20
    for r0 in range(0, N, blk):
        X[r0:r0 + blk] = torch.randn(blk, H, generator=gen, device=dev).to(torch.bfloat16)
    src = wl.small(1, H, V, seed=92)                      # W ~ N(0, 1/sqrt(H))
    rng = np.random.Generator(np.random.PCG64(93))
    t_np = rng.integers(0, V, N, dtype=np.int32)
    glp_np = rng.standard_normal(N, dtype=np.float32)
    gh_np = rng.standard_normal(N, dtype=np.float32)
    Wt = torch.from_numpy(src.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(t_np).to(dev)
    glp = torch.from_numpy(glp_np).to(dev)
    gh = torch.from_numpy(gh_np).to(dev)
    rows = wl.sample_rows(np.arange(N), SAMPLE, 94)
    Xs = X[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    sl = np.arange(rows.size)
    ref = oracle.rows_fwd_bwd(Xs, src.weight, t_np[rows], sl, glp_np[rows], gh_np[rows], True,
                              want_dw=True)

    logp, ent, saved = lmh.lmhead_fwd(X, Wt, t, None, True, True)
    gX, gW = lmh.lmhead_bwd(X, Wt, t, saved, glp, gh, True)
    torch.cuda.synchronize()
    assert lmh.lmhead_check_status(saved) == 0
    assert lmh.lmhead_read_n_kept(saved) == N
    kept = saved[1024:1024 + 4 * N].view(torch.int32)
    assert bool((kept == torch.arange(N, device=dev, dtype=torch.int32)).all())
    r_t = torch.from_numpy(rows).to(dev)
    e_lp = np.abs(logp[r_t].cpu().numpy() - ref["logp"]).max()
    e_h = np.abs(ent[r_t].cpu().numpy() - ref["entropy"]).max()
    ex = rel_fro(gX[r_t].cpu().numpy(), ref["dX"])
    dw_main = gW.cpu().numpy()
    colsum = float(np.abs(dw_main.sum(axis=0, dtype=np.float64)).max())
    say(f"largest N: logp {e_lp:.2e} entropy {e_h:.2e} dX {ex:.2e} dW colsum {colsum:.2e} "
        f"norm {np.linalg.norm(dw_main):.3e}")
    assert e_lp <= TOL_LOGP and e_h <= TOL_ENT and ex <= TOL_GRAD_REL
    assert colsum <= 1e-2 * np.linalg.norm(dw_main)
    del logp, ent, saved, gX, gW, kept
    torch.cuda.empty_cache()

    mask = torch.zeros(N, dtype=torch.uint8, device=dev)
    mask[r_t] = 1
    logp, ent, saved = lmh.lmhead_fwd(X, Wt, t, mask, True, True)
    gX, gW = lmh.lmhead_bwd(X, Wt, t, saved, glp, gh, True)
    torch.cuda.synchronize()
    assert lmh.lmhead_check_status(saved) == 0 and lmh.lmhead_read_n_kept(saved) == rows.size
    ew = rel_fro(gW.cpu().numpy(), ref["dW"])
    ex2 = rel_fro(gX[r_t].cpu().numpy(), ref["dX"])
    skip = mask == 0
    nz_lp = int((logp.view(torch.int32)[skip] != 0).sum())
    nz_x = 0
    for r0 in range(0, N, blk):
        rows_nz = (gX[r0:r0 + blk].view(torch.int32) != 0).any(dim=1)
        nz_x += int((rows_nz & skip[r0:r0 + blk]).sum())
    say(f"largest N, sampled rows kept: dW {ew:.2e} dX {ex2:.2e}; nonzero skipped rows: "
        f"logp {nz_lp} dX {nz_x}")
    assert ew <= TOL_GRAD_REL and ex2 <= TOL_GRAD_REL
    assert nz_lp == 0 and nz_x == 0
    del X, logp, ent, saved, gX, gW, mask
    torch.cuda.empty_cache()


def test_packed_grpo_full_size():
    say("case: packed_grpo packed GRPO N16384 H4096 V151936 (metric-only entropy)")
    _full_check(wl.packed_grpo(), 3)


def test_fp32_stress_full_size():
    say("case: fp32_stress fp32 stress N16384 H2560 V151936")
    _full_check(wl.fp32_stress(), 4)


def _blocksparse_check(w, g):
    """The block-sparse forward on the same batch: it runs every row of each
    256-row tile with a kept row (checked bit-exact), and its log-prob and
    entropy equal the compacting forward's bit for bit."""
    gb = run(w, backward=False, fwd=lmh.lmhead_fwd_blocksparse)
    tiles = np.flatnonzero(np.add.reduceat(w.keep.astype(np.int64), np.arange(0, w.N, 256)) > 0)
    listed = (tiles[:, None] * 256 + np.arange(256)[None, :]).ravel()
    listed = listed[listed < w.N].astype(np.int32)
    say(f"{w.name}: block-sparse runs {listed.size} rows for {int(w.keep.sum())} kept")
    np.testing.assert_array_equal(gb["kept_idx"], listed)
    assert gb["status"] == 0
    np.testing.assert_array_equal(gb["logp"].view(np.uint32), g["logp"].view(np.uint32))
    np.testing.assert_array_equal(gb["entropy"].view(np.uint32), g["entropy"].view(np.uint32))
    del gb
    gc.collect()


def test_scoring_forward_full_size():
    say("case: scoring scoring N262144 H5120 V152064 forward only, compacting and block-sparse")
    _full_check(wl.scoring(), 5, backward=False, blocksparse=True)


def test_compaction_many_chunks():
    """More than 1024 chunks of 4096 rows, so every thread of the scan owns
    several chunks: kept positions and the block-sparse listing bit-exact, a
    sample of rows against the oracle, +0.0 at skipped rows."""
    N, H, V = (1024 + 7) * 4096 + 123, 64, 300
    say(f"case: compaction over {N} rows ({(N + 4095) // 4096} chunks)")
    w = wl.small(N, H, V, seed=61, keep_fraction=0.4)
    w.keep[:300000] = 0            # whole 256-row tiles with no kept row
    w.keep[-5000:] = 0
    g = run(w, backward=False)
    kept = w.kept_rows()
    np.testing.assert_array_equal(g["kept_idx"], kept)
    assert g["n_kept"] == kept.size and g["status"] == 0
    skipped = np.setdiff1d(np.arange(N), kept)
    assert_pos_zero(g["logp"][skipped], "logp skipped")
    rows = wl.sample_rows(kept, 256, 62)
    ref = oracle.rows_fwd_bwd(w.hidden, w.weight, w.targets, rows, w.g_logp, w.g_entropy,
                              False, want_dw=False)
    assert np.abs(g["logp"][rows] - ref["logp"]).max() <= TOL_LOGP
    assert np.abs(g["entropy"][rows] - ref["entropy"]).max() <= TOL_ENT
    _blocksparse_check(w, g)


def test_full_size_runs_are_bitwise_reproducible():
    """Two runs at the bench shape, keep 0.64 (tile queues with stealing hand
    tiles to different CUs each run, and the dX tail is split): every output
    bit-identical."""
    say("case: dense_rl keep 0.64, two runs, bitwise")
    w = wl.dense_rl(0.64)
    a = run(w)
    b = run(w)
    for k in ("logp", "entropy", "dX", "dW"):
        np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32), err_msg=k)
