"""GPU parity of the fused LM-head op against the CPU float64 oracle, element
by element, on seeded inputs that span several 256-wide tiles and ragged tails.

Bars: kept-row positions bit-exact; log-prob and entropy within 2e-3 absolute;
dX (kept rows) and dW within 1e-2 relative Frobenius error; skipped rows +0.0.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_helpers import (TOL_ENT, TOL_GRAD_REL, TOL_LOGP, assert_pos_zero, rel_fro,
                               run, say)

pytestmark = pytest.mark.gpu


_WORKLOAD_MASK = object()


def check_against_oracle(w, g, keep=_WORKLOAD_MASK, erg=None, backward=True, what=""):
    """keep: the mask the GPU call used (None = every row); defaults to w.keep."""
    keep = w.keep if keep is _WORKLOAD_MASK else keep
    erg = w.entropy_requires_grad if erg is None else erg
    ref = oracle.forward(w.hidden, w.weight, w.targets, keep)
    kept = ref["kept_idx"]
    np.testing.assert_array_equal(g["kept_idx"], kept, err_msg=f"{what} kept_idx")
    assert g["n_kept"] == kept.size
    skipped = np.setdiff1d(np.arange(w.N), kept)
    if kept.size:
        e_lp = np.abs(g["logp"][kept] - ref["logp"][kept]).max()
        assert e_lp <= TOL_LOGP, f"{what} logp max abs err {e_lp}"
        if g["entropy"] is not None:
            e_h = np.abs(g["entropy"][kept] - ref["entropy"][kept]).max()
            assert e_h <= TOL_ENT, f"{what} entropy max abs err {e_h}"
    assert_pos_zero(g["logp"][skipped], f"{what} logp skipped")
    if g["entropy"] is not None:
        assert_pos_zero(g["entropy"][skipped], f"{what} entropy skipped")
    if backward:
        dX, dW = oracle.backward(w.hidden, w.weight, w.targets, keep, w.g_logp, w.g_entropy, erg)
        if kept.size:
            ex = rel_fro(g["dX"][kept], dX[kept])
            assert ex <= TOL_GRAD_REL, f"{what} dX rel err {ex}"
        ew = rel_fro(g["dW"], dW)
        assert ew <= TOL_GRAD_REL, f"{what} dW rel err {ew}"
        assert_pos_zero(g["dX"][skipped], f"{what} dX skipped rows")
        return dict(dX=ex if kept.size else 0.0, dW=ew)
    return {}


def test_tiny_batch_full_parity():
    say("case: tiny_batch tiny N128 H512 V8192 fwd+bwd")
    w = wl.tiny_batch()
    g = run(w)
    assert g["status"] == 0
    errs = check_against_oracle(w, g, what="tiny_batch")
    say(f"tiny_batch grad errors {errs}")


@pytest.mark.parametrize("N,H,V,seed", [
    (300, 192, 1000, 10),     # ragged tokens, hidden not a multiple of 256, vocab tail
    (257, 64, 257, 11),       # one past a tile in N and V
    (1, 64, 1, 12),           # single row, single-word vocabulary
    (513, 320, 2049, 13),     # several tiles plus one-element tails
    (77, 128, 50000, 14),     # many vocab tiles, few rows
    (600, 256, 4096, 15),     # exact tiles in H and V
    (130, 384, 3000, 16),     # H / 32 a multiple of 12: the unshifted main loop
    (260, 704, 1500, 17),     # H / 32 = 22: shift 2, a peeled period longer than the loop's
])
def test_ragged_shapes(N, H, V, seed):
    say(f"case: ragged N{N} H{H} V{V}")
    w = wl.small(N, H, V, seed=seed, keep_fraction=0.6)
    g = run(w)
    check_against_oracle(w, g, what=f"N{N} H{H} V{V}")


@pytest.mark.parametrize("kind", ["zeros", "ones", "null", "first", "last", "alternating",
                                  "random"])
def test_compaction_edge_cases(kind):
    say(f"case: compaction {kind}")
    N, H, V = 5000, 64, 300
    w = wl.small(N, H, V, seed=21)
    keep = {
        "zeros": np.zeros(N, np.uint8),
        "ones": np.ones(N, np.uint8),
        "null": None,
        "first": np.eye(1, N, 0, dtype=np.uint8)[0],
        "last": np.eye(1, N, N - 1, dtype=np.uint8)[0],
        "alternating": (np.arange(N) % 2).astype(np.uint8),
        "random": (np.random.default_rng(5).random(N) < 0.3).astype(np.uint8) * 3,
    }[kind]
    g = run(w, keep=keep if keep is not None else np.ones(N, np.uint8),
            use_mask=keep is not None)
    check_against_oracle(w, g, keep=keep, what=kind)


def test_empty_batch():
    say("case: N=0")
    w = wl.small(0, 64, 100, seed=1)
    g = run(w)
    assert g["n_kept"] == 0 and g["logp"].size == 0
    assert g["dX"].shape == (0, 64)
    assert_pos_zero(g["dW"], "dW with no rows")


def test_token_chunk_invariance():
    say("case: token_chunk sweep N2000 H256 V3000")
    w = wl.small(2000, 256, 3000, seed=31, keep_fraction=0.8)
    outs = {}
    n_kept = int(w.keep.sum())
    for chunk in (64, 1000, 8192, n_kept):
        outs[chunk] = run(w, token_chunk=chunk)
    base = outs[8192]
    check_against_oracle(w, base, what="chunk 8192")
    for chunk, g in outs.items():
        np.testing.assert_array_equal(g["logp"], base["logp"])  # forward ignores the chunk
        assert rel_fro(g["dX"], base["dX"]) <= 1e-3, chunk
        assert rel_fro(g["dW"], base["dW"]) <= 1e-3, chunk


# dW's K is a chunk's kept-row count, which only the device has; its kernel
# enters the stage-shift instance for that count. Kept-row counts whose stage
# counts (rows / 32 rounded up: 2, 4, 6, 7, 8, 10, 12, 12, 14) reach every
# shift, odd counts included, and a two-chunk backward (256 + 161 rows).
@pytest.mark.parametrize("rows,chunk", [(33, 0), (97, 0), (161, 0), (200, 0), (225, 0),
                                        (289, 0), (353, 0), (383, 0), (417, 0), (417, 256)])
def test_dw_every_stage_shift(rows, chunk):
    N, H, V = rows + 45, 128, 600
    say(f"case: dW stage shift, {rows} kept rows of N{N} H{H} V{V}, chunk {chunk}")
    w = wl.small(N, H, V, seed=90 + rows, keep_fraction=1.0)
    keep = np.zeros(N, np.uint8)
    keep[np.random.default_rng(rows).choice(N, rows, replace=False)] = 1
    g = run(w, keep=keep, token_chunk=chunk)
    assert g["n_kept"] == rows
    check_against_oracle(w, g, keep=keep, what=f"{rows} kept rows, chunk {chunk}")


def test_metric_only_entropy_is_bitwise_the_differentiable_one():
    say("case: metric-only vs differentiable entropy")
    w = wl.small(700, 128, 5000, seed=41)
    a = run(w, erg=True)
    b = run(w, erg=False)
    np.testing.assert_array_equal(a["logp"].view(np.uint32), b["logp"].view(np.uint32))
    np.testing.assert_array_equal(a["entropy"].view(np.uint32), b["entropy"].view(np.uint32))
    check_against_oracle(w, b, erg=False, what="metric-only")


def test_logp_only_mode():
    say("case: return_entropy off")
    w = wl.small(300, 64, 700, seed=42)
    g = run(w, erg=False, ret=False)
    assert g["entropy"] is None
    check_against_oracle(w, g, erg=False, what="logp only")


def test_bitwise_determinism():
    say("case: determinism")
    w = wl.small(1500, 192, 6000, seed=51)
    a = run(w, token_chunk=512)
    b = run(w, token_chunk=512)
    for k in ("logp", "entropy", "dX", "dW"):
        np.testing.assert_array_equal(np.ascontiguousarray(a[k]).view(np.uint32),
                                      np.ascontiguousarray(b[k]).view(np.uint32), err_msg=k)


def test_out_of_range_target_is_reported():
    say("case: invalid target")
    w = wl.small(40, 64, 100, seed=61, keep_fraction=1.0)
    keep = np.ones(40, np.uint8)
    keep[3] = 0
    w.targets[3] = -100       # skipped row: never read
    g = run(w, keep=keep, backward=False)
    assert g["status"] == 0
    w.targets[5] = 100        # kept row, target == V
    g = run(w, keep=keep, backward=False)
    assert g["status"] == 5
    assert math.isnan(g["logp"][5])
    w.targets[5] = 7
    check_against_oracle(w, run(w, keep=keep), keep=keep, what="after fix")


def test_uniform_logits_closed_form_on_gpu():
    """W = 0: every logit is 0, so logp = -ln V and entropy = ln V exactly up
    to float32 rounding; dX = 0 and dW rows follow g_lp (onehot - 1/V) x."""
    say("case: uniform logits V=131072")
    V, H, N = 131072, 64, 64
    w = wl.small(N, H, V, seed=71, keep_fraction=0.5)
    w.weight[:] = 0
    g = run(w)
    k = np.flatnonzero(w.keep)
    lnV = 17 * math.log(2)
    assert np.abs(g["logp"][k] + lnV).max() < 1e-5
    assert np.abs(g["entropy"][k] - lnV).max() < 1e-5
    assert np.abs(g["dX"]).max() == 0.0
    check_against_oracle(w, g, what="uniform")


def test_peaked_logits_entropy_near_zero():
    say("case: one-hot dominant rows")
    V, H, N, a = 8192, 64, 32, 40.0
    w = wl.small(N, H, V, seed=72, keep_fraction=1.0)
    Xf = np.zeros((N, H), np.float32)
    Xf[:, 0] = 1.0
    Wf = np.zeros((V, H), np.float32)
    hot = 1234
    Wf[hot, 0] = a
    w.hidden[:] = wl.f32_to_bf16_bits(Xf)
    w.weight[:] = wl.f32_to_bf16_bits(Wf)
    w.targets[:] = hot
    w.targets[::2] = 7
    g = run(w)
    assert np.abs(g["entropy"]).max() < 1e-5
    assert np.abs(g["logp"][1::2]).max() < 1e-5
    assert np.abs(g["logp"][::2] + a).max() < 1e-4
    check_against_oracle(w, g, what="peaked", backward=False)
    # dW has two large entries, each a sum of +-g terms that may cancel, and the
    # hit rows' dZ at the target is g (1 - p) with p = 1 - 3e-14, so relative
    # Frobenius bars measure cancellation. Check instead an elementwise bound on
    # dZ: bf16 rounding (unit roundoff 2^-8) plus float32 error of
    # p = exp(z - LSE) with |z|, |LSE| ~ 40 (relative error of p at most
    # (|z| + |LSE| + 1) 2^-22), then propagate through |W| and |X|.
    X = oracle.bf16_to_f64(w.hidden)
    Wd = oracle.bf16_to_f64(w.weight)
    t64 = w.targets.astype(np.int64)
    Z, lse, _, h, logP = oracle.row_stats(X, Wd, t64)
    g_lp = w.g_logp.astype(np.float64)
    g_h = w.g_entropy.astype(np.float64)
    dZ = oracle.logit_grad(logP, h, t64, g_lp, g_h, True)
    dX_ref, dW_ref = dZ @ Wd, dZ.T @ X
    P = np.exp(logP)
    fp32 = (P * (np.abs(g_lp)[:, None] + np.abs(g_h)[:, None] * (np.abs(logP) + h[:, None] + 1))
            * (np.abs(Z) + np.abs(lse)[:, None] + 1) * 2.0 ** -22)
    bZ = 2.0 ** -8 * np.abs(dZ) + fp32
    bW = bZ.T @ np.abs(X) + 1e-6
    bX = bZ @ np.abs(Wd) + 1e-6
    assert np.all(np.abs(g["dW"] - dW_ref) <= bW)
    assert np.all(np.abs(g["dX"] - dX_ref) <= bX)


def test_autograd_wrapper_matches_the_c_calls():
    say("case: autograd wrapper")
    import lm_head_log_amd as lmh
    from tests.gpu_helpers import dev_tensors
    w = wl.small(2 * 96, 128, 3000, seed=81)
    X, W, t, km, glp, gh = dev_tensors(w)
    Xr = X.reshape(2, 96, 128).clone().requires_grad_(True)
    Wr = W.clone().requires_grad_(True)
    lp, ent = lmh.fused_logprobs(Xr, Wr, t.reshape(2, 96), km.reshape(2, 96).bool(),
                                 return_entropy=True, entropy_requires_grad=True)
    assert lp.shape == (2, 96) and lp.dtype == torch.float32
    L = (lp * glp.reshape(2, 96)).sum() + (ent * gh.reshape(2, 96)).sum()
    L.backward()
    g = run(w)
    np.testing.assert_array_equal(lp.detach().reshape(-1).cpu().numpy(), g["logp"])
    ref_dx = torch.from_numpy(g["dX"]).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(Xr.grad.reshape(-1, 128).float().cpu().numpy(), ref_dx)
    # metric-only entropy carries no gradient
    lp2, ent2 = lmh.fused_logprobs(Xr, Wr, t.reshape(2, 96), return_entropy=True)
    assert not ent2.requires_grad and lp2.requires_grad
    # the block-sparse forward through the same wrapper: same values and gradients
    Xb = X.reshape(2, 96, 128).clone().requires_grad_(True)
    lp3, ent3 = lmh.fused_logprobs(Xb, Wr, t.reshape(2, 96), km.reshape(2, 96).bool(),
                                   return_entropy=True, entropy_requires_grad=True,
                                   block_sparse=True)
    ((lp3 * glp.reshape(2, 96)).sum() + (ent3 * gh.reshape(2, 96)).sum()).backward()
    np.testing.assert_array_equal(lp3.detach().cpu().numpy(), lp.detach().cpu().numpy())
    np.testing.assert_array_equal(ent3.detach().cpu().numpy(), ent.detach().cpu().numpy())
    np.testing.assert_array_equal(Xb.grad.float().cpu().numpy(), Xr.grad.float().cpu().numpy())


@pytest.mark.parametrize("N,H,V,chunk,seed", [
    (600, 512, 16384, 0, 51),    # 6 dX tiles on a grid of 8: all split, 8 pieces each
    (700, 256, 20000, 256, 52),  # 4 pieces (8 would overrun the dZ row); 3 chunks, each split
    (300, 192, 131072, 0, 53),   # the bench vocabulary: pieces of 16384 rows, ragged H
])
def test_dx_tail_split(N, H, V, chunk, seed):
    """dX tiles past the last whole round of the grid are computed as pieces of
    the vocabulary range and summed in a fixed order: same bar against the
    oracle, and bitwise reproducible."""
    say(f"case: dX tail split N{N} H{H} V{V} chunk {chunk}")
    w = wl.small(N, H, V, seed=seed, keep_fraction=0.9)
    g = run(w, token_chunk=chunk)
    errs = check_against_oracle(w, g, what=f"dX split N{N} H{H} V{V}")
    say(f"dX split errors {errs}")
    g2 = run(w, token_chunk=chunk)
    np.testing.assert_array_equal(g2["dX"].view(np.uint32), g["dX"].view(np.uint32))
    np.testing.assert_array_equal(g2["dW"].view(np.uint32), g["dW"].view(np.uint32))


@pytest.mark.parametrize("N,H,V,seed", [
    (64, 64, 1 << 22, 71),    # the largest vocabulary the library takes (16384 vocab tiles; dX split)
    (40, 1 << 20, 300, 72),   # the largest hidden size (32768 k stages per tile)
])
def test_maximum_sizes(N, H, V, seed):
    say(f"case: maximum size N{N} H{H} V{V}")
    w = wl.small(N, H, V, seed=seed, keep_fraction=0.7)
    g = run(w)
    errs = check_against_oracle(w, g, what=f"max N{N} H{H} V{V}")
    say(f"maximum size errors {errs}")
