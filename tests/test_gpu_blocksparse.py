"""GPU parity of the block-sparse forward (rows in place, 256-row tiles with
no kept row skipped; SkyRL PR #2374, "How it works") against the compacting
forward and the CPU float64 oracle.

Per row, log-prob, entropy and dX do not depend on which rows share a tile,
so they must equal the compacting path bit for bit; dW sums the same rows in
another order (zero rows between them) and agrees to rounding. The rows the
block-sparse forward runs are whole 256-row tiles of the original order that
hold a kept row: checked bit-exact against a numpy construction."""

import numpy as np
import pytest

import lm_head_log_amd as lmh
import workloads as wl
from tests.gpu_helpers import assert_pos_zero, rel_fro, run, say
from tests.test_gpu_parity import check_against_oracle

pytestmark = pytest.mark.gpu

TILE = 256


def listed_rows(keep, N):
    """Every row of each 256-row tile (of the original order) with a kept row."""
    if keep is None:
        return np.arange(N, dtype=np.int32)
    out = []
    for b0 in range(0, N, TILE):
        if np.any(keep[b0:b0 + TILE] != 0):
            out.append(np.arange(b0, min(N, b0 + TILE), dtype=np.int32))
    return np.concatenate(out) if out else np.zeros(0, np.int32)


def _masks(N):
    rng = np.random.default_rng(41)
    sparse = np.zeros(N, np.uint8)
    sparse[rng.choice(N, 6, replace=False)] = 1
    last = np.zeros(N, np.uint8)
    last[N - 1] = 1
    return {
        "spans": wl.span_keep(N, rng, lo=64, hi=700),
        "sparse": sparse,            # a few kept rows: most tiles skipped
        "last_row_only": last,       # only the ragged last tile
        "none_kept": np.zeros(N, np.uint8),
        "bernoulli": (rng.random(N) < 0.5).astype(np.uint8) * 2,
    }


@pytest.mark.parametrize("kind,N,H,V", [
    ("spans", 5000, 256, 3000), ("sparse", 5000, 256, 3000), ("last_row_only", 5000, 256, 3000),
    ("none_kept", 5000, 256, 3000), ("bernoulli", 5000, 256, 3000), ("null", 5000, 256, 3000),
    # V >= 16384: both row lists leave every dX tile in the split tail (all pieces)
    ("spans", 1100, 256, 16384),
])
def test_blocksparse_matches_compaction_and_oracle(kind, N, H, V):
    say(f"case: block-sparse N{N} H{H} V{V} mask {kind}")
    w = wl.small(N, H, V, seed=43)
    keep = None if kind == "null" else _masks(N)[kind]
    use_mask = keep is not None
    km = keep if use_mask else np.ones(N, np.uint8)
    gb = run(w, keep=km, use_mask=use_mask, fwd=lmh.lmhead_fwd_blocksparse)
    gc = run(w, keep=km, use_mask=use_mask)

    lst = listed_rows(keep, N)
    assert gb["n_kept"] == lst.size
    np.testing.assert_array_equal(gb["kept_idx"], lst)
    assert gb["status"] == 0
    # rows: bit for bit the compacting path's
    np.testing.assert_array_equal(gb["logp"].view(np.uint32), gc["logp"].view(np.uint32))
    np.testing.assert_array_equal(gb["entropy"].view(np.uint32), gc["entropy"].view(np.uint32))
    np.testing.assert_array_equal(gb["dX"].view(np.uint32), gc["dX"].view(np.uint32))
    if gc["n_kept"] == 0:
        assert_pos_zero(gb["dW"], "dW with no kept rows")
    else:
        assert rel_fro(gb["dW"], gc["dW"]) <= 1e-5
    # and the oracle, through the compacting path's kept rows
    g = dict(gb, kept_idx=gc["kept_idx"], n_kept=gc["n_kept"])
    check_against_oracle(w, g, keep=keep, what=f"block-sparse {kind}")


def test_blocksparse_reports_kept_target_range_only():
    # a target outside [0, V) at a row that is listed (its tile holds a kept
    # row) but not kept is never read, as in the compacting path
    N, H, V = 600, 64, 500
    say("case: block-sparse target range")
    w = wl.small(N, H, V, seed=44)
    keep = np.zeros(N, np.uint8)
    keep[10] = 1
    w.targets[11] = -100
    g = run(w, keep=keep, fwd=lmh.lmhead_fwd_blocksparse, backward=False)
    assert g["status"] == 0 and g["n_kept"] == TILE
    w.targets[10] = V
    g = run(w, keep=keep, fwd=lmh.lmhead_fwd_blocksparse, backward=False)
    assert g["status"] == 5
