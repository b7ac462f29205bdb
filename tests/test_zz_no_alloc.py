"""The allocation-free forward (lmhead_fwd_noalloc, through the C ABI) against
lmhead_fwd on the same inputs: two calls in a row, the second on a smaller
input, each bit-identical to lmhead_fwd in log-prob, entropy and saved state
(the same kernels run on the built-in workspace) and within the op's
tolerance of the oracle; the saved state drives lmhead_bwd to the same
gradients bit for bit. A shape whose workspace exceeds the built-in array is
rejected before anything runs."""

import numpy as np
import pytest
import torch

import lm_head_log_amd as lmh
import oracle
import workloads as wl
from tests.gpu_helpers import TOL_ENT, TOL_LOGP, dev_tensors, say

pytestmark = pytest.mark.gpu

HEADER_INTS = 7  # n_kept, status, N, H, V, flags, bwd_status


def _saved_fields(saved, N, n_kept):
    """The saved state's defined contents: header fields, kept rows, position
    map, LSE and entropy of the kept rows (padding excluded)."""
    a = (4 * N + 255) // 256 * 256
    b = saved.cpu().numpy()
    hdr = b[:4 * HEADER_INTS].view(np.int32)
    kept = b[1024:1024 + 4 * n_kept].view(np.int32)
    pos = b[1024 + a:1024 + a + 4 * N].view(np.int32)
    lse = b[1024 + 2 * a:1024 + 2 * a + 4 * n_kept].view(np.uint32)
    ent = b[1024 + 3 * a:1024 + 3 * a + 4 * n_kept].view(np.uint32)
    return hdr, kept, pos, lse, ent


@pytest.mark.parametrize("N,H,V,seed", [(700, 256, 3000, 51), (300, 128, 1000, 52)])
def test_noalloc_forward_matches_lmhead_fwd(N, H, V, seed):
    say(f"case: allocation-free forward N{N} H{H} V{V}")
    w = wl.small(N, H, V, seed=seed, keep_fraction=0.6)
    X, W, t, km, glp, gh = dev_tensors(w)
    lp_a, en_a, sv_a = lmh.lmhead_fwd(X, W, t, km, True, True)
    lp_b, en_b, sv_b = lmh.lmhead_fwd_noalloc(X, W, t, km, True, True)
    torch.cuda.synchronize()
    assert lmh.lmhead_check_status(sv_b) == 0
    n = lmh.lmhead_read_n_kept(sv_b)
    assert n == lmh.lmhead_read_n_kept(sv_a) == int(w.keep.sum())
    np.testing.assert_array_equal(lp_b.cpu().numpy().view(np.uint32),
                                  lp_a.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(en_b.cpu().numpy().view(np.uint32),
                                  en_a.cpu().numpy().view(np.uint32))
    for fa, fb, name in zip(_saved_fields(sv_a, N, n), _saved_fields(sv_b, N, n),
                            ("header", "kept rows", "positions", "lse", "entropy")):
        np.testing.assert_array_equal(fb, fa, err_msg=name)
    ref = oracle.forward(w.hidden, w.weight, w.targets, w.keep)
    kept = ref["kept_idx"]
    e_lp = np.abs(lp_b.cpu().numpy()[kept] - ref["logp"][kept]).max()
    e_h = np.abs(en_b.cpu().numpy()[kept] - ref["entropy"][kept]).max()
    say(f"allocation-free forward: logp {e_lp:.2e} entropy {e_h:.2e}")
    assert e_lp <= TOL_LOGP and e_h <= TOL_ENT
    gX_a, gW_a = lmh.lmhead_bwd(X, W, t, sv_a, glp, gh, True)
    gX_b, gW_b = lmh.lmhead_bwd(X, W, t, sv_b, glp, gh, True)
    torch.cuda.synchronize()
    assert lmh.lmhead_check_status(sv_b) == 0
    np.testing.assert_array_equal(gX_b.cpu().numpy().view(np.uint32),
                                  gX_a.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(gW_b.cpu().numpy().view(np.uint32),
                                  gW_a.cpu().numpy().view(np.uint32))


def test_noalloc_forward_rejects_a_workspace_beyond_the_array():
    say("case: allocation-free forward past its built-in workspace")
    N, H, V = 16384, 4096, 131072
    assert lmh.lmhead_fwd_workspace_bytes(N, H, V) > lmh.NOALLOC_SCRATCH_BYTES
    X = torch.zeros(N, H, dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros(V, H, dtype=torch.bfloat16, device="cuda:0")
    t = torch.zeros(N, dtype=torch.int32, device="cuda:0")
    with pytest.raises(lmh.LMHeadError) as e:
        lmh.lmhead_fwd_noalloc(X, W, t)
    assert e.value.status == 3
