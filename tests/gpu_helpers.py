"""Shared helpers of the GPU parity tests: move a seeded workload to the GPU,
run the library through its C ABI binding, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import lm_head_log_amd as lmh

# Tolerances stated by the op's specification: log-probs and entropies within
# 2e-3 absolute; gradients within 1e-2 relative Frobenius error.
TOL_LOGP = 2e-3
TOL_ENT = 2e-3
TOL_GRAD_REL = 1e-2

HEADER_BYTES = 1024


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensors(w, device="cuda:0", keep=None, use_mask=True):
    """bf16 / int32 / uint8 / fp32 device tensors of a workload."""
    X = torch.from_numpy(np.ascontiguousarray(w.hidden).view(np.int16)).view(torch.bfloat16).to(device)
    W = torch.from_numpy(np.ascontiguousarray(w.weight).view(np.int16)).view(torch.bfloat16).to(device)
    t = torch.from_numpy(np.ascontiguousarray(w.targets, dtype=np.int32)).to(device)
    k = w.keep if keep is None else keep
    km = torch.from_numpy(np.ascontiguousarray(k, dtype=np.uint8)).to(device) if (use_mask and k is not None) else None
    glp = torch.from_numpy(np.ascontiguousarray(w.g_logp, dtype=np.float32)).to(device)
    gh = torch.from_numpy(np.ascontiguousarray(w.g_entropy, dtype=np.float32)).to(device)
    return X, W, t, km, glp, gh


def run(w, keep=None, use_mask=True, token_chunk=0, backward=True, erg=None, ret=None,
        device="cuda:0", fwd=None):
    """Run forward (and backward) on the GPU; return numpy results. `fwd` is
    the forward call (lmhead_fwd by default)."""
    X, W, t, km, glp, gh = dev_tensors(w, device, keep, use_mask)
    erg = w.entropy_requires_grad if erg is None else erg
    ret = w.return_entropy if ret is None else ret
    logp, ent, saved = (fwd or lmh.lmhead_fwd)(X, W, t, km, ret, erg)
    out = dict(logp=logp.cpu().numpy(), entropy=None if ent is None else ent.cpu().numpy())
    n = lmh.lmhead_read_n_kept(saved)
    out["n_kept"] = n
    out["status"] = lmh.lmhead_check_status(saved)
    out["kept_idx"] = saved[HEADER_BYTES:HEADER_BYTES + 4 * n].view(torch.int32).cpu().numpy()
    if backward:
        gX, gW = lmh.lmhead_bwd(X, W, t, saved, glp, gh if erg else None, erg, token_chunk)
        torch.cuda.synchronize()
        out["dX"] = gX.cpu().numpy()
        out["dW"] = gW.cpu().numpy()
    del X, W, t, km, glp, gh, saved
    torch.cuda.synchronize()
    return out


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def assert_pos_zero(x, what):
    """Every element is +0.0 (bit pattern 0)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bad = np.count_nonzero(x.view(np.uint32))
    assert bad == 0, f"{what}: {bad} elements are not +0.0"
