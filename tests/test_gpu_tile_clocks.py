"""The instrumented build (per-tile phase clocks, LMHEAD_TILE_CLOCKS) computes
the same bits as the default build and counts every tile it runs.

Both libraries are loaded in one process, and the binding's calls are routed
to the instrumented one for the second run. The instrumented library is built
on request (python -m lm_head_log_amd.tile_clocks build); without it, or when
it is older than the kernel sources, the test is skipped.
"""

import ctypes
import glob
import os

import numpy as np
import pytest

import workloads as wl
from lm_head_log_amd import _lib
from lm_head_log_amd.tile_clocks import CLOCK_LIB
from tests.gpu_helpers import run, say

pytestmark = pytest.mark.gpu

N, H, V = 700, 320, 2000  # ragged in every dimension; V < 2048, so dX runs whole tiles


def test_instrumented_build_same_bits_and_tile_counts():
    if not os.path.exists(CLOCK_LIB):
        pytest.skip("the instrumented build is not present")
    csrc = glob.glob(os.path.join(os.path.dirname(_lib.__file__), "csrc", "*"))
    if max(os.path.getmtime(f) for f in csrc) > os.path.getmtime(CLOCK_LIB):
        pytest.skip("the instrumented build is older than the kernel sources")
    w = wl.small(N, H, V, seed=81, keep_fraction=0.7)
    ref = run(w)

    clk = _lib.load(CLOCK_LIB)
    query = clk.lmhead_tile_clocks
    query.restype = ctypes.c_int
    query.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    xquery = clk.lmhead_tile_clocks_xcd
    xquery.restype = ctypes.c_int
    xquery.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    out = (ctypes.c_ulonglong * 32)()
    xout = (ctypes.c_ulonglong * 64)()
    prev = _lib._lib
    _lib._lib = clk
    try:
        assert query(out, 1) == 0 and xquery(xout, 1) == 0
        got = run(w)
        assert query(out, 1) == 0 and xquery(xout, 1) == 0
    finally:
        _lib._lib = prev

    for key in ("logp", "entropy", "dX", "dW"):
        np.testing.assert_array_equal(got[key].view(np.uint32), ref[key].view(np.uint32),
                                      err_msg=key)

    a = np.array(out, dtype=np.uint64).reshape(4, 8)
    n = int(ref["n_kept"])
    tok, voc, hid = -(-n // 256), -(-V // 256), -(-H // 256)
    # tiles per kernel: fwd and dz (vocabulary x token tiles), dX (token x
    # hidden tiles), dW (hidden x vocabulary tiles, one chunk)
    expect = [voc * tok, voc * tok, tok * hid, hid * voc]
    for k, name in enumerate(("fwd", "dz", "dx", "dw")):
        main, epi, take, tiles, cmain, cepi, wgs = (int(x) for x in a[k][:7])
        say(f"{name}: tiles {tiles} (expect {expect[k]}), workgroups {wgs}, "
            f"main {main} ticks / {cmain} cycles, epilogue {epi} ticks / {cepi} cycles")
        assert tiles == expect[k], name
        assert wgs > 0 and main > 0 and epi > 0 and cmain > 0 and cepi > 0, name
        # per XCD: earliest workgroup start and latest exit (100 MHz ticks);
        # XCDs that ran none of this kernel's workgroups keep the reset values
        x = np.array(xout, dtype=np.uint64).reshape(4, 8, 2)[k]
        ran = x[:, 1] > 0
        assert ran.any(), name
        assert (x[ran, 0] < x[ran, 1]).all(), name
        assert (x[~ran, 0] == np.iinfo(np.uint64).max).all(), name
