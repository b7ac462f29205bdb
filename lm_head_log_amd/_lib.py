"""ctypes loader for liblmhead.so. No fallback: a missing library is an error."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; LMHEAD_LIB names another build of the same sources (for
# side-by-side timing of kernel variants).
LIB_PATH = os.environ.get("LMHEAD_LIB") or os.path.join(_HERE, "liblmhead.so")

# Every symbol include/lmhead.h declares, with its ctypes signature.
c_size = ctypes.c_size_t
c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p

SIGNATURES = {
    "lmhead_saved_bytes": (c_size, [c_i64]),
    "lmhead_fwd_workspace_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "lmhead_bwd_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i64]),
    "lmhead_fwd": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_int,
                           c_vp, c_vp, c_vp, c_size, c_vp, c_size, c_vp]),
    "lmhead_fwd_blocksparse": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int,
                                       c_int, c_vp, c_vp, c_vp, c_size, c_vp, c_size, c_vp]),
    "lmhead_fwd_noalloc": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_int,
                                   c_vp, c_vp, c_vp, c_size, c_vp]),
    "lmhead_bwd": (c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_size,
                           c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_size, c_vp]),
    "lmhead_fwd_partial": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                   c_vp, c_vp, c_size, c_vp, c_size, c_vp]),
    "lmhead_merge_partials": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_vp, c_vp, c_vp,
                                      c_size, c_vp]),
    "lmhead_bwd_partial": (c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_int, c_vp,
                                   c_size, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_size, c_vp]),
    "lmhead_logits_fwd": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_int, c_vp, c_vp, c_vp,
                                  c_vp]),
    "lmhead_logits_bwd": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_int,
                                  c_vp, c_vp]),
    "lmhead_read_n_kept": (c_int, [c_vp, ctypes.POINTER(c_i64), c_vp]),
    "lmhead_check_status": (c_int, [c_vp, c_vp]),
    "lmhead_status_string": (ctypes.c_char_p, [c_int]),
    "lmhead_version": (c_int, []),
    "lmhead_kernel_name": (ctypes.c_char_p, [c_int]),
    "lmhead_profile_begin": (c_int, []),
    "lmhead_profile_end": (c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
    "lmhead_mfma_probe_workspace_bytes": (c_size, []),
    "lmhead_mfma_probe": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_size,
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double), c_vp]),
}

NUM_KERNELS = 14

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load liblmhead.so (once). Raises if it is missing or lacks a symbol."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m lm_head_log_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is not exported
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class LMHeadError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().lmhead_status_string(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise LMHeadError(fn, status)
