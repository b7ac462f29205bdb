"""Build liblmhead.so (HIP, gfx950) in-tree with hipcc.

    python -m lm_head_log_amd.build            # build the library
    python -m lm_head_log_amd.build --asm      # also keep the gfx950 assembly
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("lmhead.hip", "logits_rows.hip", "mfma_probe.hip")]
LIB = os.path.join(PKG, "liblmhead.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-ffp-contract=fast", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build liblmhead.so")
    return p


def build(verbose: bool = False, asm: bool = False, defines=(), out: str = LIB) -> str:
    """Compile liblmhead.so next to this file (or to `out`, with the extra
    preprocessor `defines`, e.g. an instrumented build) and return its path."""
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
           "-o", out + ".tmp", *SRCS]
    if asm:
        cmd.insert(1, "-save-temps=obj")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    errs = [l for l in res.stderr.splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
