"""Per-tile phase timing of the four GEMM tile kernels (an instrumented build).

    python -m lm_head_log_amd.tile_clocks build
        compiles liblmhead_clocks.so next to liblmhead.so with LMHEAD_TILE_CLOCKS
        (CPU only; run it before sending the tree to a GPU)
    python -m lm_head_log_amd.tile_clocks run [--workload dense_rl] [--keep 1.0] [--steps 3]
        runs forward + backward steps of a synthetic workload on that build and
        prints, per kernel, the time and shader cycles of a tile's main loop and
        epilogue, the time spent taking tiles, and the clock
    python -m lm_head_log_amd.tile_clocks xcd [--workload dense_rl] [--keep 1.0] [--steps 3]
        prints, per kernel and step, when each XCD's last workgroup exited,
        counted from the kernel's first workgroup start

Every workgroup reads the shader clock (s_memtime) and the 100 MHz constant
clock (s_memrealtime) when it has taken a tile, after the tile's main loop and
after its epilogue; the main loop includes the tile's set-up and prologue. The
instrumented build runs the same arithmetic as the default one; only the clock
reads and one atomic add per counter and workgroup are added.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLOCK_LIB = os.path.join(HERE, "liblmhead_clocks.so")
KERNELS = ("fwd_tiles", "dz_tiles", "dx_tiles", "dw_tiles")


def build() -> str:
    from lm_head_log_amd import build as b
    return b.build(verbose=True, defines=("LMHEAD_TILE_CLOCKS",), out=CLOCK_LIB)


def run(workload: str, keep: float, steps: int, per_xcd: bool = False) -> None:
    if not os.path.exists(CLOCK_LIB):
        raise SystemExit(f"{CLOCK_LIB} is missing: run `python -m lm_head_log_amd.tile_clocks build`")
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch
    import lm_head_log_amd as lmh
    from lm_head_log_amd import _lib
    import workloads as wl

    # the binding's calls go to the instrumented build from here on
    _lib.LIB_PATH = CLOCK_LIB
    _lib._lib = None
    lib = _lib.load()
    query = lib.lmhead_tile_clocks
    query.restype = ctypes.c_int
    query.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]

    w = wl.dense_rl(keep) if workload == "dense_rl" else wl.WORKLOADS[workload]()
    dev = torch.device("cuda:0")
    N, H, V = w.N, w.H, w.V
    X = torch.from_numpy(w.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(w.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(w.targets).to(dev)
    km = None if w.keep is None else torch.from_numpy(w.keep).to(dev)
    n_kept = int(w.keep.sum()) if w.keep is not None else N
    glp = torch.from_numpy(w.g_logp).to(dev)
    erg = w.entropy_requires_grad
    gh = torch.from_numpy(w.g_entropy).to(dev) if erg else None
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev) if w.return_entropy else None
    saved = torch.empty(lmh.lmhead_saved_bytes(N), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(lmh.lmhead_fwd_workspace_bytes(N, H, V), dtype=torch.uint8, device=dev)
    if w.backward:
        ws_b = torch.empty(lmh.lmhead_bwd_workspace_bytes(N, H, V, 0), dtype=torch.uint8,
                           device=dev)
        gX = torch.empty(N, H, dtype=torch.float32, device=dev)
        gW = torch.empty(V, H, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        lmh.lmhead_fwd(X, W, t, km, w.return_entropy, erg, logp=logp, entropy=ent, saved=saved,
                       workspace=ws_f, stream=stream)
        if w.backward:
            lmh.lmhead_bwd(X, W, t, saved, glp, gh, erg, 0, grad_hidden=gX, grad_weight=gW,
                           workspace=ws_b, stream=stream)

    out = (ctypes.c_ulonglong * 32)()
    for _ in range(2):
        step()
    if per_xcd:
        xq = lib.lmhead_tile_clocks_xcd
        xq.restype = ctypes.c_int
        xq.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
        xo = (ctypes.c_ulonglong * 64)()
        rows = {name: [] for name in KERNELS}
        for _ in range(steps):
            if xq(xo, 1) != 0:
                raise SystemExit("lmhead_tile_clocks_xcd failed")
            step()
            if xq(xo, 0) != 0:
                raise SystemExit("lmhead_tile_clocks_xcd failed")
            a = np.array(xo, dtype=np.float64).reshape(4, 8, 2)
            for k, name in enumerate(KERNELS):
                if a[k, :, 1].max() == 0:
                    continue
                t0 = a[k, :, 0].min()
                rows[name].append((a[k, :, 1] - t0) * 1e-2)  # us after the first start
        print(f"# per-XCD finish: {w.name}, {steps} steps; microseconds from the kernel's first "
              "workgroup start to each XCD's last workgroup exit (mean over steps)")
        print(f"{'kernel':10s} {'span_us':>9s} {'spread_us':>9s} {'spread_%':>8s}  per XCD 0..7")
        for name in KERNELS:
            if not rows[name]:
                continue
            f = np.array(rows[name])
            span = f.max(axis=1).mean()
            spread = (f.max(axis=1) - f.min(axis=1)).mean()
            print(f"{name:10s} {span:9.1f} {spread:9.1f} {100 * spread / span:8.2f}  " +
                  " ".join(f"{x:8.1f}" for x in f.mean(axis=0)))
        print("# spread: last XCD exit minus first XCD exit of the same launch; dx_tiles and dw_tiles")
        print("# are the two phases of the combined dX + dW launch (a dX tail split's pieces launch, which")
        print("# runs after it, counts as dx_tiles too and then stretches that row's span)")
        return
    if query(out, 1) != 0:
        raise SystemExit("lmhead_tile_clocks failed")
    for _ in range(steps):
        step()
    if query(out, 1) != 0:
        raise SystemExit("lmhead_tile_clocks failed")
    a = np.array(out, dtype=np.float64).reshape(4, 8)
    # stages per tile of each GEMM: K / 32 (fwd and dz: H; dX: V, in pieces
    # for a split tail; dW: the chunk's kept rows)
    stages = {"fwd_tiles": H // 32, "dz_tiles": H // 32, "dx_tiles": (V + 31) // 32,
              "dw_tiles": (n_kept + 31) // 32}
    print(f"# tile clocks: {w.name}, {steps} steps, per tile and wave 0 of its workgroup")
    print(f"{'kernel':10s} {'tiles/step':>10s} {'main_us':>8s} {'epi_us':>7s} {'take_us':>7s} "
          f"{'main_GHz':>8s} {'epi_GHz':>7s} {'epi_%':>6s} {'main_cyc/stage':>14s} "
          f"{'epi_cyc':>8s}")
    for k, name in enumerate(KERNELS):
        main, epi, nxt, n, cmain, cepi, wgs, _ = a[k]
        if n == 0:
            continue
        us = 1e-2  # one 100 MHz tick
        print(f"{name:10s} {n / steps:10.0f} {main / n * us:8.2f} {epi / n * us:7.2f} "
              f"{nxt / n * us:7.2f} {cmain / (main * 10):8.3f} {cepi / max(epi * 10, 1):7.3f} "
              f"{100 * epi / (main + epi + nxt):6.2f} {cmain / n / stages[name]:14.1f} "
              f"{cepi / n:8.0f}")
    print("# main: from taking a tile to the end of its main loop (set-up, prologue, stages);")
    print("# epi: the epilogue; take: taking the next tile; GHz: shader cycles / 100 MHz ticks;")
    print("# main_cyc/stage: main-loop shader cycles per K step of 32 (64 MFMAs of 16 cycles each:")
    print("# 1024 at full MFMA rate); dX stages are per unit of a split tail when there is one")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["build", "run", "xcd"])
    ap.add_argument("--workload", default="dense_rl",
                    choices=["dense_rl", "packed_grpo", "fp32_stress", "tiny"])
    ap.add_argument("--keep", type=float, default=1.0)
    ap.add_argument("--steps", type=int, default=3)
    args = ap.parse_args()
    if args.what == "build":
        print(build())
    else:
        run(args.workload, args.keep, args.steps, per_xcd=args.what == "xcd")


if __name__ == "__main__":
    main()
