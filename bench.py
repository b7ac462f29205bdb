#!/usr/bin/env python3
"""Benchmark of the fused LM-head op: forward + backward tokens/s and TFLOP/s
(% of the bf16 dense MFMA peak) at the dense RL shape N=16384, H=4096,
V=131072 (SkyRL PR #2374, Performance), differentiable entropy, every row kept.

One step = lmhead_fwd + lmhead_bwd over one synthetic batch whose inputs are
already resident in HBM; every buffer is preallocated. After the timed steps,
the keep-fraction sweep of the same page (same batch, nested masks) is timed
and fitted as t = t0 + f * t1. An MFMA probe (the GEMMs' MFMA step with
operands in registers) gives the rate and clock the chip holds under pure MFMA
load, with this batch's own operand bits and with zeros. Prints ONE JSON line
on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--keep 1.0]
                    [--workload dense_rl] [--token-chunk 0] [--no-cpu-baseline]
                    [--no-keep-sweep] [--no-probe] [--no-blocksparse]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
# Tile kernels and the GEMMs one step's launches of each run: dxdw_tiles runs
# dX's whole tiles and then dW in one launch, dx_tiles then only the pieces of a
# split dX tail (a part of a GEMM), dw_tiles only a dW of a batch with no rows.
KERNELS_GEMM = ("fwd_tiles", "dz_tiles", "dxdw_tiles", "dx_tiles", "dw_tiles")
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "traffic_dense_rl_N16384_H4096_V131072.json")
KERNEL_SOURCES = ("lm_head_log_amd/csrc/lmhead.hip", "lm_head_log_amd/csrc/gemm_core.h")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_workload(name: str, keep: float):
    import workloads as wl
    if name == "dense_rl":
        return wl.dense_rl(keep)
    return wl.WORKLOADS[name]()


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload_name: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    table (FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB copy), or None when the
    table is absent, covers another workload, or predates the current kernel
    sources."""
    try:
        with open(TRAFFIC_TABLE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    if tab.get("source_sha256") != kernel_source_hash() or tab.get("workload") != workload_name:
        return None
    k = tab.get("kernels", {}).get(kernel)
    return None if k is None else int(k["hbm_bytes_per_launch"])


def cpu_baseline(w, rows_n: int):
    """The oracle, as it stands, on a bounded sample of kept rows of the same
    batch (forward + backward including those rows' dW)."""
    import oracle
    import workloads as wl
    host_cpus = os.cpu_count() or 1
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in pools] or [host_cpus])
        if pools:
            blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
                                     for i in pools}))
    except Exception:
        threads = host_cpus
    rows = wl.sample_rows(w.kept_rows(), rows_n, 99)
    t0 = time.perf_counter()
    oracle.rows_fwd_bwd(w.hidden, w.weight, w.targets, rows, w.g_logp, w.g_entropy,
                        w.entropy_requires_grad, want_dw=w.backward)
    dt = time.perf_counter() - t0
    return {
        "value": round(len(rows) / dt, 3),
        "unit": "tokens/s",
        "cores": int(threads),
        "host_cpus": int(host_cpus),
        "blas": blas,
        "kind": "oracle",
        "sample": (f"{len(rows)} kept rows of the same batch, float64 numpy, "
                   f"forward{' + backward incl. dW' if w.backward else ''}, "
                   f"{dt:.1f} s including the bf16 weight decode"),
    }


# One tensor-parallel rank's share of the dense RL batch: P2's TP4 x CP2 layout
# at H=4096, V=131072, 16K tokens gives each rank 8192 tokens and 32768
# vocabulary rows.
SHARD_ROWS, SHARD_VOCAB, SHARD_RANKS = 8192, 32768, 4


def shard_leg(lmh, X, W, t, glp, gh, erg, stream, dev, steps):
    """Times lmhead_fwd_partial + lmhead_merge_partials (over SHARD_RANKS
    records, as after the all-gather) + lmhead_bwd_partial on one rank's
    share. The collectives themselves are not run (one GPU)."""
    import torch
    N, H = X.shape
    V = W.shape[0]
    Ns, Vs = min(SHARD_ROWS, N), min(SHARD_VOCAB, V)
    Xs, ts, Ws = X[:Ns].contiguous(), t[:Ns].contiguous(), W[:Vs].contiguous()
    gls = glp[:Ns].contiguous()
    ghs = gh[:Ns].contiguous() if (erg and gh is not None) else None
    parts = torch.empty(SHARD_RANKS, Ns, 4, dtype=torch.float32, device=dev)
    saved = torch.empty(lmh.lmhead_saved_bytes(Ns), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(1, lmh.lmhead_fwd_workspace_bytes(Ns, H, Vs)), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(max(1, lmh.lmhead_bwd_workspace_bytes(Ns, H, Vs, 0)), dtype=torch.uint8,
                       device=dev)
    lp = torch.empty(Ns, dtype=torch.float32, device=dev)
    en = torch.empty(Ns, dtype=torch.float32, device=dev)
    gXs = torch.empty(Ns, H, dtype=torch.float32, device=dev)
    gWs = torch.empty(Vs, H, dtype=torch.float32, device=dev)

    def one():
        # this rank's record goes to slot 0; the other ranks' slots hold records
        # of the same shape from the warm-up
        lmh.lmhead_fwd_partial(Xs, Ws, ts, 0, V, None, partial=parts[0], saved=saved,
                               workspace=ws_f, stream=stream)
        lmh.lmhead_merge_partials(parts, saved, True, erg, logp=lp, entropy=en, stream=stream)
        lmh.lmhead_bwd_partial(Xs, Ws, ts, 0, saved, gls, ghs, erg, 0, grad_hidden=gXs,
                               grad_weight=gWs, workspace=ws_b, stream=stream)

    lmh.lmhead_fwd_partial(Xs, Ws, ts, 0, V, None, partial=parts[0], saved=saved,
                           workspace=ws_f, stream=stream)
    parts[1:].copy_(parts[0].expand(SHARD_RANKS - 1, Ns, 4))
    for _ in range(2):
        one()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = 8.0 * Ns * H * Vs
    return {
        "workload": f"one tensor-parallel rank (TP4 x CP2 layout) of the dense RL batch: "
                    f"N {Ns} H {H} V_shard {Vs} of V {V}, fwd_partial + merge of "
                    f"{SHARD_RANKS} shard records + bwd_partial; collectives not run",
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(Ns / (ms * 1e-3), 1),
        "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
        "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "steps": steps,
    }


# Materialised-logits entry at the shape of twinkle PR #283's experiment
# (16384 tokens, vocabulary 151936, bf16 logits).
LOGITS_N, LOGITS_V = 16384, 151936
PEAK_HBM_GBPS = 8000.0


def logits_leg(lmh, stream, dev, steps):
    """Times lmhead_logits_fwd + lmhead_logits_bwd on synthetic bf16 logits
    already in HBM; both are HBM-bound streams (the forward reads the logits,
    the backward reads them and writes the gradient)."""
    import torch
    N, V = LOGITS_N, LOGITS_V
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    z = (torch.randn(N, V, generator=g, device=dev) * 2.0).to(torch.bfloat16)
    t = torch.randint(0, V, (N,), generator=g, device=dev, dtype=torch.int32)
    glp = torch.randn(N, generator=g, device=dev)
    gh = torch.randn(N, generator=g, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev)
    en = torch.empty(N, dtype=torch.float32, device=dev)
    st = torch.empty(N, 2, dtype=torch.float32, device=dev)
    gz = torch.empty_like(z)

    def fwd():
        lmh.lmhead_logits_fwd(z, t, None, True, logp=lp, entropy=en, saved_stats=st,
                              stream=stream)

    def bwd():
        lmh.lmhead_logits_bwd(z, t, st, glp, gh, True, None, grad_logits=gz, stream=stream)

    for _ in range(2):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fwd()
        ev[2 * i + 1].record(stream)
        bwd()
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    f = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]))
    b = float(np.median([ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps)]))
    nbytes = N * V * 2
    del z, gz
    return {
        "workload": f"materialised bf16 logits N {N} V {V}, fwd (log-prob + entropy) + bwd "
                    f"(dL/dlogits with the entropy term)",
        "fwd_ms": round(f, 4),
        "bwd_ms": round(b, 4),
        "ms_per_step": round(f + b, 4),
        "tokens_per_s": round(N / ((f + b) * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "fwd_GBps": round(nbytes / (f * 1e-3) / 1e9, 1),
            "bwd_GBps": round(2 * nbytes / (b * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "fwd_frac": round(nbytes / (f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "bwd_frac": round(2 * nbytes / (b * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "bytes": "fwd reads N*V*2; bwd reads N*V*2 and writes N*V*2 (per-row vectors "
                     "are < 0.1 %)",
        },
        "steps": steps,
    }


def blocksparse_leg(lmh, stream, dev, steps):
    """The scoring batch (N 262144, H 5120, V 152064, keep in contiguous spans
    of 64-2048 tokens), forward only: the compacting forward against the
    block-sparse one, which runs every row of each 256-row tile that holds a
    kept row in place (SkyRL PR #2374, "How it works")."""
    import torch

    import workloads as wl
    w = wl.scoring()
    N, H, V = w.N, w.H, w.V
    X = torch.from_numpy(w.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(w.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(w.targets).to(dev)
    km = torch.from_numpy(w.keep).to(dev)
    n_kept = int(w.keep.sum())
    del w
    lp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev)
    saved = torch.empty(lmh.lmhead_saved_bytes(N), dtype=torch.uint8, device=dev)
    ws = torch.empty(lmh.lmhead_fwd_workspace_bytes(N, H, V), dtype=torch.uint8, device=dev)
    out = {"workload": f"scoring N{N} H{H} V{V}, keep in spans of 64-2048 tokens, forward only",
           "n_kept": n_kept, "steps": steps,
           # every device buffer of this leg (the op allocates nothing itself)
           # against the fp32 logits a materialising forward would hold
           "device_bytes": sum(x.numel() * x.element_size()
                               for x in (X, W, t, km, lp, ent, saved, ws)),
           "fp32_logits_bytes": N * V * 4}
    for name, fn in (("compact", lmh.lmhead_fwd), ("block_sparse", lmh.lmhead_fwd_blocksparse)):
        def call():
            fn(X, W, t, km, True, False, logp=lp, entropy=ent, saved=saved, workspace=ws,
               stream=stream)
        call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        rows = lmh.lmhead_read_n_kept(saved)
        out[name] = {"ms": round(ms, 3), "rows_run": rows,
                     "tflops_over_kept_rows": round(2.0 * n_kept * H * V / (ms * 1e-3) / 1e12, 1),
                     "tflops_over_rows_run": round(2.0 * rows * H * V / (ms * 1e-3) / 1e12, 1)}
    out["block_sparse_over_compact_time"] = round(out["block_sparse"]["ms"] / out["compact"]["ms"], 4)
    return out


def probe_leg(lmh, W, X, stream, step_tflops, kernel_tflops, iters=200000):
    """The GEMM engine's MFMA step with operands in registers (no loads, LDS
    or epilogue), once with fragments of this batch's own W and X bits and
    once with zero operands: the rate and clock the chip holds under pure MFMA
    load, against which the step and its dominant kernel are also given."""
    import torch
    ws = torch.empty(lmh.lmhead_mfma_probe_workspace_bytes(), dtype=torch.uint8, device=X.device)
    # warm-up: from idle the clock takes tens of milliseconds to settle
    lmh.lmhead_mfma_probe(W, X, iters // 4, workspace=ws, stream=stream)
    data = lmh.lmhead_mfma_probe(W, X, iters, workspace=ws, stream=stream)
    zero = lmh.lmhead_mfma_probe(None, None, iters, workspace=ws, stream=stream,
                                 device=X.device)

    def rec(r):
        return {"tflops": round(r["tflops"], 1), "clock_ghz": round(r["clock_ghz"], 3),
                "ms": round(r["ms"], 3), "frac_of_bf16_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4)}

    return {
        "what": "v_mfma_f32_16x16x32_bf16, 8x8 blocks per wave, 4 waves per CU, one workgroup "
                "per CU, operands in registers (no loads, LDS, barriers or epilogue)",
        "operands_from_batch": rec(data),
        "zero_operands": rec(zero),
        "step_frac_of_batch_ceiling": round(step_tflops / data["tflops"], 4),
        "dominant_kernel_frac_of_batch_ceiling": round(kernel_tflops / data["tflops"], 4),
        "iters": iters,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_rl",
                    choices=["dense_rl", "packed_grpo", "fp32_stress", "scoring", "tiny"],
                    help="dense_rl: N 16384 H 4096 V 131072 (the metric); packed_grpo: "
                         "N 16384 H 4096 V 151936; fp32_stress: N 16384 H 2560 V 151936; "
                         "scoring: N 262144 H 5120 V 152064, forward only; tiny: N 128 H 512 V 8192")
    ap.add_argument("--keep", type=float, default=1.0)
    ap.add_argument("--token-chunk", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-keep-sweep", action="store_true")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--no-logits", action="store_true",
                    help="skip the materialised-logits entry timing")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the vocabulary-shard (one tensor-parallel rank) timing")
    ap.add_argument("--no-blocksparse", action="store_true",
                    help="skip the block-sparse vs compacting forward on the scoring batch")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the MFMA ceiling probe (operands in registers, no memory traffic)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the op runs on one GPU; --gpus {args.gpus} is not supported "
              "(the op shards by rows or vocabulary, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import lm_head_log_amd as lmh
    from lm_head_log_amd import _lib
    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    w = make_workload(args.workload, args.keep)
    log(f"workload {w.name} generated in {time.time() - t0:.1f}s")
    N, H, V = w.N, w.H, w.V
    X = torch.from_numpy(w.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(w.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(w.targets).to(dev)
    km = None if w.keep is None else torch.from_numpy(w.keep).to(dev)
    glp = torch.from_numpy(w.g_logp).to(dev)
    erg = w.entropy_requires_grad
    gh = torch.from_numpy(w.g_entropy).to(dev) if erg else None
    ret = w.return_entropy
    n_kept = int(w.keep.sum()) if w.keep is not None else N

    logp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev) if ret else None
    saved = torch.empty(lmh.lmhead_saved_bytes(N), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(1, lmh.lmhead_fwd_workspace_bytes(N, H, V)), dtype=torch.uint8,
                       device=dev)
    do_bwd = w.backward
    if do_bwd:
        ws_b = torch.empty(max(1, lmh.lmhead_bwd_workspace_bytes(N, H, V, args.token_chunk)),
                           dtype=torch.uint8, device=dev)
        gX = torch.empty(N, H, dtype=torch.float32, device=dev)
        gW = torch.empty(V, H, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd(mask):
        lmh.lmhead_fwd(X, W, t, mask, ret, erg, logp=logp, entropy=ent, saved=saved,
                       workspace=ws_f, stream=stream)

    def bwd():
        if do_bwd:
            lmh.lmhead_bwd(X, W, t, saved, glp, gh, erg, args.token_chunk, grad_hidden=gX,
                           grad_weight=gW, workspace=ws_b, stream=stream)

    def step():
        fwd(km)
        bwd()

    def timed_steps(mask, k):
        """k steps with an event after each forward and each backward."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * k + 1)]
        ev[0].record(stream)
        for i in range(k):
            fwd(mask)
            ev[2 * i + 1].record(stream)
            bwd()
            ev[2 * i + 2].record(stream)
        torch.cuda.synchronize()
        f = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(k)]
        b = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(k)]
        return ev[0].elapsed_time(ev[2 * k]), f, b

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    torch.cuda.synchronize()
    lmh.lmhead_profile_begin()
    ms_total, f_ms, b_ms = timed_steps(km, args.steps)
    prof = lmh.lmhead_profile_end()
    assert lmh.lmhead_read_n_kept(saved) == n_kept
    ms_step = ms_total / args.steps
    step_ms = [a + b for a, b in zip(f_ms, b_ms)]
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step")

    def spread(xs):
        return {"median": round(float(np.median(xs)), 4), "min": round(min(xs), 4),
                "max": round(max(xs), 4)}

    fl_gemm = 2.0 * n_kept * H * V  # one logit-sized contraction over kept rows
    n_gemm = 4 if do_bwd else 1
    flops_step = n_gemm * fl_gemm
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    kern = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
            for k, v in prof.items() if v[1] > 0}
    for k, v in kern.items():
        log(f"  kernel {k:13s} {v['ms_per_step']:9.3f} ms/step  "
            f"({v['launches_per_step']:.0f} launches)")
    pieces_ms = kern.get("dx_tiles", {}).get("ms_per_step", 0.0)

    def gemm_flops(k):
        """GEMM flops of one step's launches of tile kernel k, or None where they
        hold a part of a GEMM: with a split dX tail the combined dX + dW launch
        carries dX's whole tiles only and dx_tiles the rest."""
        if k in ("fwd_tiles", "dz_tiles", "dw_tiles"):
            return fl_gemm
        if k == "dxdw_tiles":
            return 2 * fl_gemm if pieces_ms < 0.01 * kern[k]["ms_per_step"] else None
        if k == "dx_tiles" and "dxdw_tiles" not in kern:
            return fl_gemm
        return None

    whole = [k for k in kern if k in KERNELS_GEMM and gemm_flops(k) is not None]
    dom = max(whole, key=lambda k: kern[k]["ms_per_step"])
    dom_ms = kern[dom]["ms_per_step"]
    achieved = gemm_flops(dom) / (dom_ms * 1e-3) / 1e12
    for k in whole:
        kern[k]["tflops"] = round(gemm_flops(k) / (kern[k]["ms_per_step"] * 1e-3) / 1e12, 1)
        kern[k]["gemms"] = round(gemm_flops(k) / fl_gemm)

    probe = None
    if not args.no_probe:
        probe = probe_leg(lmh, W, X, stream, tflops, achieved)
        log(f"mfma probe {probe}")

    sweep = None
    if not args.no_keep_sweep and args.workload == "dense_rl":
        import workloads as wl
        masks = wl.dense_rl_masks(wl.KEEP_SWEEP, N=N)
        fr, ms, kept = [], [], []
        for f in wl.KEEP_SWEEP:
            m_dev = torch.from_numpy(masks[f]).to(dev)
            for _ in range(2):
                fwd(m_dev)
                bwd()
            tot, _, _ = timed_steps(m_dev, args.sweep_steps)
            fr.append(f)
            kept.append(int(masks[f].sum()))
            ms.append(tot / args.sweep_steps)
            log(f"keep {f:.2f}: {ms[-1]:.3f} ms/step ({kept[-1]} kept rows)")
        kf = np.array(kept, dtype=np.float64) / N
        A = np.stack([np.ones_like(kf), kf], axis=1)
        coef, *_ = np.linalg.lstsq(A, np.array(ms), rcond=None)
        pred = A @ coef
        ss_res = float(((np.array(ms) - pred) ** 2).sum())
        ss_tot = float(((np.array(ms) - np.mean(ms)) ** 2).sum())
        sweep = {
            "keep_fraction": fr, "kept_rows": kept, "ms_per_step": [round(x, 4) for x in ms],
            "fit": "ms = t0 + t1 * kept_fraction (least squares)",
            "t0_ms": round(float(coef[0]), 4), "t1_ms": round(float(coef[1]), 4),
            "r2": round(1.0 - ss_res / ss_tot, 6) if ss_tot > 0 else None,
            "steps_each": args.sweep_steps,
        }

    shard = None
    if not args.no_shard and args.workload == "dense_rl" and do_bwd:
        shard = shard_leg(lmh, X, W, t, glp, gh, erg, stream, dev, max(args.sweep_steps, 5))
        log(f"tp shard {shard}")

    logits = None
    if not args.no_logits and args.workload == "dense_rl":
        logits = logits_leg(lmh, stream, dev, max(args.sweep_steps, 5))
        log(f"logits entry {logits}")

    bsp = None
    if not args.no_blocksparse and args.workload == "dense_rl":
        bsp = blocksparse_leg(lmh, stream, dev, 3)
        log(f"block-sparse vs compacting forward {bsp}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, args.cpu_rows)
        log(f"cpu baseline {cpu}")

    out = {
        "metric": "fused LM-head fwd+bwd tokens/s & TFLOP/s (% bf16 MFMA peak), H4096 V131072",
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name + (" fwd+bwd" if do_bwd else " fwd"),
            "N": N, "H": H, "V": V, "n_kept": n_kept,
            "keep_fraction": round(n_kept / max(N, 1), 4),
            "return_entropy": bool(ret), "entropy_requires_grad": bool(erg),
            "token_chunk": args.token_chunk or "default (dZ budget 8 GiB)",
        },
        "tflops": round(tflops, 1),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        # model FLOPs: 6 K_n H V (2 without backward), i.e. without the logit recompute
        "model_tflops": round((6 if do_bwd else 2) * n_kept * H * V / (ms_step * 1e-3) / 1e12, 1),
        "kept_tokens_per_s": round(n_kept / (ms_step * 1e-3), 1),
        "flops_per_step": flops_step,
        "step_ms": spread(step_ms),
        "fwd_ms": spread(f_ms),
        "bwd_ms": spread(b_ms) if do_bwd else None,
        "kernels": kern,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(dom, w.name),
        },
        "cpu_baseline": cpu,
        "mfma_ceiling": probe,
        "keep_sweep": sweep,
        "tp_shard": shard,
        "logits_input": logits,
        "block_sparse_scoring": bsp,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
