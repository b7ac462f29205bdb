"""Fused LM-head log-prob / entropy op for MI355X (gfx950).

Thin Python binding over liblmhead.so (C ABI in include/lmhead.h). The
functions named ``lmhead_*`` marshal torch tensors to the C calls of the same
name; every step of the computation runs in the library's HIP kernels. PyTorch
provides device memory and the current stream only.

``fused_logprobs`` wraps the two calls in a ``torch.autograd.Function`` with the
argument set of the pages' fused head: ``keep_mask`` (prime-rl PR #3326,
Overview), ``return_entropy`` / ``entropy_requires_grad`` (SkyRL PR #2374,
"How it works" and "Usage"), float32 outputs for bf16 inputs (twinkle PR #283,
section 1), and a token chunk that bounds backward memory (prime-rl PR #3326,
Overview); 0 selects the library's memory-budget default.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LMHeadError, check

__all__ = [
    "lmhead_saved_bytes", "lmhead_fwd_workspace_bytes", "lmhead_bwd_workspace_bytes",
    "lmhead_fwd", "lmhead_fwd_blocksparse", "lmhead_fwd_noalloc", "lmhead_bwd",
    "lmhead_read_n_kept", "NOALLOC_SCRATCH_BYTES",
    "lmhead_check_status",
    "lmhead_status_string", "lmhead_version", "fused_logprobs", "LMHeadError",
    "DEFAULT_TOKEN_CHUNK", "lmhead_kernel_name", "lmhead_profile_begin", "lmhead_profile_end",
    "lmhead_fwd_partial", "lmhead_merge_partials", "lmhead_bwd_partial",
    "lmhead_logits_fwd", "lmhead_logits_bwd", "lmhead_mfma_probe_workspace_bytes",
    "lmhead_mfma_probe",
]

_LOGIT_DTYPES = {torch.bfloat16: 0, torch.float32: 1}  # LMHEAD_DTYPE_BF16 / _F32

DEFAULT_TOKEN_CHUNK = 0  # library default: largest chunk whose dZ fits 8 GiB


def _L():
    return _lib.load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def lmhead_saved_bytes(N: int) -> int:
    return int(_L().lmhead_saved_bytes(N))


def lmhead_fwd_workspace_bytes(N: int, H: int, V: int) -> int:
    return int(_L().lmhead_fwd_workspace_bytes(N, H, V))


def lmhead_bwd_workspace_bytes(N: int, H: int, V: int, token_chunk: int = 0) -> int:
    return int(_L().lmhead_bwd_workspace_bytes(N, H, V, token_chunk))


def lmhead_status_string(status: int) -> str:
    return _L().lmhead_status_string(status).decode()


def lmhead_version() -> int:
    return int(_L().lmhead_version())


def lmhead_fwd(hidden, weight, targets, keep_mask=None, return_entropy=False,
               entropy_requires_grad=False, *, logp=None, entropy=None, saved=None,
               workspace=None, stream=None, _entry="lmhead_fwd"):
    """Forward. hidden bf16 [N, H], weight bf16 [V, H], targets int32 [N],
    keep_mask uint8/bool [N] or None. Returns (logp fp32 [N], entropy fp32 [N]
    or None, saved uint8 tensor). Output and scratch buffers may be passed in
    preallocated; the rest are allocated with torch."""
    _need(hidden, "hidden", torch.bfloat16)
    if hidden.dim() != 2:
        raise ValueError("hidden must be [N, H]")
    N, H = hidden.shape
    dev = hidden.device
    _need(weight, "weight", torch.bfloat16, device=dev)
    if weight.dim() != 2 or weight.shape[1] != H:
        raise ValueError("weight must be [V, H]")
    V = weight.shape[0]
    _need(targets, "targets", torch.int32, (N,), dev)
    if keep_mask is not None:
        if keep_mask.dtype == torch.bool:
            keep_mask = keep_mask.view(torch.uint8)
        _need(keep_mask, "keep_mask", torch.uint8, (N,), dev)
    if logp is None:
        logp = torch.empty(N, dtype=torch.float32, device=dev)
    _need(logp, "logp", torch.float32, (N,), dev)
    if return_entropy:
        if entropy is None:
            entropy = torch.empty(N, dtype=torch.float32, device=dev)
        _need(entropy, "entropy", torch.float32, (N,), dev)
    else:
        entropy = None
    L = _L()
    sb = int(L.lmhead_saved_bytes(N))
    if saved is None:
        saved = torch.empty(sb, dtype=torch.uint8, device=dev)
    args = [_ptr(hidden), _ptr(weight), _ptr(targets), _ptr(keep_mask), N, H, V,
            int(bool(return_entropy)), int(bool(entropy_requires_grad)), _ptr(logp),
            _ptr(entropy), _ptr(saved), saved.numel()]
    if _entry != "lmhead_fwd_noalloc":
        wb = int(L.lmhead_fwd_workspace_bytes(N, H, V))
        if workspace is None:
            workspace = torch.empty(max(wb, 1), dtype=torch.uint8, device=dev)
        args += [_ptr(workspace), workspace.numel()]
    st = getattr(L, _entry)(*args, _stream(stream, dev))
    check(_entry, st)
    return logp, entropy, saved


def lmhead_fwd_blocksparse(hidden, weight, targets, keep_mask=None, return_entropy=False,
                           entropy_requires_grad=False, *, logp=None, entropy=None, saved=None,
                           workspace=None, stream=None):
    """Block-sparse forward: as lmhead_fwd, but the rows stay in place and only
    256-row tiles with no kept row are skipped. Same outputs; the backward is
    lmhead_bwd."""
    return lmhead_fwd(hidden, weight, targets, keep_mask, return_entropy, entropy_requires_grad,
                      logp=logp, entropy=entropy, saved=saved, workspace=workspace,
                      stream=stream, _entry="lmhead_fwd_blocksparse")


def lmhead_fwd_noalloc(hidden, weight, targets, keep_mask=None, return_entropy=False,
                       entropy_requires_grad=False, *, logp=None, entropy=None, saved=None,
                       stream=None):
    """Allocation-free forward: as lmhead_fwd, with the workspace in the
    library's built-in device array (LMHEAD_NOALLOC_SCRATCH_BYTES per GPU).
    The C call allocates nothing; pass `logp`, `entropy` and `saved` to keep
    this wrapper from allocating them with torch."""
    return lmhead_fwd(hidden, weight, targets, keep_mask, return_entropy, entropy_requires_grad,
                      logp=logp, entropy=entropy, saved=saved, stream=stream,
                      _entry="lmhead_fwd_noalloc")


NOALLOC_SCRATCH_BYTES = 128 << 20  # LMHEAD_NOALLOC_SCRATCH_BYTES in include/lmhead.h


def lmhead_bwd(hidden, weight, targets, saved, grad_logp, grad_entropy=None,
               entropy_requires_grad=False, token_chunk=0, *, grad_hidden=None,
               grad_weight=None, workspace=None, stream=None):
    """Backward. Returns (grad_hidden fp32 [N, H], grad_weight fp32 [V, H])."""
    _need(hidden, "hidden", torch.bfloat16)
    N, H = hidden.shape
    dev = hidden.device
    _need(weight, "weight", torch.bfloat16, device=dev)
    V = weight.shape[0]
    _need(targets, "targets", torch.int32, (N,), dev)
    _need(saved, "saved", torch.uint8, device=dev)
    _need(grad_logp, "grad_logp", torch.float32, (N,), dev)
    if entropy_requires_grad:
        _need(grad_entropy, "grad_entropy", torch.float32, (N,), dev)
    else:
        grad_entropy = None
    if grad_hidden is None:
        grad_hidden = torch.empty(N, H, dtype=torch.float32, device=dev)
    if grad_weight is None:
        grad_weight = torch.empty(V, H, dtype=torch.float32, device=dev)
    _need(grad_hidden, "grad_hidden", torch.float32, (N, H), dev)
    _need(grad_weight, "grad_weight", torch.float32, (V, H), dev)
    L = _L()
    wb = int(L.lmhead_bwd_workspace_bytes(N, H, V, token_chunk))
    if workspace is None:
        workspace = torch.empty(max(wb, 1), dtype=torch.uint8, device=dev)
    st = L.lmhead_bwd(_ptr(hidden), _ptr(weight), _ptr(targets), N, H, V,
                      int(bool(entropy_requires_grad)), _ptr(saved), saved.numel(),
                      _ptr(grad_logp), _ptr(grad_entropy), _ptr(grad_hidden),
                      _ptr(grad_weight), int(token_chunk), _ptr(workspace), workspace.numel(),
                      _stream(stream, dev))
    check("lmhead_bwd", st)
    return grad_hidden, grad_weight


def lmhead_fwd_partial(hidden, weight_shard, targets, vocab_start, V_total, keep_mask=None, *,
                       partial=None, saved=None, workspace=None, stream=None):
    """Vocabulary-shard forward: weight_shard bf16 [V_shard, H] holds rows
    vocab_start .. vocab_start + V_shard of a V_total-row weight. Returns
    (partial fp32 [N, 4] = {m, s, b, z_t} per row, saved uint8 tensor)."""
    _need(hidden, "hidden", torch.bfloat16)
    if hidden.dim() != 2:
        raise ValueError("hidden must be [N, H]")
    N, H = hidden.shape
    dev = hidden.device
    _need(weight_shard, "weight_shard", torch.bfloat16, device=dev)
    if weight_shard.dim() != 2 or weight_shard.shape[1] != H:
        raise ValueError("weight_shard must be [V_shard, H]")
    Vs = weight_shard.shape[0]
    _need(targets, "targets", torch.int32, (N,), dev)
    if keep_mask is not None:
        if keep_mask.dtype == torch.bool:
            keep_mask = keep_mask.view(torch.uint8)
        _need(keep_mask, "keep_mask", torch.uint8, (N,), dev)
    if partial is None:
        partial = torch.empty(N, 4, dtype=torch.float32, device=dev)
    _need(partial, "partial", torch.float32, (N, 4), dev)
    L = _L()
    if saved is None:
        saved = torch.empty(int(L.lmhead_saved_bytes(N)), dtype=torch.uint8, device=dev)
    wb = int(L.lmhead_fwd_workspace_bytes(N, H, Vs))
    if workspace is None:
        workspace = torch.empty(max(wb, 1), dtype=torch.uint8, device=dev)
    st = L.lmhead_fwd_partial(_ptr(hidden), _ptr(weight_shard), _ptr(targets), _ptr(keep_mask),
                              N, H, Vs, int(vocab_start), int(V_total), _ptr(partial),
                              _ptr(saved), saved.numel(), _ptr(workspace), workspace.numel(),
                              _stream(stream, dev))
    check("lmhead_fwd_partial", st)
    return partial, saved


def lmhead_merge_partials(partials, saved, return_entropy=False, entropy_requires_grad=False, *,
                          logp=None, entropy=None, stream=None):
    """Combine the P shards' records partials fp32 [P, N, 4] into (logp fp32
    [N], entropy fp32 [N] or None); completes `saved` for lmhead_bwd_partial."""
    _need(partials, "partials", torch.float32)
    if partials.dim() != 3 or partials.shape[2] != 4:
        raise ValueError("partials must be [P, N, 4]")
    P, N = partials.shape[0], partials.shape[1]
    dev = partials.device
    _need(saved, "saved", torch.uint8, device=dev)
    if logp is None:
        logp = torch.empty(N, dtype=torch.float32, device=dev)
    _need(logp, "logp", torch.float32, (N,), dev)
    if return_entropy:
        if entropy is None:
            entropy = torch.empty(N, dtype=torch.float32, device=dev)
        _need(entropy, "entropy", torch.float32, (N,), dev)
    else:
        entropy = None
    st = _L().lmhead_merge_partials(_ptr(partials), P, N, int(bool(return_entropy)),
                                    int(bool(entropy_requires_grad)), _ptr(logp), _ptr(entropy),
                                    _ptr(saved), saved.numel(), _stream(stream, dev))
    check("lmhead_merge_partials", st)
    return logp, entropy


def lmhead_bwd_partial(hidden, weight_shard, targets, vocab_start, saved, grad_logp,
                       grad_entropy=None, entropy_requires_grad=False, token_chunk=0, *,
                       grad_hidden=None, grad_weight=None, workspace=None, stream=None):
    """Vocabulary-shard backward. Returns (grad_hidden fp32 [N, H], this shard's
    share of dX, and grad_weight fp32 [V_shard, H], the shard's rows of dW)."""
    _need(hidden, "hidden", torch.bfloat16)
    N, H = hidden.shape
    dev = hidden.device
    _need(weight_shard, "weight_shard", torch.bfloat16, device=dev)
    Vs = weight_shard.shape[0]
    _need(targets, "targets", torch.int32, (N,), dev)
    _need(saved, "saved", torch.uint8, device=dev)
    _need(grad_logp, "grad_logp", torch.float32, (N,), dev)
    if entropy_requires_grad:
        _need(grad_entropy, "grad_entropy", torch.float32, (N,), dev)
    else:
        grad_entropy = None
    if grad_hidden is None:
        grad_hidden = torch.empty(N, H, dtype=torch.float32, device=dev)
    if grad_weight is None:
        grad_weight = torch.empty(Vs, H, dtype=torch.float32, device=dev)
    _need(grad_hidden, "grad_hidden", torch.float32, (N, H), dev)
    _need(grad_weight, "grad_weight", torch.float32, (Vs, H), dev)
    L = _L()
    wb = int(L.lmhead_bwd_workspace_bytes(N, H, Vs, token_chunk))
    if workspace is None:
        workspace = torch.empty(max(wb, 1), dtype=torch.uint8, device=dev)
    st = L.lmhead_bwd_partial(_ptr(hidden), _ptr(weight_shard), _ptr(targets), N, H, Vs,
                              int(vocab_start), int(bool(entropy_requires_grad)), _ptr(saved),
                              saved.numel(), _ptr(grad_logp), _ptr(grad_entropy),
                              _ptr(grad_hidden), _ptr(grad_weight), int(token_chunk),
                              _ptr(workspace), workspace.numel(), _stream(stream, dev))
    check("lmhead_bwd_partial", st)
    return grad_hidden, grad_weight


def _logit_dtype(logits):
    if not isinstance(logits, torch.Tensor):
        raise TypeError("logits must be a torch.Tensor")
    if logits.dtype not in _LOGIT_DTYPES:
        raise TypeError(f"logits must be bf16 or fp32, got {logits.dtype}")
    _need(logits, "logits", logits.dtype)
    if logits.dim() != 2:
        raise ValueError("logits must be [N, V]")
    return _LOGIT_DTYPES[logits.dtype]


def lmhead_logits_fwd(logits, targets, keep_mask=None, return_entropy=False, *, logp=None,
                      entropy=None, saved_stats=None, stream=None):
    """Log-prob / entropy from materialised logits bf16 or fp32 [N, V].
    Returns (logp fp32 [N], entropy fp32 [N] or None, saved_stats fp32 [N, 2])."""
    dt = _logit_dtype(logits)
    N, V = logits.shape
    dev = logits.device
    _need(targets, "targets", torch.int32, (N,), dev)
    if keep_mask is not None:
        if keep_mask.dtype == torch.bool:
            keep_mask = keep_mask.view(torch.uint8)
        _need(keep_mask, "keep_mask", torch.uint8, (N,), dev)
    if logp is None:
        logp = torch.empty(N, dtype=torch.float32, device=dev)
    _need(logp, "logp", torch.float32, (N,), dev)
    if return_entropy:
        if entropy is None:
            entropy = torch.empty(N, dtype=torch.float32, device=dev)
        _need(entropy, "entropy", torch.float32, (N,), dev)
    else:
        entropy = None
    if saved_stats is None:
        saved_stats = torch.empty(N, 2, dtype=torch.float32, device=dev)
    _need(saved_stats, "saved_stats", torch.float32, (N, 2), dev)
    st = _L().lmhead_logits_fwd(_ptr(logits), dt, N, V, _ptr(targets), _ptr(keep_mask),
                                int(bool(return_entropy)), _ptr(logp), _ptr(entropy),
                                _ptr(saved_stats), _stream(stream, dev))
    check("lmhead_logits_fwd", st)
    return logp, entropy, saved_stats


def lmhead_logits_bwd(logits, targets, saved_stats, grad_logp, grad_entropy=None,
                      entropy_requires_grad=False, keep_mask=None, *, grad_logits=None,
                      stream=None):
    """dL/dlogits in the logits' dtype [N, V]."""
    dt = _logit_dtype(logits)
    N, V = logits.shape
    dev = logits.device
    _need(targets, "targets", torch.int32, (N,), dev)
    if keep_mask is not None:
        if keep_mask.dtype == torch.bool:
            keep_mask = keep_mask.view(torch.uint8)
        _need(keep_mask, "keep_mask", torch.uint8, (N,), dev)
    _need(saved_stats, "saved_stats", torch.float32, (N, 2), dev)
    _need(grad_logp, "grad_logp", torch.float32, (N,), dev)
    if entropy_requires_grad:
        _need(grad_entropy, "grad_entropy", torch.float32, (N,), dev)
    else:
        grad_entropy = None
    if grad_logits is None:
        grad_logits = torch.empty_like(logits)
    _need(grad_logits, "grad_logits", logits.dtype, (N, V), dev)
    st = _L().lmhead_logits_bwd(_ptr(logits), dt, N, V, _ptr(targets), _ptr(keep_mask),
                                _ptr(saved_stats), _ptr(grad_logp), _ptr(grad_entropy),
                                int(bool(entropy_requires_grad)), _ptr(grad_logits),
                                _stream(stream, dev))
    check("lmhead_logits_bwd", st)
    return grad_logits


def lmhead_read_n_kept(saved, stream=None) -> int:
    out = ctypes.c_int64(0)
    check("lmhead_read_n_kept",
          _L().lmhead_read_n_kept(_ptr(saved), ctypes.byref(out), _stream(stream, saved.device)))
    return int(out.value)


def lmhead_check_status(saved, stream=None) -> int:
    return int(_L().lmhead_check_status(_ptr(saved), _stream(stream, saved.device)))


def lmhead_kernel_name(kind: int):
    n = _L().lmhead_kernel_name(kind)
    return None if n is None else n.decode()


def lmhead_profile_begin() -> None:
    check("lmhead_profile_begin", _L().lmhead_profile_begin())


def lmhead_profile_end() -> dict:
    """Per-kernel {name: (total_ms, launches)} recorded since lmhead_profile_begin."""
    k = _lib.NUM_KERNELS
    ms = (ctypes.c_double * k)()
    cnt = (ctypes.c_int64 * k)()
    check("lmhead_profile_end", _L().lmhead_profile_end(ms, cnt))
    return {lmhead_kernel_name(i): (float(ms[i]), int(cnt[i])) for i in range(k)}


def lmhead_mfma_probe_workspace_bytes() -> int:
    return int(_L().lmhead_mfma_probe_workspace_bytes())


def lmhead_mfma_probe(a=None, b=None, iters=40000, *, workspace=None, stream=None,
                      device=None) -> dict:
    """Benchmark-only MFMA ceiling: the GEMM kernels' MFMA step with operands
    in registers. `a`, `b`: bf16 GPU tensors whose bits feed the operand
    fragments, or both None for zero operands. Returns
    {"ms", "tflops", "clock_ghz"}."""
    if (a is None) != (b is None):
        raise ValueError("pass both operand tensors or neither")
    for t, n in ((a, "a"), (b, "b")):
        if t is not None:
            _need(t, n, torch.bfloat16)
    dev = a.device if a is not None else torch.device(device or "cuda:0")
    if workspace is None:
        workspace = torch.empty(lmhead_mfma_probe_workspace_bytes(), dtype=torch.uint8,
                                device=dev)
    ms, fl, clk = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    check("lmhead_mfma_probe", _L().lmhead_mfma_probe(
        _ptr(a), 0 if a is None else a.numel(), _ptr(b), 0 if b is None else b.numel(), iters,
        _ptr(workspace), workspace.numel(), ctypes.byref(ms), ctypes.byref(fl),
        ctypes.byref(clk), _stream(stream, dev)))
    return {"ms": ms.value, "tflops": fl.value / (ms.value * 1e-3) / 1e12 if ms.value > 0 else 0.0,
            "clock_ghz": clk.value}


class _FusedLMHead(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, targets, keep_mask, return_entropy, entropy_requires_grad,
                token_chunk, block_sparse):
        fwd = lmhead_fwd_blocksparse if block_sparse else lmhead_fwd
        logp, ent, saved = fwd(hidden, weight, targets, keep_mask, return_entropy,
                               entropy_requires_grad)
        ctx.save_for_backward(hidden, weight, targets, saved)
        ctx.erg = bool(entropy_requires_grad)
        ctx.ret_ent = bool(return_entropy)
        ctx.token_chunk = int(token_chunk)
        if not return_entropy:
            return logp
        if not entropy_requires_grad:
            ctx.mark_non_differentiable(ent)
        return logp, ent

    @staticmethod
    def backward(ctx, g_logp, g_ent=None):
        hidden, weight, targets, saved = ctx.saved_tensors
        g_logp = g_logp.float().contiguous()
        if ctx.erg:
            g_ent = (torch.zeros_like(g_logp) if g_ent is None else g_ent.float().contiguous())
        gX, gW = lmhead_bwd(hidden, weight, targets, saved, g_logp,
                            g_ent if ctx.erg else None, ctx.erg, ctx.token_chunk)
        gX = gX.to(hidden.dtype) if ctx.needs_input_grad[0] else None
        gW = gW.to(weight.dtype) if ctx.needs_input_grad[1] else None
        return gX, gW, None, None, None, None, None, None


def fused_logprobs(hidden, weight, targets, keep_mask=None, return_entropy=False,
                   entropy_requires_grad=False, token_chunk_size=DEFAULT_TOKEN_CHUNK,
                   block_sparse=False):
    """Selected-target log-probs (and entropy) of ``hidden @ weight.T`` without
    materialising the logits. ``hidden`` may be [..., H]; outputs have the
    leading shape of ``hidden`` and dtype float32. Rows where ``keep_mask`` is
    false get 0 and no gradient. ``block_sparse`` runs the rows in place and
    skips only 256-row tiles with no kept row (lmhead_fwd_blocksparse) instead
    of compacting them; the results are the same."""
    if entropy_requires_grad and not return_entropy:
        raise ValueError("entropy_requires_grad requires return_entropy")
    lead = hidden.shape[:-1]
    h2 = hidden.reshape(-1, hidden.shape[-1]).contiguous()
    t = targets.reshape(-1).to(torch.int32).contiguous()
    km = None
    if keep_mask is not None:
        km = keep_mask.reshape(-1).to(torch.uint8).contiguous()
    out = _FusedLMHead.apply(h2, weight.contiguous(), t, km, bool(return_entropy),
                             bool(entropy_requires_grad), int(token_chunk_size),
                             bool(block_sparse))
    if return_entropy:
        lp, ent = out
        return lp.reshape(lead), ent.reshape(lead)
    return out.reshape(lead)
