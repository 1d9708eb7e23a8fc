"""Fused, chunked KL distillation loss over the LM output head, for MI355X.

The loss of "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and
a Fused Chunked KL Loss" (§3 "Offline distillation", "Fused chunked KL") and its
full-vocabulary variant through a frozen teacher head (KDFlow abstract).  All
arithmetic runs in the HIP kernels of libkdloss.so; this package only allocates
outputs and workspace with torch and passes pointers.

    kl = topk_kl(H, W, topk_idx, topk_logits, mask, tau)        # autograd
    kl = full_kl(H, Ws, Ht, Wt, mask, tau)                      # autograd
    kl, lse, z = topk_kl_forward(...); dH, dW = topk_kl_backward(...)

The C-ABI mirrors (kd_topk_kl_fwd, ...) are re-exported with the header's names.
"""
from __future__ import annotations

import torch

from ._binding import (  # noqa: F401
    EXPORTS, KD_BF16, KD_DEFAULT_CHUNK_ROWS, KD_F32, KD_MAX_K, LIB_PATH, KDError, kd_full_kl_bwd, kd_full_kl_fwd,
    kd_full_kl_fwd_bwd, kd_full_kl_fwd_bwd_workspace_size, kd_full_kl_workspace_size, kd_topk_kl_bwd_ex,
    kd_topk_kl_fwd_bwd_ex, kd_topk_kl_fwd_ex, topk_opts, kd_full_kl_fwd_ex, kd_full_kl_bwd_ex, kd_full_kl_fwd_bwd_ex,
    full_opts, kd_topk_kl_bwd, kd_topk_kl_fwd, kd_topk_kl_fwd_bwd, kd_topk_kl_fwd_bwd_workspace_size,
    kd_topk_kl_workspace_size, kd_version, lib, kd_topk_kl_fwd_noalloc, KD_NOALLOC_SCRATCH_BYTES,
    profile_enable, profile_read, profile_reset,
    kd_topk_kl_shard_workspace_size, kd_topk_kl_fwd_shard, kd_topk_kl_shard_combine, kd_topk_kl_bwd_shard,
    kd_full_kl_fwd_shard, kd_full_kl_shard_combine, kd_full_kl_bwd_shard,
)

__all__ = [
    "topk_kl", "full_kl", "topk_kl_forward", "topk_kl_backward", "topk_kl_forward_backward", "full_kl_forward",
    "full_kl_backward", "full_kl_forward_backward", "kd_topk_kl_fwd", "kd_topk_kl_bwd", "kd_topk_kl_fwd_bwd",
    "kd_full_kl_fwd", "kd_full_kl_bwd", "kd_full_kl_fwd_bwd", "kd_topk_kl_workspace_size",
    "kd_topk_kl_fwd_bwd_workspace_size", "kd_full_kl_workspace_size", "kd_full_kl_fwd_bwd_workspace_size", "KDError",
    "kd_topk_kl_fwd_ex", "kd_topk_kl_bwd_ex", "kd_topk_kl_fwd_bwd_ex", "kd_topk_kl_fwd_noalloc", "topk_opts",
    "kd_full_kl_fwd_ex",
    "kd_full_kl_bwd_ex", "kd_full_kl_fwd_bwd_ex", "full_opts",
    "topk_kl_shard_forward", "topk_kl_shard_combine", "topk_kl_shard_backward", "kd_topk_kl_shard_workspace_size",
    "kd_topk_kl_fwd_shard", "kd_topk_kl_shard_combine", "kd_topk_kl_bwd_shard",
    "full_kl_shard_forward", "full_kl_shard_combine", "full_kl_shard_backward", "kd_full_kl_fwd_shard",
    "kd_full_kl_shard_combine", "kd_full_kl_bwd_shard",
]


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# Optional parts of the top-K loss, as keyword arguments of the functions below
# (kd_topk_opts of kdloss.h): tau_rows [T] float32 per-token temperature,
# teacher_lse [T] float32 teacher log-normaliser (partial-mass teacher),
# labels [T] int32 with ce_weight in [0, 1] (loss = (1 - w) KD + w CE),
# rev_weight r in [0, 1] (KD = (1 - r) KL(p || q) + r times the reverse KL on
# the cached entries; the backward then also takes the forward's z_topk).
def topk_kl_forward(H, W, topk_idx, topk_logits, mask=None, tau=1.0, want_z_topk=False, workspace=None,
                    **options):
    """Per-token loss, log-normaliser and the gathered raw logits (None unless
    want_z_topk, or rev_weight > 0, which needs them)."""
    T, d = H.shape
    V, K = W.shape[1], topk_idx.shape[1]
    kl = torch.empty(T, dtype=torch.float32, device=H.device)
    lse = torch.empty(T, dtype=torch.float32, device=H.device)
    want_z_topk = want_z_topk or bool(options.get("rev_weight"))
    z = torch.empty(T, K, dtype=torch.float32, device=H.device) if want_z_topk else None
    if workspace is None:
        workspace = _workspace(kd_topk_kl_workspace_size(T, d, V, K, H.dtype), H.device)
    kd_topk_kl_fwd_ex(H, W, topk_idx, topk_logits, mask, tau, topk_opts(**options), kl, lse, z, workspace)
    return kl, lse, z


def topk_kl_backward(H, W, topk_idx, topk_logits, mask, tau, lse, grad_kl, chunk_rows=0, workspace=None,
                     **options):
    """dH (dtype of H) and dW (float32) for the per-token upstream gradient."""
    T, d = H.shape
    V, K = W.shape[1], topk_idx.shape[1]
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_topk_kl_workspace_size(T, d, V, K, H.dtype, chunk_rows), H.device)
    kd_topk_kl_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, topk_opts(**options), lse,
                      grad_kl.float().contiguous(), dH, dW, chunk_rows, workspace)
    return dH, dW


def topk_kl_forward_backward(H, W, topk_idx, topk_logits, mask, tau, grad_kl, chunk_rows=0, want_z_topk=False,
                             workspace=None, **options):
    """kl, lse, z_topk (None unless want_z_topk or rev_weight > 0), dH and dW
    in one call, for a known grad_kl."""
    T, d = H.shape
    V, K = W.shape[1], topk_idx.shape[1]
    kl = torch.empty(T, dtype=torch.float32, device=H.device)
    lse = torch.empty(T, dtype=torch.float32, device=H.device)
    want_z_topk = want_z_topk or bool(options.get("rev_weight"))
    z = torch.empty(T, K, dtype=torch.float32, device=H.device) if want_z_topk else None
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_topk_kl_fwd_bwd_workspace_size(T, d, V, K, H.dtype, chunk_rows), H.device)
    kd_topk_kl_fwd_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, topk_opts(**options),
                          grad_kl.float().contiguous(), kl, lse, z, dH, dW, chunk_rows, workspace)
    return kl, lse, z, dH, dW


# One vocabulary shard of the top-K loss: W_shard holds columns
# [v0, v0 + W_shard.shape[1]) of the head; the caller all-gathers the ranks'
# records before the combine and sums the ranks' dH partials after the
# backward (kdloss.h, "top-K, one vocabulary shard").
def topk_kl_shard_forward(H, W_shard, v0, topk_idx, topk_logits, mask=None, tau=1.0, want_z_topk=False,
                          workspace=None, **options):
    """This shard's row records rec [T,4], teacher terms trow [T,2] and (optionally) its hits' raw logits."""
    T, d = H.shape
    V, K = W_shard.shape[1], topk_idx.shape[1]
    rec = torch.empty(T, 4, dtype=torch.float32, device=H.device)
    trow = torch.empty(T, 2, dtype=torch.float32, device=H.device)
    z = torch.empty(T, K, dtype=torch.float32, device=H.device) if want_z_topk else None
    if workspace is None:
        workspace = _workspace(kd_topk_kl_shard_workspace_size(T, d, V, v0, K, H.dtype), H.device)
    kd_topk_kl_fwd_shard(H, W_shard, v0, topk_idx, topk_logits, mask, tau, topk_opts(**options), rec, trow, z,
                         workspace)
    return rec, trow, z


def topk_kl_shard_combine(recs, trow, mask=None):
    """kl and the whole head's lse from the shards' records (a list in rank order, or one [R,T,4] tensor)."""
    rec = recs if isinstance(recs, torch.Tensor) else torch.stack(list(recs))
    T = rec.shape[1]
    kl = torch.empty(T, dtype=torch.float32, device=rec.device)
    lse = torch.empty(T, dtype=torch.float32, device=rec.device)
    kd_topk_kl_shard_combine(rec.contiguous(), trow, mask, kl, lse)
    return kl, lse


def topk_kl_shard_backward(H, W_shard, v0, topk_idx, topk_logits, mask, tau, lse, grad_kl, chunk_rows=0,
                           workspace=None, **options):
    """This shard's dH partial [T,d] float32 and its columns of dW [d,V_shard] float32."""
    T, d = H.shape
    V, K = W_shard.shape[1], topk_idx.shape[1]
    dH = torch.empty(T, d, dtype=torch.float32, device=H.device)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_topk_kl_shard_workspace_size(T, d, V, v0, K, H.dtype, chunk_rows), H.device)
    kd_topk_kl_bwd_shard(H, W_shard, v0, topk_idx, topk_logits, mask, tau, topk_opts(**options), lse,
                         grad_kl.float().contiguous(), dH, dW, chunk_rows, workspace)
    return dH, dW


# One vocabulary shard of the full-vocabulary loss: Ws_shard and Wt_shard hold
# the same columns of the two heads (kdloss.h, "full vocabulary, one
# vocabulary shard"); the caller all-gathers the records and sums dH.
def full_kl_shard_forward(H, Ws_shard, Ht, Wt_shard, mask=None, tau=1.0, workspace=None, tau_rows=None):
    """This shard's row records rec [T,8] float32."""
    T, d = H.shape
    dt, V = Ht.shape[1], Ws_shard.shape[1]
    rec = torch.empty(T, 8, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_full_kl_workspace_size(T, d, dt, V, H.dtype), H.device)
    kd_full_kl_fwd_shard(H, Ws_shard, Ht, Wt_shard, mask, tau, full_opts(tau_rows=tau_rows), rec, workspace)
    return rec


def full_kl_shard_combine(recs, mask=None, rev_weight=0.0, want_kl_rev=False):
    """kl, lse_s, lse_t (and kl_rev, or None) of the whole heads from the shards' records (a list in rank
    order, or one [R,T,8] tensor)."""
    rec = recs if isinstance(recs, torch.Tensor) else torch.stack(list(recs))
    T = rec.shape[1]
    kl, lse_s, lse_t = (torch.empty(T, dtype=torch.float32, device=rec.device) for _ in range(3))
    kl_rev = torch.empty(T, dtype=torch.float32, device=rec.device) if want_kl_rev or rev_weight else None
    kd_full_kl_shard_combine(rec.contiguous(), mask, rev_weight, kl, lse_s, lse_t, kl_rev)
    return kl, lse_s, lse_t, kl_rev


def full_kl_shard_backward(H, Ws_shard, Ht, Wt_shard, mask, tau, lse_s, lse_t, grad_kl, chunk_rows=0,
                           workspace=None, tau_rows=None, rev_weight=0.0, kl_rev=None):
    """This shard's dH partial [T,d] float32 and its columns of dWs [d,V_shard] float32."""
    T, d = H.shape
    dt, V = Ht.shape[1], Ws_shard.shape[1]
    dH = torch.empty(T, d, dtype=torch.float32, device=H.device)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_full_kl_workspace_size(T, d, dt, V, H.dtype, chunk_rows), H.device)
    kd_full_kl_bwd_shard(H, Ws_shard, Ht, Wt_shard, mask, tau, full_opts(tau_rows=tau_rows, rev_weight=rev_weight),
                         lse_s, lse_t, kl_rev, grad_kl.float().contiguous(), dH, dW, chunk_rows, workspace)
    return dH, dW


# Options of the full-vocabulary loss (kd_full_opts of kdloss.h): tau_rows
# [T] float32 per-token temperature; rev_weight r in [0, 1] mixes in the
# reverse KL, (1 - r) KL(p||q) + r KL(q||p).  With want_kl_rev the forward
# also returns KL(q||p) per row, which the backward needs when r > 0.
def full_kl_forward(H, Ws, Ht, Wt, mask=None, tau=1.0, workspace=None, tau_rows=None, rev_weight=0.0,
                    want_kl_rev=False):
    """kl, lse_s, lse_t (and kl_rev with want_kl_rev)."""
    T, d = H.shape
    dt, V = Ht.shape[1], Ws.shape[1]
    kl = torch.empty(T, dtype=torch.float32, device=H.device)
    ls = torch.empty(T, dtype=torch.float32, device=H.device)
    lt = torch.empty(T, dtype=torch.float32, device=H.device)
    kr = torch.empty(T, dtype=torch.float32, device=H.device) if want_kl_rev else None
    if workspace is None:
        workspace = _workspace(kd_full_kl_workspace_size(T, d, dt, V, H.dtype), H.device)
    kd_full_kl_fwd_ex(H, Ws, Ht, Wt, mask, tau, full_opts(tau_rows, rev_weight), kl, ls, lt, kr, workspace)
    return (kl, ls, lt, kr) if want_kl_rev else (kl, ls, lt)


def full_kl_backward(H, Ws, Ht, Wt, mask, tau, lse_s, lse_t, grad_kl, chunk_rows=0, workspace=None, tau_rows=None,
                     rev_weight=0.0, kl_rev=None):
    """dH (dtype of H) and dWs (float32)."""
    T, d = H.shape
    dt, V = Ht.shape[1], Ws.shape[1]
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_full_kl_workspace_size(T, d, dt, V, H.dtype, chunk_rows), H.device)
    kd_full_kl_bwd_ex(H, Ws, Ht, Wt, mask, tau, full_opts(tau_rows, rev_weight), lse_s, lse_t, kl_rev,
                      grad_kl.float().contiguous(), dH, dW, chunk_rows, workspace)
    return dH, dW


def full_kl_forward_backward(H, Ws, Ht, Wt, mask, tau, grad_kl, chunk_rows=0, workspace=None, tau_rows=None,
                             rev_weight=0.0, want_kl_rev=False):
    """kl, lse_s, lse_t, (kl_rev,) dH and dWs in one call, for a known grad_kl."""
    T, d = H.shape
    dt, V = Ht.shape[1], Ws.shape[1]
    kl = torch.empty(T, dtype=torch.float32, device=H.device)
    ls = torch.empty(T, dtype=torch.float32, device=H.device)
    lt = torch.empty(T, dtype=torch.float32, device=H.device)
    kr = torch.empty(T, dtype=torch.float32, device=H.device) if want_kl_rev else None
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, dtype=torch.float32, device=H.device)
    if workspace is None:
        workspace = _workspace(kd_full_kl_fwd_bwd_workspace_size(T, d, dt, V, H.dtype, chunk_rows), H.device)
    kd_full_kl_fwd_bwd_ex(H, Ws, Ht, Wt, mask, tau, full_opts(tau_rows, rev_weight), grad_kl.float().contiguous(),
                          kl, ls, lt, kr, dH, dW, chunk_rows, workspace)
    return (kl, ls, lt, kr, dH, dW) if want_kl_rev else (kl, ls, lt, dH, dW)


class _TopkKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, topk_idx, topk_logits, mask, tau, chunk_rows, options):
        kl, lse, z = topk_kl_forward(H, W, topk_idx, topk_logits, mask, tau, **options)
        ctx.save_for_backward(H, W, topk_idx, topk_logits, lse, z)
        ctx.mask, ctx.tau, ctx.chunk_rows, ctx.options = mask, tau, chunk_rows, options
        return kl

    @staticmethod
    def backward(ctx, g):
        H, W, idx, logits, lse, z = ctx.saved_tensors
        opts = dict(ctx.options, z_topk=z) if z is not None else ctx.options
        dH, dW = topk_kl_backward(H, W, idx, logits, ctx.mask, ctx.tau, lse, g, ctx.chunk_rows, **opts)
        return dH, dW.to(W.dtype), None, None, None, None, None, None


class _FullKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, Ws, Ht, Wt, mask, tau, chunk_rows, tau_rows, rev_weight):
        kl, ls, lt, kr = full_kl_forward(H, Ws, Ht, Wt, mask, tau, tau_rows=tau_rows, rev_weight=rev_weight,
                                         want_kl_rev=True)
        ctx.save_for_backward(H, Ws, Ht, Wt, ls, lt, kr)
        ctx.mask, ctx.tau, ctx.chunk_rows = mask, tau, chunk_rows
        ctx.tau_rows, ctx.rev_weight = tau_rows, rev_weight
        return kl

    @staticmethod
    def backward(ctx, g):
        H, Ws, Ht, Wt, ls, lt, kr = ctx.saved_tensors
        dH, dW = full_kl_backward(H, Ws, Ht, Wt, ctx.mask, ctx.tau, ls, lt, g, ctx.chunk_rows,
                                  tau_rows=ctx.tau_rows, rev_weight=ctx.rev_weight, kl_rev=kr)
        return dH, dW.to(Ws.dtype), None, None, None, None, None, None, None


def topk_kl(H, W, topk_idx, topk_logits, mask=None, tau=1.0, chunk_rows=0, tau_rows=None, teacher_lse=None,
            labels=None, ce_weight=0.0, rev_weight=0.0):
    """Per-token KL(p_teacher || q_student) with a top-K teacher (with the
    options: the mixed loss of kd_topk_opts); differentiable in H and W (W's
    gradient is cast to W's dtype; the float32 one is available from
    topk_kl_backward)."""
    options = dict(tau_rows=tau_rows, teacher_lse=teacher_lse, labels=labels, ce_weight=float(ce_weight),
                   rev_weight=float(rev_weight))
    return _TopkKL.apply(H, W, topk_idx, topk_logits, mask, float(tau), int(chunk_rows), options)


def full_kl(H, Ws, Ht, Wt, mask=None, tau=1.0, chunk_rows=0, tau_rows=None, rev_weight=0.0):
    """Per-token full-vocabulary KL through a frozen teacher head (with the
    options: the KL mixture of kd_full_opts); differentiable in H and Ws only."""
    return _FullKL.apply(H, Ws, Ht, Wt, mask, float(tau), int(chunk_rows), tau_rows, float(rev_weight))
