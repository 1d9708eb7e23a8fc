"""ctypes binding of libkdloss (include/kdloss.h).

Argument marshalling only: every step of the loss runs in the library's HIP
kernels.  torch provides device memory and the current stream.  There is no
fallback: if libkdloss.so is missing, or a tensor is not on the GPU, the call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdloss.so")

KD_F32, KD_BF16 = 0, 1
KD_MAX_K = 8192
KD_DEFAULT_CHUNK_ROWS = 4096
STATUS = {
    0: "KD_OK", 1: "KD_ERR_INVALID_ARG", 2: "KD_ERR_UNSUPPORTED", 3: "KD_ERR_ALIGNMENT",
    4: "KD_ERR_WORKSPACE_TOO_SMALL", 5: "KD_ERR_INDEX_OUT_OF_RANGE", 6: "KD_ERR_HIP",
}

EXPORTS = (
    "kd_topk_kl_workspace_size", "kd_topk_kl_fwd", "kd_topk_kl_bwd",
    "kd_topk_kl_fwd_bwd_workspace_size", "kd_topk_kl_fwd_bwd",
    "kd_topk_kl_fwd_ex", "kd_topk_kl_bwd_ex", "kd_topk_kl_fwd_bwd_ex",
    "kd_topk_kl_shard_workspace_size", "kd_topk_kl_fwd_shard", "kd_topk_kl_shard_combine", "kd_topk_kl_bwd_shard",
    "kd_full_kl_fwd_shard", "kd_full_kl_shard_combine", "kd_full_kl_bwd_shard",
    "kd_full_kl_workspace_size", "kd_full_kl_fwd", "kd_full_kl_bwd",
    "kd_full_kl_fwd_bwd_workspace_size", "kd_full_kl_fwd_bwd",
    "kd_full_kl_fwd_ex", "kd_full_kl_bwd_ex", "kd_full_kl_fwd_bwd_ex",
    "kd_status_string", "kd_last_error", "kd_version",
    "kd_profile_enable", "kd_profile_count", "kd_profile_get", "kd_profile_reset",
)


class KdTopkOpts(ctypes.Structure):
    """kd_topk_opts of kdloss.h: device pointers (0 = NULL) and the CE weight."""
    _fields_ = [("tau_rows", ctypes.c_void_p), ("teacher_lse", ctypes.c_void_p), ("labels", ctypes.c_void_p),
                ("ce_weight", ctypes.c_float)]


class KdFullOpts(ctypes.Structure):
    """kd_full_opts of kdloss.h."""
    _fields_ = [("tau_rows", ctypes.c_void_p), ("rev_weight", ctypes.c_float)]


class KDError(RuntimeError):
    """A libkdloss call returned a status other than KD_OK."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m chunked_kl_loss_logit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, f32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    st = ctypes.c_int
    L.kd_topk_kl_workspace_size.argtypes = [i64, i64, i64, i64, st, i64, ctypes.POINTER(sz)]
    L.kd_topk_kl_fwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_bwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, i64, vp, sz, vp]
    L.kd_topk_kl_fwd_bwd_workspace_size.argtypes = [i64, i64, i64, i64, st, i64, ctypes.POINTER(sz)]
    L.kd_topk_kl_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp, i64,
                                     vp, sz, vp]
    op = ctypes.POINTER(KdTopkOpts)
    L.kd_topk_kl_fwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, op, i64, i64, i64, i64, st, vp, vp, vp, vp, sz, vp]
    L.kd_topk_kl_bwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, op, i64, i64, i64, i64, st, vp, vp, vp, vp, i64, vp, sz,
                                    vp]
    L.kd_topk_kl_fwd_bwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, op, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp,
                                        i64, vp, sz, vp]
    fo = ctypes.POINTER(KdFullOpts)
    L.kd_topk_kl_shard_workspace_size.argtypes = [i64, i64, i64, i64, i64, st, i64, ctypes.POINTER(sz)]
    L.kd_topk_kl_fwd_shard.argtypes = [vp, vp, vp, vp, vp, f32, op, i64, i64, i64, i64, i64, st, vp, vp, vp, vp, sz,
                                       vp]
    L.kd_topk_kl_shard_combine.argtypes = [vp, i64, vp, vp, i64, vp, vp, vp]
    L.kd_topk_kl_bwd_shard.argtypes = [vp, vp, vp, vp, vp, f32, op, i64, i64, i64, i64, i64, st, vp, vp, vp, vp, i64,
                                       vp, sz, vp]
    L.kd_full_kl_fwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, fo, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, sz, vp]
    L.kd_full_kl_bwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, fo, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp, i64,
                                    vp, sz, vp]
    L.kd_full_kl_fwd_bwd_ex.argtypes = [vp, vp, vp, vp, vp, f32, fo, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp,
                                        vp, i64, vp, sz, vp]
    L.kd_full_kl_fwd_shard.argtypes = [vp, vp, vp, vp, vp, f32, fo, i64, i64, i64, i64, st, vp, vp, sz, vp]
    L.kd_full_kl_shard_combine.argtypes = [vp, i64, vp, i64, f32, vp, vp, vp, vp, vp]
    L.kd_full_kl_bwd_shard.argtypes = [vp, vp, vp, vp, vp, f32, fo, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp,
                                       i64, vp, sz, vp]
    L.kd_full_kl_workspace_size.argtypes = [i64, i64, i64, i64, st, i64, ctypes.POINTER(sz)]
    L.kd_full_kl_fwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, sz, vp]
    L.kd_full_kl_bwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, i64, vp, sz,
                                 vp]
    L.kd_full_kl_fwd_bwd_workspace_size.argtypes = [i64, i64, i64, i64, st, i64, ctypes.POINTER(sz)]
    L.kd_full_kl_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp, vp, vp, i64,
                                     vp, sz, vp]
    for f in ("kd_topk_kl_workspace_size", "kd_topk_kl_fwd", "kd_topk_kl_bwd", "kd_topk_kl_fwd_bwd_workspace_size",
              "kd_topk_kl_fwd_bwd", "kd_topk_kl_fwd_ex", "kd_topk_kl_bwd_ex", "kd_topk_kl_fwd_bwd_ex",
              "kd_full_kl_workspace_size",
              "kd_full_kl_fwd", "kd_full_kl_bwd", "kd_full_kl_fwd_bwd_workspace_size", "kd_full_kl_fwd_bwd",
              "kd_full_kl_fwd_ex", "kd_full_kl_bwd_ex", "kd_full_kl_fwd_bwd_ex",
              "kd_profile_enable", "kd_profile_get", "kd_profile_reset"):
        getattr(L, f).restype = st
    L.kd_status_string.argtypes = [st]
    L.kd_status_string.restype = ctypes.c_char_p
    L.kd_last_error.argtypes = []
    L.kd_last_error.restype = ctypes.c_char_p
    L.kd_version.restype = ctypes.c_int
    L.kd_profile_enable.argtypes = [ctypes.c_int]
    L.kd_profile_count.restype = ctypes.c_int
    L.kd_profile_get.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i64),
                                 ctypes.POINTER(ctypes.c_double)]
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KDError(status, where, lib().kd_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KD_BF16
    if t == torch.float32:
        return KD_F32
    raise TypeError(f"unsupported dtype {t}; use torch.bfloat16 or torch.float32")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkdloss tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("libkdloss tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- C-ABI mirrors
def kd_topk_kl_workspace_size(T, d, V, K, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kd_topk_kl_workspace_size(T, d, V, K, _dtype_code(dtype), chunk_rows, ctypes.byref(out)),
           "kd_topk_kl_workspace_size")
    return out.value


def kd_topk_kl_fwd_bwd_workspace_size(T, d, V, K, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kd_topk_kl_fwd_bwd_workspace_size(T, d, V, K, _dtype_code(dtype), chunk_rows, ctypes.byref(out)),
           "kd_topk_kl_fwd_bwd_workspace_size")
    return out.value


def kd_full_kl_workspace_size(T, d, dt_hidden, V, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kd_full_kl_workspace_size(T, d, dt_hidden, V, _dtype_code(dtype), chunk_rows, ctypes.byref(out)),
           "kd_full_kl_workspace_size")
    return out.value


def kd_topk_kl_fwd(H, W, topk_idx, topk_logits, mask, tau, kl, lse, z_topk, workspace, stream=None):
    """Enqueue the top-K forward; outputs kl, lse (and z_topk if given) in place."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_fwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                T, d, V, K, _dtype_code(H.dtype), _ptr(kl), _ptr(lse), _ptr(z_topk),
                                _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                _stream(stream)), "kd_topk_kl_fwd")


def kd_topk_kl_bwd(H, W, topk_idx, topk_logits, mask, tau, lse, grad_kl, dH, dW, chunk_rows, workspace,
                   stream=None):
    """Enqueue the top-K backward; outputs dH and dW in place."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_bwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                T, d, V, K, _dtype_code(H.dtype), _ptr(lse), _ptr(grad_kl), _ptr(dH), _ptr(dW),
                                int(chunk_rows), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_topk_kl_bwd")


def kd_topk_kl_fwd_bwd(H, W, topk_idx, topk_logits, mask, tau, grad_kl, kl, lse, z_topk, dH, dW, chunk_rows,
                       workspace, stream=None):
    """Enqueue the top-K forward and backward in one call (no recompute)."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_fwd_bwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                    T, d, V, K, _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl), _ptr(lse),
                                    _ptr(z_topk), _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace),
                                    workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_topk_kl_fwd_bwd")


def topk_opts(tau_rows=None, teacher_lse=None, labels=None, ce_weight=0.0):
    """The kd_topk_opts struct for these device tensors (or None when no option is set).  The
    tensors must stay alive until the call that takes the struct has been enqueued."""
    if tau_rows is None and teacher_lse is None and labels is None and not ce_weight:
        return None
    for name, t, dt in (("tau_rows", tau_rows, torch.float32), ("teacher_lse", teacher_lse, torch.float32),
                        ("labels", labels, torch.int32)):
        if t is not None and t.dtype != dt:
            raise TypeError(f"{name} must be {dt}")
    return KdTopkOpts(_ptr(tau_rows), _ptr(teacher_lse), _ptr(labels), float(ce_weight))


def _opts_ref(opts):
    return None if opts is None else ctypes.byref(opts)


def kd_topk_kl_fwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, kl, lse, z_topk, workspace, stream=None):
    """kd_topk_kl_fwd with a kd_topk_opts (topk_opts(...)) or None."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_fwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                   _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype), _ptr(kl), _ptr(lse),
                                   _ptr(z_topk), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                   _stream(stream)), "kd_topk_kl_fwd_ex")


def kd_topk_kl_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, lse, grad_kl, dH, dW, chunk_rows, workspace,
                      stream=None):
    """kd_topk_kl_bwd with a kd_topk_opts (the forward call's) or None."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_bwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                   _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype), _ptr(lse), _ptr(grad_kl),
                                   _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace),
                                   workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_topk_kl_bwd_ex")


def kd_topk_kl_fwd_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, grad_kl, kl, lse, z_topk, dH, dW,
                          chunk_rows, workspace, stream=None):
    """kd_topk_kl_fwd_bwd with a kd_topk_opts or None."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_fwd_bwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask),
                                       float(tau), _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype), _ptr(grad_kl),
                                       _ptr(kl), _ptr(lse), _ptr(z_topk), _ptr(dH), _ptr(dW), int(chunk_rows),
                                       _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                       _stream(stream)), "kd_topk_kl_fwd_bwd_ex")


def kd_topk_kl_shard_workspace_size(T, d, V, v0, K, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t()
    _check(lib().kd_topk_kl_shard_workspace_size(T, d, V, v0, K, _dtype_code(dtype), int(chunk_rows),
                                                 ctypes.byref(out)), "kd_topk_kl_shard_workspace_size")
    return out.value


def kd_topk_kl_fwd_shard(H, W, v0, topk_idx, topk_logits, mask, tau, opts, rec, trow, z_topk, workspace,
                         stream=None):
    """One vocabulary shard's forward: W holds columns [v0, v0 + W.shape[1]) of the head; rec [T,4] and
    trow [T,2] float32 out."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_fwd_shard(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, V, int(v0), K, _dtype_code(H.dtype), _ptr(rec),
                                      _ptr(trow), _ptr(z_topk), _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_topk_kl_fwd_shard")


def kd_topk_kl_shard_combine(rec, trow, mask, kl, lse, stream=None):
    """rec [R,T,4] (the shards' records in rank order), trow [T,2] -> kl [T], lse [T]."""
    R, T = rec.shape[0], rec.shape[1]
    _check(lib().kd_topk_kl_shard_combine(_ptr(rec), R, _ptr(trow), _ptr(mask), T, _ptr(kl), _ptr(lse),
                                          _stream(stream)), "kd_topk_kl_shard_combine")


def kd_topk_kl_bwd_shard(H, W, v0, topk_idx, topk_logits, mask, tau, opts, lse, grad_kl, dH, dW, chunk_rows,
                         workspace, stream=None):
    """One vocabulary shard's backward with the whole head's lse: dH [T,d] float32 (a partial) and
    dW [d,V] float32 (the shard's columns)."""
    T, d = H.shape
    V = W.shape[1]
    K = topk_idx.shape[1]
    _check(lib().kd_topk_kl_bwd_shard(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, V, int(v0), K, _dtype_code(H.dtype), _ptr(lse),
                                      _ptr(grad_kl), _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_topk_kl_bwd_shard")


def kd_full_kl_fwd(H, Ws, Ht, Wt, mask, tau, kl, lse_s, lse_t, workspace, stream=None):
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_fwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                _dtype_code(H.dtype), _ptr(kl), _ptr(lse_s), _ptr(lse_t), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_full_kl_fwd")


def kd_full_kl_bwd(H, Ws, Ht, Wt, mask, tau, lse_s, lse_t, grad_kl, dH, dWs, chunk_rows, workspace, stream=None):
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_bwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t), _ptr(grad_kl), _ptr(dH),
                                _ptr(dWs), int(chunk_rows), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_full_kl_bwd")


def kd_full_kl_fwd_bwd_workspace_size(T, d, dt_hidden, V, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kd_full_kl_fwd_bwd_workspace_size(T, d, dt_hidden, V, _dtype_code(dtype), chunk_rows,
                                                   ctypes.byref(out)),
           "kd_full_kl_fwd_bwd_workspace_size")
    return out.value


def kd_full_kl_fwd_bwd(H, Ws, Ht, Wt, mask, tau, grad_kl, kl, lse_s, lse_t, dH, dWs, chunk_rows, workspace,
                       stream=None):
    """Enqueue the full-vocabulary forward and backward in one call (no recompute)."""
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_fwd_bwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                    _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl), _ptr(lse_s), _ptr(lse_t),
                                    _ptr(dH), _ptr(dWs), int(chunk_rows), _ptr(workspace),
                                    workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_full_kl_fwd_bwd")


def full_opts(tau_rows=None, rev_weight=0.0):
    """The kd_full_opts struct (or None when no option is set)."""
    if tau_rows is None and not rev_weight:
        return None
    if tau_rows is not None and tau_rows.dtype != torch.float32:
        raise TypeError("tau_rows must be torch.float32")
    return KdFullOpts(_ptr(tau_rows), float(rev_weight))


def kd_full_kl_fwd_ex(H, Ws, Ht, Wt, mask, tau, opts, kl, lse_s, lse_t, kl_rev, workspace, stream=None):
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_fwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), _opts_ref(opts),
                                   T, d, dt, V, _dtype_code(H.dtype), _ptr(kl), _ptr(lse_s), _ptr(lse_t),
                                   _ptr(kl_rev), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                   _stream(stream)), "kd_full_kl_fwd_ex")


def kd_full_kl_bwd_ex(H, Ws, Ht, Wt, mask, tau, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, chunk_rows, workspace,
                      stream=None):
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_bwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), _opts_ref(opts),
                                   T, d, dt, V, _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t), _ptr(kl_rev),
                                   _ptr(grad_kl), _ptr(dH), _ptr(dWs), int(chunk_rows), _ptr(workspace),
                                   workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_full_kl_bwd_ex")


def kd_full_kl_fwd_bwd_ex(H, Ws, Ht, Wt, mask, tau, opts, grad_kl, kl, lse_s, lse_t, kl_rev, dH, dWs, chunk_rows,
                          workspace, stream=None):
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_fwd_bwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                       _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl),
                                       _ptr(lse_s), _ptr(lse_t), _ptr(kl_rev), _ptr(dH), _ptr(dWs), int(chunk_rows),
                                       _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                       _stream(stream)), "kd_full_kl_fwd_bwd_ex")


def kd_full_kl_fwd_shard(H, Ws, Ht, Wt, mask, tau, opts, rec, workspace, stream=None):
    """One vocabulary shard's full-vocabulary forward: Ws and Wt hold the same columns of both heads;
    rec [T,8] float32 out."""
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_fwd_shard(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(rec), _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, _stream(stream)),
           "kd_full_kl_fwd_shard")


def kd_full_kl_shard_combine(rec, mask, rev_weight, kl, lse_s, lse_t, kl_rev, stream=None):
    """rec [R,T,8] (the shards' records in rank order) -> kl, lse_s, lse_t [T] and kl_rev [T] or None."""
    R, T = rec.shape[0], rec.shape[1]
    _check(lib().kd_full_kl_shard_combine(_ptr(rec), R, _ptr(mask), T, float(rev_weight), _ptr(kl), _ptr(lse_s),
                                          _ptr(lse_t), _ptr(kl_rev), _stream(stream)), "kd_full_kl_shard_combine")


def kd_full_kl_bwd_shard(H, Ws, Ht, Wt, mask, tau, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, chunk_rows,
                         workspace, stream=None):
    """One vocabulary shard's full-vocabulary backward with the whole heads' log-normalisers: dH [T,d] float32
    (a partial) and dWs [d,V] float32 (the shard's columns)."""
    T, d = H.shape
    dt = Ht.shape[1]
    V = Ws.shape[1]
    _check(lib().kd_full_kl_bwd_shard(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t),
                                      _ptr(kl_rev), _ptr(grad_kl), _ptr(dH), _ptr(dWs), int(chunk_rows),
                                      _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                      _stream(stream)), "kd_full_kl_bwd_shard")


def kd_version() -> int:
    return lib().kd_version()


# ---------------------------------------------------------------- profiling
def profile_enable(on: bool = True) -> None:
    _check(lib().kd_profile_enable(1 if on else 0), "kd_profile_enable")


def profile_reset() -> None:
    _check(lib().kd_profile_reset(), "kd_profile_reset")


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} of the events recorded so far."""
    L = lib()
    n = L.kd_profile_count()
    out = {}
    for i in range(n):
        name, launches, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(L.kd_profile_get(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms)), "kd_profile_get")
        out[name.value.decode()] = (launches.value, ms.value)
    return out
