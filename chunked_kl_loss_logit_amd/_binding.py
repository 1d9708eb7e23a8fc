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
KD_NOALLOC_SCRATCH_BYTES = 64 << 20
STATUS = {
    0: "KD_OK", 1: "KD_ERR_INVALID_ARG", 2: "KD_ERR_UNSUPPORTED", 3: "KD_ERR_ALIGNMENT",
    4: "KD_ERR_WORKSPACE_TOO_SMALL", 5: "KD_ERR_INDEX_OUT_OF_RANGE", 6: "KD_ERR_HIP",
}

EXPORTS = (
    "kd_topk_kl_workspace_size", "kd_topk_kl_fwd", "kd_topk_kl_bwd",
    "kd_topk_kl_fwd_bwd_workspace_size", "kd_topk_kl_fwd_bwd",
    "kd_topk_kl_fwd_ex", "kd_topk_kl_bwd_ex", "kd_topk_kl_fwd_bwd_ex", "kd_topk_kl_fwd_noalloc",
    "kd_topk_kl_shard_workspace_size", "kd_topk_kl_fwd_shard", "kd_topk_kl_shard_combine", "kd_topk_kl_bwd_shard",
    "kd_full_kl_fwd_shard", "kd_full_kl_shard_combine", "kd_full_kl_bwd_shard",
    "kd_full_kl_workspace_size", "kd_full_kl_fwd", "kd_full_kl_bwd",
    "kd_full_kl_fwd_bwd_workspace_size", "kd_full_kl_fwd_bwd",
    "kd_full_kl_fwd_ex", "kd_full_kl_bwd_ex", "kd_full_kl_fwd_bwd_ex",
    "kd_status_string", "kd_last_error", "kd_version",
    "kd_profile_enable", "kd_profile_count", "kd_profile_get", "kd_profile_reset",
)


class KdTopkOpts(ctypes.Structure):
    """kd_topk_opts of kdloss.h: device pointers (0 = NULL), the CE weight, the index-check flag, the
    reverse-KL weight and the forward's z_topk (read by the backward under KL mixing)."""
    _fields_ = [("tau_rows", ctypes.c_void_p), ("teacher_lse", ctypes.c_void_p), ("labels", ctypes.c_void_p),
                ("ce_weight", ctypes.c_float), ("check_indices", ctypes.c_int32), ("rev_weight", ctypes.c_float),
                ("z_topk", ctypes.c_void_p)]


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
    L.kd_topk_kl_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, st, vp, vp, vp, vp]
    L.kd_topk_kl_fwd_noalloc.restype = st
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


# ---------------------------------------------------------------- argument checks
# The C ABI sees plain pointers and sizes, so this layer is the only one that
# can see shapes, dtypes and devices: every mirror below checks its tensors
# here, before any pointer is taken, and raises TypeError (dtype) or
# ValueError (shape, device, missing tensor).  Nothing is converted: an int64
# index tensor, say, is refused rather than read as pairs of int32.
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_MASK = (torch.uint8, torch.bool)
_HEAD = (torch.bfloat16, torch.float32)


def _need(name, t, shape=None, dtypes=None, optional=False):
    """t is a tensor of one of `dtypes` and exactly `shape` (None: any)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        want = " or ".join(str(d) for d in dtypes)
        hint = " (convert the indices with .int())" if dtypes == _I32 and t.dtype == torch.int64 else ""
        raise TypeError(f"{name} must be {want}, got {t.dtype}{hint}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _matrix(name, t, rows=None, dtypes=None):
    """A 2-D tensor (with `rows` rows if given); returns its shape."""
    _need(name, t, None, dtypes)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name} must have {rows} rows, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _one_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"libkdloss tensors must all be on one device, got {sorted(str(d) for d in devs)}")


def _ws_bytes(workspace):
    _need("workspace", workspace, optional=True)
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _topk_in(H, W, topk_idx, topk_logits, mask):
    """Inputs of a top-K call: H [T,d], W [d,V] of H's dtype, topk_idx [T,K]
    int32, topk_logits [T,K] float32, mask [T] uint8/bool or None."""
    T, d = _matrix("H", H, None, _HEAD)
    _, V = _matrix("W", W, d, (H.dtype,))
    _, K = _matrix("topk_idx", topk_idx, T, _I32)
    _need("topk_logits", topk_logits, (T, K), _F32)
    _need("mask", mask, (T,), _MASK, optional=True)
    return T, d, V, K


def _full_in(H, Ws, Ht, Wt, mask):
    """Inputs of a full-vocabulary call: H [T,d], Ws [d,V], Ht [T,dt], Wt [dt,V],
    all of H's dtype, mask [T] or None."""
    T, d = _matrix("H", H, None, _HEAD)
    _, V = _matrix("Ws", Ws, d, (H.dtype,))
    _, dt = _matrix("Ht", Ht, T, (H.dtype,))
    _need("Wt", Wt, (dt, V), (H.dtype,))
    _need("mask", mask, (T,), _MASK, optional=True)
    return T, d, dt, V


def _opts_in(opts, T, K=None):
    """The tensors an options struct points at (kept on it by topk_opts /
    full_opts) are [T] (z_topk: [T, K]) and of their documented dtype."""
    if opts is None:
        return ()
    kept = getattr(opts, "_tensors", None)
    if kept is None:
        raise TypeError("options must come from topk_opts(...) or full_opts(...)")
    for name, t, dtypes in kept:
        _need(name, t, (T, K) if name == "z_topk" else (T,), dtypes, optional=True)
    return tuple(t for _, t, _ in kept)


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


def _topk_fwd_checked(H, W, topk_idx, topk_logits, mask, opts, kl, lse, z_topk, workspace):
    T, d, V, K = _topk_in(H, W, topk_idx, topk_logits, mask)
    _need("kl", kl, (T,), _F32)
    _need("lse", lse, (T,), _F32)
    _need("z_topk", z_topk, (T, K), _F32, optional=True)
    nbytes = _ws_bytes(workspace)
    _one_device(H, W, topk_idx, topk_logits, mask, kl, lse, z_topk, workspace, *_opts_in(opts, T, K))
    return T, d, V, K, nbytes


def _topk_bwd_checked(H, W, topk_idx, topk_logits, mask, opts, lse, grad_kl, dH, dW, workspace, dh_dtype=None):
    T, d, V, K = _topk_in(H, W, topk_idx, topk_logits, mask)
    _need("lse", lse, (T,), _F32)
    _need("grad_kl", grad_kl, (T,), _F32)
    _need("dH", dH, (T, d), (dh_dtype or H.dtype,))
    _need("dW", dW, (d, V), _F32)
    nbytes = _ws_bytes(workspace)
    _one_device(H, W, topk_idx, topk_logits, mask, lse, grad_kl, dH, dW, workspace, *_opts_in(opts, T, K))
    return T, d, V, K, nbytes


def kd_topk_kl_fwd(H, W, topk_idx, topk_logits, mask, tau, kl, lse, z_topk, workspace, stream=None):
    """Enqueue the top-K forward; outputs kl, lse (and z_topk if given) in place."""
    T, d, V, K, nb = _topk_fwd_checked(H, W, topk_idx, topk_logits, mask, None, kl, lse, z_topk, workspace)
    _check(lib().kd_topk_kl_fwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                T, d, V, K, _dtype_code(H.dtype), _ptr(kl), _ptr(lse), _ptr(z_topk),
                                _ptr(workspace), nb, _stream(stream)), "kd_topk_kl_fwd")


def kd_topk_kl_fwd_noalloc(H, W, topk_idx, topk_logits, mask, tau, kl, lse, z_topk, stream=None):
    """kd_topk_kl_fwd without a workspace: the library's fixed scratch array serves instead (for callers
    that cannot allocate); calls that overlap on one GPU race."""
    T, d, V, K, _ = _topk_fwd_checked(H, W, topk_idx, topk_logits, mask, None, kl, lse, z_topk, None)
    _check(lib().kd_topk_kl_fwd_noalloc(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask),
                                        float(tau), T, d, V, K, _dtype_code(H.dtype), _ptr(kl), _ptr(lse),
                                        _ptr(z_topk), _stream(stream)), "kd_topk_kl_fwd_noalloc")


def kd_topk_kl_bwd(H, W, topk_idx, topk_logits, mask, tau, lse, grad_kl, dH, dW, chunk_rows, workspace,
                   stream=None):
    """Enqueue the top-K backward; outputs dH and dW in place."""
    T, d, V, K, nb = _topk_bwd_checked(H, W, topk_idx, topk_logits, mask, None, lse, grad_kl, dH, dW, workspace)
    _check(lib().kd_topk_kl_bwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                T, d, V, K, _dtype_code(H.dtype), _ptr(lse), _ptr(grad_kl), _ptr(dH), _ptr(dW),
                                int(chunk_rows), _ptr(workspace), nb, _stream(stream)), "kd_topk_kl_bwd")


def kd_topk_kl_fwd_bwd(H, W, topk_idx, topk_logits, mask, tau, grad_kl, kl, lse, z_topk, dH, dW, chunk_rows,
                       workspace, stream=None):
    """Enqueue the top-K forward and backward in one call (no recompute)."""
    kd_topk_kl_fwd_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, None, grad_kl, kl, lse, z_topk, dH, dW,
                          chunk_rows, workspace, stream, _name="kd_topk_kl_fwd_bwd")


def topk_opts(tau_rows=None, teacher_lse=None, labels=None, ce_weight=0.0, check_indices=False, rev_weight=0.0,
              z_topk=None):
    """The kd_topk_opts struct for these device tensors (or None when no option is set).  The
    tensors must stay alive until the call that takes the struct has been enqueued; the struct
    keeps a reference to them, and each call checks them against its T (z_topk: [T, K], the
    forward's output, which the backward reads when rev_weight > 0).  check_indices asks
    for the device-side index range check (the call then synchronises its stream once)."""
    if (tau_rows is None and teacher_lse is None and labels is None and not ce_weight and not check_indices
            and not rev_weight and z_topk is None):
        return None
    kept = (("tau_rows", tau_rows, _F32), ("teacher_lse", teacher_lse, _F32), ("labels", labels, _I32),
            ("z_topk", z_topk, _F32))
    for name, t, dtypes in kept:
        _need(name, t, None, dtypes, optional=True)
        want = 2 if name == "z_topk" else 1
        if t is not None and t.dim() != want:
            raise ValueError(f"{name} must be {want}-D, got shape {tuple(t.shape)}")
    o = KdTopkOpts(None, None, None, float(ce_weight), 1 if check_indices else 0, float(rev_weight), None)
    o._tensors = kept
    return o


def _opts_ref(opts):
    """A pointer to the options struct, its device pointers filled in from the tensors it keeps (after the
    call's checks, so a CPU test can reach every rejection first)."""
    if opts is None:
        return None
    for name, t, _ in opts._tensors:
        setattr(opts, name, None if t is None else _ptr(t).value)
    return ctypes.byref(opts)


def kd_topk_kl_fwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, kl, lse, z_topk, workspace, stream=None):
    """kd_topk_kl_fwd with a kd_topk_opts (topk_opts(...)) or None."""
    T, d, V, K, nb = _topk_fwd_checked(H, W, topk_idx, topk_logits, mask, opts, kl, lse, z_topk, workspace)
    _check(lib().kd_topk_kl_fwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                   _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype), _ptr(kl), _ptr(lse),
                                   _ptr(z_topk), _ptr(workspace), nb, _stream(stream)), "kd_topk_kl_fwd_ex")


def kd_topk_kl_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, lse, grad_kl, dH, dW, chunk_rows, workspace,
                      stream=None):
    """kd_topk_kl_bwd with a kd_topk_opts (the forward call's) or None."""
    T, d, V, K, nb = _topk_bwd_checked(H, W, topk_idx, topk_logits, mask, opts, lse, grad_kl, dH, dW, workspace)
    _check(lib().kd_topk_kl_bwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                   _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype), _ptr(lse), _ptr(grad_kl),
                                   _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace), nb, _stream(stream)),
           "kd_topk_kl_bwd_ex")


def kd_topk_kl_fwd_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, opts, grad_kl, kl, lse, z_topk, dH, dW,
                          chunk_rows, workspace, stream=None, _name="kd_topk_kl_fwd_bwd_ex"):
    """kd_topk_kl_fwd_bwd with a kd_topk_opts or None."""
    T, d, V, K = _topk_in(H, W, topk_idx, topk_logits, mask)
    _need("grad_kl", grad_kl, (T,), _F32)
    _need("kl", kl, (T,), _F32)
    _need("lse", lse, (T,), _F32)
    _need("z_topk", z_topk, (T, K), _F32, optional=True)
    _need("dH", dH, (T, d), (H.dtype,))
    _need("dW", dW, (d, V), _F32)
    nb = _ws_bytes(workspace)
    _one_device(H, W, topk_idx, topk_logits, mask, grad_kl, kl, lse, z_topk, dH, dW, workspace,
                *_opts_in(opts, T, K))
    if _name == "kd_topk_kl_fwd_bwd":
        st = lib().kd_topk_kl_fwd_bwd(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                      T, d, V, K, _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl), _ptr(lse),
                                      _ptr(z_topk), _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace), nb,
                                      _stream(stream))
    else:
        st = lib().kd_topk_kl_fwd_bwd_ex(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask),
                                         float(tau), _opts_ref(opts), T, d, V, K, _dtype_code(H.dtype),
                                         _ptr(grad_kl), _ptr(kl), _ptr(lse), _ptr(z_topk), _ptr(dH), _ptr(dW),
                                         int(chunk_rows), _ptr(workspace), nb, _stream(stream))
    _check(st, _name)


def kd_topk_kl_shard_workspace_size(T, d, V, v0, K, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t()
    _check(lib().kd_topk_kl_shard_workspace_size(T, d, V, v0, K, _dtype_code(dtype), int(chunk_rows),
                                                 ctypes.byref(out)), "kd_topk_kl_shard_workspace_size")
    return out.value


def kd_topk_kl_fwd_shard(H, W, v0, topk_idx, topk_logits, mask, tau, opts, rec, trow, z_topk, workspace,
                         stream=None):
    """One vocabulary shard's forward: W holds columns [v0, v0 + W.shape[1]) of the head; rec [T,4] and
    trow [T,2] float32 out."""
    T, d, V, K = _topk_in(H, W, topk_idx, topk_logits, mask)
    _need("rec", rec, (T, 4), _F32)
    _need("trow", trow, (T, 2), _F32)
    _need("z_topk", z_topk, (T, K), _F32, optional=True)
    nb = _ws_bytes(workspace)
    _one_device(H, W, topk_idx, topk_logits, mask, rec, trow, z_topk, workspace, *_opts_in(opts, T, K))
    _check(lib().kd_topk_kl_fwd_shard(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, V, int(v0), K, _dtype_code(H.dtype), _ptr(rec),
                                      _ptr(trow), _ptr(z_topk), _ptr(workspace), nb, _stream(stream)),
           "kd_topk_kl_fwd_shard")


def kd_topk_kl_shard_combine(rec, trow, mask, kl, lse, stream=None):
    """rec [R,T,4] (the shards' records in rank order), trow [T,2] -> kl [T], lse [T]."""
    _need("rec", rec, None, _F32)
    if rec.dim() != 3 or rec.shape[2] != 4:
        raise ValueError(f"rec must have shape (R, T, 4), got {tuple(rec.shape)}")
    R, T = int(rec.shape[0]), int(rec.shape[1])
    _need("trow", trow, (T, 2), _F32)
    _need("mask", mask, (T,), _MASK, optional=True)
    _need("kl", kl, (T,), _F32)
    _need("lse", lse, (T,), _F32)
    _one_device(rec, trow, mask, kl, lse)
    _check(lib().kd_topk_kl_shard_combine(_ptr(rec), R, _ptr(trow), _ptr(mask), T, _ptr(kl), _ptr(lse),
                                          _stream(stream)), "kd_topk_kl_shard_combine")


def kd_topk_kl_bwd_shard(H, W, v0, topk_idx, topk_logits, mask, tau, opts, lse, grad_kl, dH, dW, chunk_rows,
                         workspace, stream=None):
    """One vocabulary shard's backward with the whole head's lse: dH [T,d] float32 (a partial) and
    dW [d,V] float32 (the shard's columns)."""
    T, d, V, K, nb = _topk_bwd_checked(H, W, topk_idx, topk_logits, mask, opts, lse, grad_kl, dH, dW, workspace,
                                       dh_dtype=torch.float32)
    _check(lib().kd_topk_kl_bwd_shard(_ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logits), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, V, int(v0), K, _dtype_code(H.dtype), _ptr(lse),
                                      _ptr(grad_kl), _ptr(dH), _ptr(dW), int(chunk_rows), _ptr(workspace), nb,
                                      _stream(stream)), "kd_topk_kl_bwd_shard")


def full_opts(tau_rows=None, rev_weight=0.0):
    """The kd_full_opts struct (or None when no option is set); it keeps a reference to tau_rows."""
    if tau_rows is None and not rev_weight:
        return None
    _need("tau_rows", tau_rows, None, _F32, optional=True)
    if tau_rows is not None and tau_rows.dim() != 1:
        raise ValueError(f"tau_rows must be 1-D [T], got shape {tuple(tau_rows.shape)}")
    o = KdFullOpts(None, float(rev_weight))
    o._tensors = (("tau_rows", tau_rows, _F32),)
    return o


def _full_fwd_checked(H, Ws, Ht, Wt, mask, opts, kl, lse_s, lse_t, kl_rev, workspace):
    T, d, dt, V = _full_in(H, Ws, Ht, Wt, mask)
    for name, t in (("kl", kl), ("lse_s", lse_s), ("lse_t", lse_t)):
        _need(name, t, (T,), _F32)
    _need("kl_rev", kl_rev, (T,), _F32, optional=True)
    nb = _ws_bytes(workspace)
    _one_device(H, Ws, Ht, Wt, mask, kl, lse_s, lse_t, kl_rev, workspace, *_opts_in(opts, T))
    return T, d, dt, V, nb


def _full_bwd_checked(H, Ws, Ht, Wt, mask, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, workspace, dh_dtype=None):
    T, d, dt, V = _full_in(H, Ws, Ht, Wt, mask)
    for name, t in (("lse_s", lse_s), ("lse_t", lse_t), ("grad_kl", grad_kl)):
        _need(name, t, (T,), _F32)
    _need("kl_rev", kl_rev, (T,), _F32, optional=True)
    _need("dH", dH, (T, d), (dh_dtype or H.dtype,))
    _need("dWs", dWs, (d, V), _F32)
    nb = _ws_bytes(workspace)
    _one_device(H, Ws, Ht, Wt, mask, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, workspace, *_opts_in(opts, T))
    return T, d, dt, V, nb


def kd_full_kl_fwd(H, Ws, Ht, Wt, mask, tau, kl, lse_s, lse_t, workspace, stream=None):
    T, d, dt, V, nb = _full_fwd_checked(H, Ws, Ht, Wt, mask, None, kl, lse_s, lse_t, None, workspace)
    _check(lib().kd_full_kl_fwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                _dtype_code(H.dtype), _ptr(kl), _ptr(lse_s), _ptr(lse_t), _ptr(workspace), nb,
                                _stream(stream)), "kd_full_kl_fwd")


def kd_full_kl_bwd(H, Ws, Ht, Wt, mask, tau, lse_s, lse_t, grad_kl, dH, dWs, chunk_rows, workspace, stream=None):
    T, d, dt, V, nb = _full_bwd_checked(H, Ws, Ht, Wt, mask, None, lse_s, lse_t, None, grad_kl, dH, dWs,
                                        workspace)
    _check(lib().kd_full_kl_bwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t), _ptr(grad_kl), _ptr(dH),
                                _ptr(dWs), int(chunk_rows), _ptr(workspace), nb, _stream(stream)), "kd_full_kl_bwd")


def kd_full_kl_fwd_bwd_workspace_size(T, d, dt_hidden, V, dtype, chunk_rows=0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kd_full_kl_fwd_bwd_workspace_size(T, d, dt_hidden, V, _dtype_code(dtype), chunk_rows,
                                                   ctypes.byref(out)),
           "kd_full_kl_fwd_bwd_workspace_size")
    return out.value


def _full_fwd_bwd_checked(H, Ws, Ht, Wt, mask, opts, grad_kl, kl, lse_s, lse_t, kl_rev, dH, dWs, workspace):
    T, d, dt, V = _full_in(H, Ws, Ht, Wt, mask)
    for name, t in (("grad_kl", grad_kl), ("kl", kl), ("lse_s", lse_s), ("lse_t", lse_t)):
        _need(name, t, (T,), _F32)
    _need("kl_rev", kl_rev, (T,), _F32, optional=True)
    _need("dH", dH, (T, d), (H.dtype,))
    _need("dWs", dWs, (d, V), _F32)
    nb = _ws_bytes(workspace)
    _one_device(H, Ws, Ht, Wt, mask, grad_kl, kl, lse_s, lse_t, kl_rev, dH, dWs, workspace, *_opts_in(opts, T))
    return T, d, dt, V, nb


def kd_full_kl_fwd_bwd(H, Ws, Ht, Wt, mask, tau, grad_kl, kl, lse_s, lse_t, dH, dWs, chunk_rows, workspace,
                       stream=None):
    """Enqueue the full-vocabulary forward and backward in one call (no recompute)."""
    T, d, dt, V, nb = _full_fwd_bwd_checked(H, Ws, Ht, Wt, mask, None, grad_kl, kl, lse_s, lse_t, None, dH, dWs,
                                            workspace)
    _check(lib().kd_full_kl_fwd_bwd(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), T, d, dt, V,
                                    _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl), _ptr(lse_s), _ptr(lse_t),
                                    _ptr(dH), _ptr(dWs), int(chunk_rows), _ptr(workspace), nb, _stream(stream)),
           "kd_full_kl_fwd_bwd")


def kd_full_kl_fwd_ex(H, Ws, Ht, Wt, mask, tau, opts, kl, lse_s, lse_t, kl_rev, workspace, stream=None):
    T, d, dt, V, nb = _full_fwd_checked(H, Ws, Ht, Wt, mask, opts, kl, lse_s, lse_t, kl_rev, workspace)
    _check(lib().kd_full_kl_fwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), _opts_ref(opts),
                                   T, d, dt, V, _dtype_code(H.dtype), _ptr(kl), _ptr(lse_s), _ptr(lse_t),
                                   _ptr(kl_rev), _ptr(workspace), nb, _stream(stream)), "kd_full_kl_fwd_ex")


def kd_full_kl_bwd_ex(H, Ws, Ht, Wt, mask, tau, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, chunk_rows, workspace,
                      stream=None):
    T, d, dt, V, nb = _full_bwd_checked(H, Ws, Ht, Wt, mask, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs,
                                        workspace)
    _check(lib().kd_full_kl_bwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau), _opts_ref(opts),
                                   T, d, dt, V, _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t), _ptr(kl_rev),
                                   _ptr(grad_kl), _ptr(dH), _ptr(dWs), int(chunk_rows), _ptr(workspace), nb,
                                   _stream(stream)), "kd_full_kl_bwd_ex")


def kd_full_kl_fwd_bwd_ex(H, Ws, Ht, Wt, mask, tau, opts, grad_kl, kl, lse_s, lse_t, kl_rev, dH, dWs, chunk_rows,
                          workspace, stream=None):
    T, d, dt, V, nb = _full_fwd_bwd_checked(H, Ws, Ht, Wt, mask, opts, grad_kl, kl, lse_s, lse_t, kl_rev, dH, dWs,
                                            workspace)
    _check(lib().kd_full_kl_fwd_bwd_ex(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                       _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(grad_kl), _ptr(kl),
                                       _ptr(lse_s), _ptr(lse_t), _ptr(kl_rev), _ptr(dH), _ptr(dWs), int(chunk_rows),
                                       _ptr(workspace), nb, _stream(stream)), "kd_full_kl_fwd_bwd_ex")


def kd_full_kl_fwd_shard(H, Ws, Ht, Wt, mask, tau, opts, rec, workspace, stream=None):
    """One vocabulary shard's full-vocabulary forward: Ws and Wt hold the same columns of both heads;
    rec [T,8] float32 out."""
    T, d, dt, V = _full_in(H, Ws, Ht, Wt, mask)
    _need("rec", rec, (T, 8), _F32)
    nb = _ws_bytes(workspace)
    _one_device(H, Ws, Ht, Wt, mask, rec, workspace, *_opts_in(opts, T))
    _check(lib().kd_full_kl_fwd_shard(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(rec), _ptr(workspace),
                                      nb, _stream(stream)), "kd_full_kl_fwd_shard")


def kd_full_kl_shard_combine(rec, mask, rev_weight, kl, lse_s, lse_t, kl_rev, stream=None):
    """rec [R,T,8] (the shards' records in rank order) -> kl, lse_s, lse_t [T] and kl_rev [T] or None."""
    _need("rec", rec, None, _F32)
    if rec.dim() != 3 or rec.shape[2] != 8:
        raise ValueError(f"rec must have shape (R, T, 8), got {tuple(rec.shape)}")
    R, T = int(rec.shape[0]), int(rec.shape[1])
    _need("mask", mask, (T,), _MASK, optional=True)
    for name, t in (("kl", kl), ("lse_s", lse_s), ("lse_t", lse_t)):
        _need(name, t, (T,), _F32)
    _need("kl_rev", kl_rev, (T,), _F32, optional=True)
    _one_device(rec, mask, kl, lse_s, lse_t, kl_rev)
    _check(lib().kd_full_kl_shard_combine(_ptr(rec), R, _ptr(mask), T, float(rev_weight), _ptr(kl), _ptr(lse_s),
                                          _ptr(lse_t), _ptr(kl_rev), _stream(stream)), "kd_full_kl_shard_combine")


def kd_full_kl_bwd_shard(H, Ws, Ht, Wt, mask, tau, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs, chunk_rows,
                         workspace, stream=None):
    """One vocabulary shard's full-vocabulary backward with the whole heads' log-normalisers: dH [T,d] float32
    (a partial) and dWs [d,V] float32 (the shard's columns)."""
    T, d, dt, V, nb = _full_bwd_checked(H, Ws, Ht, Wt, mask, opts, lse_s, lse_t, kl_rev, grad_kl, dH, dWs,
                                        workspace, dh_dtype=torch.float32)
    _check(lib().kd_full_kl_bwd_shard(_ptr(H), _ptr(Ws), _ptr(Ht), _ptr(Wt), _ptr(mask), float(tau),
                                      _opts_ref(opts), T, d, dt, V, _dtype_code(H.dtype), _ptr(lse_s), _ptr(lse_t),
                                      _ptr(kl_rev), _ptr(grad_kl), _ptr(dH), _ptr(dWs), int(chunk_rows),
                                      _ptr(workspace), nb, _stream(stream)), "kd_full_kl_bwd_shard")


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
