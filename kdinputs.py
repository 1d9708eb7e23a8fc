"""Seeded synthetic inputs for the fused chunked KL loss.

This module only draws random numbers and shapes them; it holds none of the
loss's arithmetic.  Both the oracle's tests and the GPU path read the tensors it
returns, so the two sides always see the same bits.

Workload shapes and distributions follow the loss-only output-head benchmark
described on the page "Efficient Knowledge Distillation for LLMs: Offline Top-K
Logits and a Fused Chunked KL Loss" (App. B, "Controlled configuration":
deterministic hidden states, output-projection weights and sparse teacher
targets, generated once per configuration and reused by every loss).  The pages
give no d, V or K for that benchmark; the presets below use a Llama-3-style head
(d=3072, V=128256) with a K=64 cache (the paper's own cache keeps K=100, §3).

Conventions:
  * ``N(0, v)`` means variance ``v`` (std ``sqrt(v)``).
  * Values are drawn in float32 from NumPy PCG64 streams and rounded to the
    storage dtype (bf16 rounding is round-to-nearest-even, done by torch).
  * Every tensor role has its own seed: H=1, W=2, A (teacher logits)=3,
    I (indices)=4, mask=5, g (upstream gradient)=6, Ht=7, Wt=8, per-token
    temperature=9, cached probabilities=10, labels=11, each plus
    ``100 * preset_number``.
  * Large tensors are filled block by block; block ``b`` of role ``r`` always
    uses ``SeedSequence([seed_r, b])``, so results do not depend on the thread
    count.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, field

import numpy as np
import torch

ROLE_H, ROLE_W, ROLE_A, ROLE_I, ROLE_MASK, ROLE_G, ROLE_HT, ROLE_WT = 1, 2, 3, 4, 5, 6, 7, 8
ROLE_TAU, ROLE_MASS, ROLE_Y = 9, 10, 11
_BLOCK = 1 << 22  # elements per independently seeded block


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_f32(seed: int, n: int, std: float) -> np.ndarray:
    """n draws of N(0, std^2) in float32, block-seeded and filled in parallel."""
    out = np.empty(n, dtype=np.float32)
    nblocks = (n + _BLOCK - 1) // _BLOCK

    def fill(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nblocks <= 1:
        for b in range(nblocks):
            fill(b)
    else:
        with _fut.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def normal(seed: int, shape, var: float, dtype: torch.dtype) -> torch.Tensor:
    """Tensor of N(0, var) draws with the given shape, rounded to ``dtype``."""
    n = int(np.prod(shape)) if len(shape) else 1
    x = torch.from_numpy(_normal_f32(seed, n, float(np.sqrt(var)))).reshape(shape)
    return x.to(dtype)


def distinct_indices(seed: int, T: int, K: int, V: int) -> torch.Tensor:
    """[T, K] int32: K distinct indices per row, uniform over [0, V)."""
    if K > V:
        raise ValueError("K > V")
    rng = np.random.Generator(np.random.PCG64(seed))
    if 4 * K >= V:
        # dense case: a random permutation prefix per row
        keys = rng.random((T, V))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :K]
        return torch.from_numpy(idx.astype(np.int32))
    idx = rng.integers(0, V, size=(T, K), dtype=np.int64)
    while True:
        s = np.sort(idx, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            break
        idx[bad] = rng.integers(0, V, size=(bad.size, K), dtype=np.int64)
    return torch.from_numpy(idx.astype(np.int32))


def teacher_logits(seed: int, T: int, K: int, var: float) -> torch.Tensor:
    """[T, K] float32 teacher top-K logits ~ N(0, var), sorted descending per row
    (a top-K cache stores the K largest entries in order)."""
    a = _normal_f32(seed, T * K, float(np.sqrt(var))).reshape(T, K)
    a = -np.sort(-a, axis=1)
    return torch.from_numpy(np.ascontiguousarray(a))


def mask_random_rows(seed: int, T: int, n_masked: int) -> torch.Tensor:
    """[T] uint8 mask with exactly ``n_masked`` rows set to 0 (seeded permutation)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.ones(T, dtype=np.uint8)
    m[rng.permutation(T)[:n_masked]] = 0
    return torch.from_numpy(m)


def mask_packed_tail(T: int, seq_len: int, n_pad: int) -> torch.Tensor:
    """[T] uint8 mask for T rows packed as sequences of ``seq_len`` whose last
    ``n_pad`` rows are padding (0)."""
    m = np.ones(T, dtype=np.uint8)
    for s in range(0, T, seq_len):
        m[max(s, s + seq_len - n_pad):s + seq_len] = 0
    return torch.from_numpy(m)


@dataclass
class Preset:
    """One named workload."""
    name: str
    number: int
    T: int
    d: int
    V: int
    K: int
    dtype: torch.dtype
    tau: float
    teacher_var: float = 3.0
    mask: str = "none"          # "none" | "random10" | "packed"
    seq_len: int = 4096
    n_pad: int = 205
    full_vocab: bool = False
    dt_hidden: int = 0
    extra: dict = field(default_factory=dict)


PRESETS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny_topk_fp32": Preset("tiny_topk_fp32", 1, T=256, d=256, V=4096, K=16,
                             dtype=torch.float32, tau=1.0, teacher_var=2.0, mask="random10"),
    # the output-head workload: 4096 tokens through a 3072 x 128256 head
    "head_topk_t4096": Preset("head_topk_t4096", 2, T=4096, d=3072, V=128256, K=64,
                              dtype=torch.bfloat16, tau=1.0),
    # long context: 8 packed sequences of 4096 with 205 padding rows each
    "head_topk_t32768_packed": Preset("head_topk_t32768_packed", 3, T=32768, d=3072, V=128256,
                                      K=64, dtype=torch.bfloat16, tau=2.0, mask="packed"),
    # full-vocabulary KL through a frozen teacher head
    "full_vocab_t16384": Preset("full_vocab_t16384", 5, T=16384, d=3072, V=128256, K=0,
                                dtype=torch.bfloat16, tau=1.0, full_vocab=True, dt_hidden=4096),
}

SWEEP_T = (4096, 16384, 65536, 262144)


def sweep_preset(T: int) -> Preset:
    """Loss-only scaling sweep point: the output-head workload at T tokens."""
    return Preset(f"head_topk_sweep_t{T}", 4, T=T, d=3072, V=128256, K=64,
                  dtype=torch.bfloat16, tau=1.0)


def make_topk(T, d, V, K, dtype, tau=1.0, teacher_var=3.0, mask="none", number=0,
              seq_len=4096, n_pad=205, n_masked=None, g="mean"):
    """Inputs of the top-K loss as CPU tensors.

    Returns a dict with H [T,d], W [d,V] (dtype), I [T,K] int32, A [T,K] float32,
    mask [T] uint8 or None, g [T] float32 and tau.  ``g="mean"`` gives
    1/N_valid on valid rows (mean over valid tokens); ``g="normal"`` gives N(0,1).
    """
    base = 100 * number
    H = normal(ROLE_H + base, (T, d), 1.0, dtype)
    W = normal(ROLE_W + base, (d, V), 1.0 / d, dtype)
    A = teacher_logits(ROLE_A + base, T, K, teacher_var)
    I = distinct_indices(ROLE_I + base, T, K, V)
    if mask == "none":
        M = None
    elif mask == "random10":
        M = mask_random_rows(ROLE_MASK + base, T, (T // 10) if n_masked is None else n_masked)
    elif mask == "packed":
        M = mask_packed_tail(T, seq_len, n_pad)
    else:
        raise ValueError(mask)
    nvalid = T if M is None else int(M.sum())
    if g == "mean":
        G = torch.full((T,), 1.0 / max(1, nvalid), dtype=torch.float32)
    elif g == "normal":
        G = normal(ROLE_G + base, (T,), 1.0, torch.float32)
    else:
        raise ValueError(g)
    return dict(H=H, W=W, I=I, A=A, mask=M, g=G, tau=float(tau))


def add_topk_options(inp, tau_rows=False, partial_mass=False, labels=False, ce_weight=0.0, number=0):
    """Inputs of the optional parts of the top-K loss, added to a make_topk dict.

    tau_rows: [T] float32 per-token temperatures, uniform in [0.5, 2).
    partial_mass: the cache holds probabilities of the full teacher softmax.
      Row t draws a mass m_t uniform in [0.5, 0.99) and K heavy-tailed weights
      u^4 (u uniform), sorted descending and scaled to sum to m_t; A is
      replaced by tau_t (log p + c_t) and teacher_lse is c_t ~ N(0, 1), so the
      cached entries are exactly those probabilities at the row's temperature.
    labels: [T] int32 next-token labels: the row's first cached index with
      probability 1/2, else uniform over [0, V); ce_weight is stored with them.
    """
    base = 100 * number
    T, K = inp["I"].shape
    V = inp["W"].shape[1]
    out = dict(inp)
    taus = np.full(T, inp["tau"], dtype=np.float64)
    if tau_rows:
        rng = np.random.Generator(np.random.PCG64(ROLE_TAU + base))
        tr = rng.uniform(0.5, 2.0, T).astype(np.float32)
        out["tau_rows"] = torch.from_numpy(tr)
        taus = tr.astype(np.float64)
    if partial_mass:
        rng = np.random.Generator(np.random.PCG64(ROLE_MASS + base))
        m = rng.uniform(0.5, 0.99, T)
        u = -np.sort(-(rng.random((T, K)) ** 4), axis=1)
        u = np.maximum(u, 1e-30)
        p = u * (m / u.sum(axis=1))[:, None]
        c = rng.standard_normal(T)
        out["A"] = torch.from_numpy((taus[:, None] * (np.log(p) + c[:, None])).astype(np.float32))
        out["teacher_lse"] = torch.from_numpy(c.astype(np.float32))
    if labels:
        rng = np.random.Generator(np.random.PCG64(ROLE_Y + base))
        y = rng.integers(0, V, T)
        top = rng.random(T) < 0.5
        y[top] = inp["I"].numpy()[top, 0]
        out["labels"] = torch.from_numpy(y.astype(np.int32))
        out["ce_weight"] = float(ce_weight)
    return out


def add_full_options(inp, tau_rows=False, rev_weight=0.0, number=0):
    """Options of the full-vocabulary loss added to a make_full dict:
    tau_rows [T] float32 uniform in [0.5, 2) (per-token temperature) and the
    weight of the reverse KL."""
    out = dict(inp)
    if tau_rows:
        rng = np.random.Generator(np.random.PCG64(ROLE_TAU + 100 * number))
        out["tau_rows"] = torch.from_numpy(rng.uniform(0.5, 2.0, inp["H"].shape[0]).astype(np.float32))
    out["rev_weight"] = float(rev_weight)
    return out


def make_full(T, d, dt, V, dtype, tau=1.0, mask="none", number=0, g="mean", n_masked=None):
    """Inputs of the full-vocabulary loss as CPU tensors: H [T,d], Ws [d,V],
    Ht [T,dt], Wt [dt,V], mask, g, tau.  Each head is N(0, 1/its own width)."""
    base = 100 * number
    H = normal(ROLE_H + base, (T, d), 1.0, dtype)
    Ws = normal(ROLE_W + base, (d, V), 1.0 / d, dtype)
    Ht = normal(ROLE_HT + base, (T, dt), 1.0, dtype)
    Wt = normal(ROLE_WT + base, (dt, V), 1.0 / dt, dtype)
    if mask == "none":
        M = None
    elif mask == "random10":
        M = mask_random_rows(ROLE_MASK + base, T, (T // 10) if n_masked is None else n_masked)
    else:
        raise ValueError(mask)
    nvalid = T if M is None else int(M.sum())
    if g == "mean":
        G = torch.full((T,), 1.0 / max(1, nvalid), dtype=torch.float32)
    else:
        G = normal(ROLE_G + base, (T,), 1.0, torch.float32)
    return dict(H=H, Ws=Ws, Ht=Ht, Wt=Wt, mask=M, g=G, tau=float(tau))


def make_preset(p: Preset, g="mean"):
    if p.full_vocab:
        return make_full(p.T, p.d, p.dt_hidden, p.V, p.dtype, tau=p.tau, number=p.number, g=g)
    return make_topk(p.T, p.d, p.V, p.K, p.dtype, tau=p.tau, teacher_var=p.teacher_var,
                     mask=p.mask, number=p.number, seq_len=p.seq_len, n_pad=p.n_pad, g=g)
