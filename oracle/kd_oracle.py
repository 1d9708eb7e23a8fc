"""fp64 CPU oracle for the fused, chunked KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is the plain, slow, obviously correct definition of what the fused kernels
compute.  Sources, cited by page title and section:

[EKD]    "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
         Fused Chunked KL Loss" (paperlayer.ai summary of arXiv 2608.03796).
         §1 and §3 "Online distillation": the objective is the forward KL
         KL(p_teacher || q_student).  §3 "Offline distillation": only the K
         cached teacher entries are kept; the teacher-entropy, cross and mass
         terms use support entries only and the student log-normaliser log Z is
         the one full-vocabulary reduction.  §3 "Offline implementations": the
         dense reconstruction (scatter the top-K into a dense teacher) is the
         correctness baseline; the sparse variant writes a scalar log Z per row
         and scatter-adds over the K retained entries.  §3 "Fused chunked KL":
         the output projection Z = H.W is part of the loss.
[KDFlow] KDFlow abstract (thelatestinai.com/papers/2606.20005): full-vocabulary
         distillation recomputes the teacher logits from the teacher's final
         hidden states through a frozen copy of the teacher's output head.

[KLD]    KL-direction abstract (thelatestinai.com/papers/2606.20005): forward
         and reverse token-level KL, and their mixture ("KL mixing").
[AKD]    Adaptive-distillation abstract (on the WASD page,
         thelatestinai.com/papers/2610.07706): the distillation temperature is
         adjusted per token.
[TS]     Teacher-strength abstract (thelatestinai.com/papers/2605.11513): the
         language-modelling and distillation losses are mixed.

Readings where the pages are silent (each is listed with its reason in the
design notes of this repository):
  * Teacher top-K logits are renormalised over the K entries at temperature tau
    (mass m = 1) by default.  ``topk_loss_*`` also take the pages' partial-mass
    form: a per-row teacher log-normaliser gives the cached probabilities
    p_k = exp(A_k / tau - teacher_lse), whose mass m = sum_k p_k may be < 1.
  * Per-token temperature: tau_t replaces tau for row t, on both sides.
  * The LM cross-entropy term is the K = 1 case of the same loss (one cached
    entry, the label, with p = 1) at the same temperature; the mixed loss is
    (1 - beta) KD + beta CE.
  * KL mixing (full vocabulary): (1 - r) KL(p || q) + r KL(q || p), both at
    the row's temperature.
  * KL mixing (top-K): the reverse direction needs the teacher wherever the
    student has mass, and outside the K cached entries the teacher is unknown.
    Both sides are therefore restricted to the cached entries and renormalised
    there: q~ = softmax over the K entries of s[I_tk], p^ = softmax(A_t / tau_t)
    (the cached probabilities renormalised, also with a partial mass), each
    entry its own outcome (a duplicated index counts once per entry), and
        RKL_t = sum_k q~_k (log q~_k - log p^_k),
        loss_t = (1 - beta) [(1 - r) KD_t + r RKL_t] + beta CE_t.
  * Both teacher and student logits are divided by tau; there is no tau^2.
  * The output is per token; the caller reduces.  ``g`` is dLoss/dKL_t.
  * mask[t] == 1 marks a valid row.  Masked rows give KL = 0, lse = 0,
    z_topk = 0, dH = 0 and contribute nothing to dW, whatever their contents.
  * Duplicate indices in a row add (scatter-add).
  * W is [d, V] row-major; Z = H @ W.

Parity of every function here is pinned by ``tests/test_oracle.py`` against
closed forms, library routines, finite differences and brute force.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64", "logsumexp_rows", "teacher_log_probs",
    "topk_kl_forward", "topk_kl_backward", "topk_kl_rows",
    "topk_loss_forward", "topk_loss_backward", "topk_loss_rows",
    "topk_shard_terms", "topk_shard_backward", "full_shard_terms", "full_shard_backward",
    "full_kl_forward", "full_kl_backward", "full_kl_rows",
    "full_loss_forward", "full_loss_backward", "full_loss_rows",
]


def as_f64(x):
    """Exact float64 copy of a NumPy array or a torch tensor (bf16 included)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 has no NumPy dtype
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _take_rows(x, rows):
    """x[rows] for a NumPy array or a torch tensor (no arithmetic)."""
    if x is None:
        return None
    if hasattr(x, "index_select"):
        import torch
        return x.index_select(0, torch.as_tensor(rows, dtype=torch.long))
    return np.asarray(x)[rows]


def _valid_rows(mask, T):
    if mask is None:
        return np.ones(T, dtype=bool)
    m = np.asarray(mask.cpu().numpy() if hasattr(mask, "cpu") else mask)
    return m.astype(np.int64) != 0


def logsumexp_rows(x):
    """log sum_j exp(x[i, j]) per row, max-shifted.  ([EKD] §3: the scalar log Z
    of each row, computed with a stable vocabulary reduction.)"""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]


def teacher_log_probs(A, tau):
    """Teacher log-probabilities over its K cached entries: log softmax(A / tau)
    per row (top-K renormalised at temperature tau)."""
    a = np.asarray(A, dtype=np.float64) / tau
    return a - logsumexp_rows(a)[:, None]


def _student_block(Hb, W, tau):
    """Scaled logits s = (Hb @ W) / tau and their row log-normaliser L."""
    z = Hb @ W
    s = z / tau
    return z, s, logsumexp_rows(s)


def topk_kl_forward(H, W, I, A, mask, tau, row_block=64):
    """Per-token KL(p_t || q_t) against a top-K teacher ([EKD] §3 "Offline
    distillation").

    For a valid row t with s = (H_t W) / tau, L_t = logsumexp(s) and
    p = softmax(A_t / tau) over the K entries:
        KL_t = sum_k p_k (log p_k - s[I_tk] + L_t)
             = [teacher entropy term] - [cross term] + [mass * log Z], mass = 1.
    Returns (kl [T], lse [T] = L_t, z_topk [T, K] = z at the cached indices).
    """
    H, W, A = as_f64(H), as_f64(W), as_f64(A)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, K = I.shape
    valid = _valid_rows(mask, T)
    kl = np.zeros(T)
    lse = np.zeros(T)
    ztk = np.zeros((T, K))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        z, s, L = _student_block(H[rb], W, tau)
        logp = teacher_log_probs(A[rb], tau)
        p = np.exp(logp)
        s_at = np.take_along_axis(s, I[rb], axis=1)
        kl[rb] = (p * (logp - s_at + L[:, None])).sum(axis=1)
        lse[rb] = L
        ztk[rb] = np.take_along_axis(z, I[rb], axis=1)
    return kl, lse, ztk


def _topk_dz(s, L, I_rows, p, g_rows, tau):
    """dKL/dz for a block of rows: (g/tau) (softmax(s) - scatter_add(I, p))."""
    q = np.exp(s - L[:, None])
    r = np.repeat(np.arange(s.shape[0]), I_rows.shape[1])
    np.add.at(q, (r, I_rows.reshape(-1)), -p.reshape(-1))  # duplicates add
    return q * (g_rows / tau)[:, None]


def topk_kl_backward(H, W, I, A, mask, tau, g, row_block=64, v_panel=16384):
    """Gradients of sum_t g_t KL_t w.r.t. H and W ([EKD] §3: the backward pass
    needs each row's log Z and the scatter over the K retained entries).

    dZ_t = (g_t / tau) (softmax(s_t) - scatter_add(I_t, p_t)); dH = dZ W^T;
    dW = H^T dZ; masked rows have dZ_t = 0.  Returns (dH [T, d], dW [d, V])."""
    H, W, A, g = as_f64(H), as_f64(W), as_f64(A), as_f64(g)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, d = H.shape
    V = W.shape[1]
    valid = _valid_rows(mask, T)
    dH = np.zeros((T, d))
    dW = np.zeros((d, V))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, L = _student_block(H[rb], W, tau)
        p = np.exp(teacher_log_probs(A[rb], tau))
        D = _topk_dz(s, L, I[rb], p, g[rb], tau)
        dH[rb] = D @ W.T
        for v0 in range(0, V, v_panel):
            dW[:, v0:v0 + v_panel] += H[rb].T @ D[:, v0:v0 + v_panel]
    return dH, dW


def topk_kl_rows(H, W, I, A, mask, tau, g, rows):
    """kl, lse, z_topk and dH for selected rows only: each depends on its own
    row and on W alone, so large workloads are checked on a sample of rows."""
    rows = np.asarray(rows, dtype=np.int64)
    Hr, Ir, Ar = as_f64(_take_rows(H, rows)), _take_rows(I, rows), _take_rows(A, rows)
    mr, gr = _take_rows(mask, rows), _take_rows(g, rows)
    W = as_f64(W)
    kl, lse, ztk = topk_kl_forward(Hr, W, Ir, Ar, mr, tau)
    dH, _ = _rows_dh_topk(Hr, W, Ir, Ar, mr, tau, gr)
    return kl, lse, ztk, dH


def _rows_dh_topk(H, W, I, A, mask, tau, g, row_block=64):
    H, A, g = as_f64(H), as_f64(A), as_f64(g)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, d = H.shape
    valid = _valid_rows(mask, T)
    dH = np.zeros((T, d))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, L = _student_block(H[rb], W, tau)
        p = np.exp(teacher_log_probs(A[rb], tau))
        dH[rb] = _topk_dz(s, L, I[rb], p, g[rb], tau) @ W.T
    return dH, None


def _row_values(x, T, default):
    """Per-row array of length T from an optional NumPy array / tensor."""
    if x is None:
        return np.full(T, default, dtype=np.float64)
    return as_f64(x).reshape(T)


def _loss_block(H, W, A, rb, taus, tlse):
    """What the general top-K loss needs for a block of valid rows rb: raw
    logits z, scaled logits s, their log-normaliser L, the teacher's
    probabilities p and log-probabilities, and the mass m = sum_k p_k."""
    tau = taus[rb][:, None]
    z = H[rb] @ W
    s = z / tau
    L = logsumexp_rows(s)
    a = A[rb] / tau
    if tlse is None:   # renormalised over the K entries
        logp = a - logsumexp_rows(a)[:, None]
    else:              # the cached probabilities of the full teacher softmax
        logp = a - tlse[rb][:, None]
    p = np.exp(logp)
    m = p.sum(axis=1)
    return z, s, L, p, logp, m


def topk_loss_forward(H, W, I, A, mask, tau, tau_rows=None, teacher_lse=None, labels=None, ce_weight=0.0,
                      rev_weight=0.0, row_block=64):
    """Per-token top-K distillation loss with the optional parts of the method.

    For a valid row t, with tau_t the row's temperature ([AKD]; tau when
    tau_rows is None), s = (H_t W) / tau_t, L_t = logsumexp(s) and the cached
    teacher probabilities p (renormalised, or with mass m_t = sum_k p_k when
    teacher_lse is given: [EKD] §3 "Offline distillation", partial mass):
        KD_t = sum_k p_k log p_k - sum_k p_k s[I_tk] + m_t L_t
    (teacher-entropy, cross and mass terms; only L_t needs the vocabulary).
    With labels y ([TS]):  CE_t = L_t - s[y_t],  loss_t = (1 - beta) KD_t + beta CE_t.
    With r = rev_weight > 0 ([KLD], KL mixing restricted to the cached
    entries, _support_reverse): KD_t is replaced by (1 - r) KD_t + r RKL_t.
    Returns (loss [T], lse [T] = L_t, z_topk [T, K])."""
    H, W, A = as_f64(H), as_f64(W), as_f64(A)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, K = I.shape
    taus = _row_values(tau_rows, T, tau)
    tlse = None if teacher_lse is None else _row_values(teacher_lse, T, 0.0)
    y = None if labels is None else np.asarray(labels.cpu().numpy() if hasattr(labels, "cpu") else labels,
                                               dtype=np.int64)
    beta = float(ce_weight)
    r = float(rev_weight)
    valid = _valid_rows(mask, T)
    loss, lse, ztk = np.zeros(T), np.zeros(T), np.zeros((T, K))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        z, s, L, p, logp, m = _loss_block(H, W, A, rb, taus, tlse)
        s_at = np.take_along_axis(s, I[rb], axis=1)
        kd = (p * logp).sum(axis=1) - (p * s_at).sum(axis=1) + m * L
        if r != 0.0:
            rkl, _ = _support_reverse(s_at, A[rb] / taus[rb][:, None])
            kd = (1.0 - r) * kd + r * rkl
        if y is not None and beta != 0.0:
            ce = L - s[np.arange(rb.size), y[rb]]
            loss[rb] = (1.0 - beta) * kd + beta * ce
        else:
            loss[rb] = kd
        lse[rb] = L
        ztk[rb] = np.take_along_axis(z, I[rb], axis=1)
    return loss, lse, ztk


def _support_reverse(a, b):
    """Reverse KL over the K cached entries ([KLD] reverse token-level KL, on
    the support where the teacher is known): a [n, K] the student's scaled
    logits at the entries, b [n, K] the teacher's A / tau.  With
    q~ = softmax(a) and p^ = softmax(b) over the K entries,
        RKL = sum_k q~_k (log q~_k - log p^_k),
        dRKL/da_k = q~_k (log q~_k - log p^_k - RKL).
    Returns (RKL [n], dRKL/da [n, K])."""
    lq = a - logsumexp_rows(a)[:, None]
    lp = b - logsumexp_rows(b)[:, None]
    q = np.exp(lq)
    rkl = (q * (lq - lp)).sum(axis=1)
    return rkl, q * (lq - lp - rkl[:, None])


def _loss_dz(s, L, I_rows, p, m, y_rows, beta, g_rows, tau_rows):
    """dLoss/dz for a block of rows:
    (g/tau) [(1 - beta)(m q - scatter_add(I, p)) + beta (q - onehot(y))]."""
    q = np.exp(s - L[:, None])
    D = q * m[:, None]
    r = np.repeat(np.arange(s.shape[0]), I_rows.shape[1])
    np.add.at(D, (r, I_rows.reshape(-1)), -p.reshape(-1))  # duplicates add
    if y_rows is not None and beta != 0.0:
        E = q.copy()
        E[np.arange(s.shape[0]), y_rows] -= 1.0
        D = (1.0 - beta) * D + beta * E
    return D * (g_rows / tau_rows)[:, None]


def topk_loss_backward(H, W, I, A, mask, tau, g, tau_rows=None, teacher_lse=None, labels=None, ce_weight=0.0,
                       rev_weight=0.0, row_block=64, v_panel=16384, want_dw=True):
    """Gradients of sum_t g_t loss_t (topk_loss_forward) w.r.t. H and W:
    dZ_t as in _loss_dz, dH = dZ W^T, dW = H^T dZ, masked rows contribute
    nothing.  With r = rev_weight > 0 the forward-KL part is weighted 1 - r
    (p and m scaled, the dZ being linear in both) and the reverse part adds
    (g_t / tau_t)(1 - beta) r dRKL/da_k at column I_tk (scatter-add).
    Returns (dH [T, d], dW [d, V] or None without want_dw)."""
    H, W, A, g = as_f64(H), as_f64(W), as_f64(A), as_f64(g)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, d = H.shape
    V = W.shape[1]
    taus = _row_values(tau_rows, T, tau)
    tlse = None if teacher_lse is None else _row_values(teacher_lse, T, 0.0)
    y = None if labels is None else np.asarray(labels.cpu().numpy() if hasattr(labels, "cpu") else labels,
                                               dtype=np.int64)
    beta = float(ce_weight)
    r = float(rev_weight)
    valid = _valid_rows(mask, T)
    dH, dW = np.zeros((T, d)), (np.zeros((d, V)) if want_dw else None)
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, L, p, _, m = _loss_block(H, W, A, rb, taus, tlse)
        D = _loss_dz(s, L, I[rb], (1.0 - r) * p, (1.0 - r) * m, None if y is None else y[rb], beta, g[rb],
                     taus[rb])
        if r != 0.0:
            _, da = _support_reverse(np.take_along_axis(s, I[rb], axis=1), A[rb] / taus[rb][:, None])
            wr = r * (1.0 - beta if y is not None else 1.0) * g[rb] / taus[rb]
            n = rb.size
            np.add.at(D, (np.repeat(np.arange(n), I.shape[1]), I[rb].reshape(-1)),
                      (da * wr[:, None]).reshape(-1))  # duplicates add
        dH[rb] = D @ W.T
        if want_dw:
            for v0 in range(0, V, v_panel):
                dW[:, v0:v0 + v_panel] += H[rb].T @ D[:, v0:v0 + v_panel]
    return dH, dW


def topk_loss_rows(H, W, I, A, mask, tau, g, rows, tau_rows=None, teacher_lse=None, labels=None, ce_weight=0.0,
                   rev_weight=0.0):
    """loss, lse, z_topk and dH of topk_loss_* for selected rows only."""
    rows = np.asarray(rows, dtype=np.int64)
    Hr, Ir, Ar = as_f64(_take_rows(H, rows)), _take_rows(I, rows), _take_rows(A, rows)
    mr, gr = _take_rows(mask, rows), _take_rows(g, rows)
    kw = dict(tau_rows=_take_rows(tau_rows, rows), teacher_lse=_take_rows(teacher_lse, rows),
              labels=_take_rows(labels, rows), ce_weight=ce_weight, rev_weight=rev_weight)
    W = as_f64(W)
    loss, lse, ztk = topk_loss_forward(Hr, W, Ir, Ar, mr, tau, **kw)
    dH, _ = topk_loss_backward(Hr, W, Ir, Ar, mr, tau, gr, want_dw=False, **kw)
    return loss, lse, ztk, dH


def topk_shard_terms(H, W_shard, v0, I, A, mask, tau, tau_rows=None, teacher_lse=None, labels=None,
                     ce_weight=0.0):
    """The terms of topk_loss_forward that one vocabulary shard of the head
    holds, W_shard being columns [v0, v0 + Vs) of W (the head split by
    vocabulary columns across tensor-parallel ranks; [EKD] App. B reports the
    loss benchmark at the largest tensor-parallel rank).  Per valid row t, with
    s = (H_t W_shard) / tau_t and the support weights w (p_k, times 1 - beta
    with a CE label, which weighs beta):
        lse_shard_t = logsumexp over the shard's columns of s
        cross_t     = sum of w_k s[I_tk - v0] over the entries inside the shard
        ent_t       = sum of w_k log p_k over all K entries
        mass_t      = m_t, or (1 - beta) m_t + beta with a label
    so that over a partition of the vocabulary into shards
        L_t = logsumexp_shards(lse_shard_t),
        loss_t = ent_t - sum_shards(cross_t) + mass_t L_t.
    Masked rows give zeros.  Returns (lse_shard, cross, ent, mass), each [T]."""
    H, W_shard, A = as_f64(H), as_f64(W_shard), as_f64(A)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, K = I.shape
    Vs = W_shard.shape[1]
    taus = _row_values(tau_rows, T, tau)
    tlse = None if teacher_lse is None else _row_values(teacher_lse, T, 0.0)
    y = None if labels is None else np.asarray(labels.cpu().numpy() if hasattr(labels, "cpu") else labels,
                                               dtype=np.int64)
    beta = float(ce_weight) if y is not None else 0.0
    valid = _valid_rows(mask, T)
    out = [np.zeros(T) for _ in range(4)]
    for t in np.nonzero(valid)[0]:
        _, s, Ls, p, logp, m = _loss_block(H, W_shard, A, np.array([t]), taus, tlse)
        s, p, logp = s[0], p[0], logp[0]
        wk = 1.0 - beta
        cross = 0.0
        for k in range(K):
            j = I[t, k] - v0
            if 0 <= j < Vs:
                cross += wk * p[k] * s[j]
        if beta != 0.0 and 0 <= y[t] - v0 < Vs:
            cross += beta * s[y[t] - v0]
        out[0][t] = Ls[0]
        out[1][t] = cross
        out[2][t] = wk * float((p * logp).sum())
        out[3][t] = wk * float(m[0]) + beta
    return tuple(out)


def topk_shard_backward(H, W, v0, Vs, I, A, mask, tau, g, tau_rows=None, teacher_lse=None, labels=None,
                        ce_weight=0.0, row_block=64):
    """One vocabulary shard's part of topk_loss_backward: with dZ the whole
    head's gradient (_loss_dz, whose softmax needs every column of W) and
    columns c = [v0, v0 + Vs), the shard's dH partial dZ[:, c] W[:, c]^T and
    its columns of dW, H^T dZ[:, c].  Summed over a partition of the columns,
    the partials give dH.  Returns (dH_partial [T, d], dW_shard [d, Vs])."""
    H, W, A, g = as_f64(H), as_f64(W), as_f64(A), as_f64(g)
    I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
    T, d = H.shape
    taus = _row_values(tau_rows, T, tau)
    tlse = None if teacher_lse is None else _row_values(teacher_lse, T, 0.0)
    y = None if labels is None else np.asarray(labels.cpu().numpy() if hasattr(labels, "cpu") else labels,
                                               dtype=np.int64)
    beta = float(ce_weight)
    valid = _valid_rows(mask, T)
    dH, dW = np.zeros((T, d)), np.zeros((d, Vs))
    Wc = W[:, v0:v0 + Vs]
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, L, p, _, m = _loss_block(H, W, A, rb, taus, tlse)
        D = _loss_dz(s, L, I[rb], p, m, None if y is None else y[rb], beta, g[rb], taus[rb])[:, v0:v0 + Vs]
        dH[rb] = D @ Wc.T
        dW += H[rb].T @ D
    return dH, dW


def full_kl_forward(H, Ws, Ht, Wt, mask, tau, row_block=64):
    """Full-vocabulary KL(p_t || q_t) with teacher logits recomputed through a
    frozen teacher head ([KDFlow]; objective as [EKD] §1).

    u = (Ht_t Wt) / tau, s = (H_t Ws) / tau, p = softmax(u):
        KL_t = sum_v p_v (u_v - s_v) - logsumexp(u) + logsumexp(s).
    Returns (kl [T], lse_s [T], lse_t [T])."""
    H, Ws, Ht, Wt = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt)
    T = H.shape[0]
    valid = _valid_rows(mask, T)
    kl, ls, lt = np.zeros(T), np.zeros(T), np.zeros(T)
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, Ls = _student_block(H[rb], Ws, tau)
        _, u, Lt = _student_block(Ht[rb], Wt, tau)
        p = np.exp(u - Lt[:, None])
        kl[rb] = (p * (u - s)).sum(axis=1) - Lt + Ls
        ls[rb], lt[rb] = Ls, Lt
    return kl, ls, lt


def full_kl_backward(H, Ws, Ht, Wt, mask, tau, g, row_block=64, v_panel=16384):
    """Gradients of sum_t g_t KL_t w.r.t. the student's H and Ws only (the
    teacher head is frozen, [KDFlow]).  dZ_t = (g_t / tau)(softmax(s_t) - p_t);
    dH = dZ Ws^T; dWs = H^T dZ.  Returns (dH, dWs)."""
    H, Ws, Ht, Wt, g = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt), as_f64(g)
    T, d = H.shape
    V = Ws.shape[1]
    valid = _valid_rows(mask, T)
    dH = np.zeros((T, d))
    dW = np.zeros((d, V))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, Ls = _student_block(H[rb], Ws, tau)
        _, u, Lt = _student_block(Ht[rb], Wt, tau)
        D = (np.exp(s - Ls[:, None]) - np.exp(u - Lt[:, None])) * (g[rb] / tau)[:, None]
        dH[rb] = D @ Ws.T
        for v0 in range(0, V, v_panel):
            dW[:, v0:v0 + v_panel] += H[rb].T @ D[:, v0:v0 + v_panel]
    return dH, dW


def full_kl_rows(H, Ws, Ht, Wt, mask, tau, g, rows):
    """kl, lse_s, lse_t and dH for selected rows (each depends only on its own
    row and the two heads)."""
    rows = np.asarray(rows, dtype=np.int64)
    Hr, Htr = as_f64(_take_rows(H, rows)), as_f64(_take_rows(Ht, rows))
    mr, gr = _take_rows(mask, rows), _take_rows(g, rows)
    Ws, Wt = as_f64(Ws), as_f64(Wt)
    kl, ls, lt = full_kl_forward(Hr, Ws, Htr, Wt, mr, tau)
    dH, _ = _rows_dh_full(Hr, Ws, Htr, Wt, mr, tau, gr)
    return kl, ls, lt, dH


def _rows_dh_full(H, Ws, Ht, Wt, mask, tau, g, row_block=64):
    H, Ws, Ht, Wt, g = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt), as_f64(g)
    T, d = H.shape
    valid = _valid_rows(mask, T)
    dH = np.zeros((T, d))
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        _, s, Ls = _student_block(H[rb], Ws, tau)
        _, u, Lt = _student_block(Ht[rb], Wt, tau)
        D = (np.exp(s - Ls[:, None]) - np.exp(u - Lt[:, None])) * (g[rb] / tau)[:, None]
        dH[rb] = D @ Ws.T
    return dH, None


def _full_block(H, Ws, Ht, Wt, rb, taus):
    """Both heads' scaled logits of a block of valid rows and their softmaxes."""
    tau = taus[rb][:, None]
    s = (H[rb] @ Ws) / tau
    u = (Ht[rb] @ Wt) / tau
    Ls, Lt = logsumexp_rows(s), logsumexp_rows(u)
    q = np.exp(s - Ls[:, None])
    p = np.exp(u - Lt[:, None])
    return s, u, Ls, Lt, q, p


def full_loss_forward(H, Ws, Ht, Wt, mask, tau, tau_rows=None, rev_weight=0.0, row_block=64):
    """Full-vocabulary loss with KL mixing ([KLD]) and per-token temperature
    ([AKD]), teacher logits through the frozen teacher head ([KDFlow]).

    Per valid row t at temperature tau_t, with s = H_t Ws / tau_t, u = Ht_t Wt / tau_t,
    q = softmax(s), p = softmax(u):
        KLf = sum_v p_v (u_v - s_v) - logsumexp(u) + logsumexp(s)     KL(p || q)
        KLr = sum_v q_v (s_v - u_v) - logsumexp(s) + logsumexp(u)     KL(q || p)
        loss = (1 - r) KLf + r KLr.
    Returns (loss [T], lse_s [T], lse_t [T], kl_rev [T])."""
    H, Ws, Ht, Wt = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt)
    T = H.shape[0]
    taus = _row_values(tau_rows, T, tau)
    r = float(rev_weight)
    valid = _valid_rows(mask, T)
    loss, ls, lt, krev = np.zeros(T), np.zeros(T), np.zeros(T), np.zeros(T)
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        s, u, Ls, Lt, q, p = _full_block(H, Ws, Ht, Wt, rb, taus)
        klf = (p * (u - s)).sum(axis=1) - Lt + Ls
        klr = (q * (s - u)).sum(axis=1) - Ls + Lt
        loss[rb] = (1.0 - r) * klf + r * klr
        ls[rb], lt[rb], krev[rb] = Ls, Lt, klr
    return loss, ls, lt, krev


def _full_loss_dz(s, u, Ls, Lt, q, p, g_rows, tau_rows, r):
    """dLoss/dz_s: (g/tau) [(1 - r)(q - p) + r q ((s - Ls) - (u - Lt) - KLr)]."""
    D = (1.0 - r) * (q - p)
    if r != 0.0:
        lr = (s - Ls[:, None]) - (u - Lt[:, None])
        klr = (q * lr).sum(axis=1)
        D = D + r * q * (lr - klr[:, None])
    return D * (g_rows / tau_rows)[:, None]


def full_loss_backward(H, Ws, Ht, Wt, mask, tau, g, tau_rows=None, rev_weight=0.0, row_block=64, v_panel=16384,
                       want_dw=True):
    """Gradients of sum_t g_t loss_t (full_loss_forward) w.r.t. the student's
    H and Ws only.  Returns (dH [T, d], dWs [d, V] or None)."""
    H, Ws, Ht, Wt, g = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt), as_f64(g)
    T, d = H.shape
    V = Ws.shape[1]
    taus = _row_values(tau_rows, T, tau)
    valid = _valid_rows(mask, T)
    dH, dW = np.zeros((T, d)), (np.zeros((d, V)) if want_dw else None)
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        s, u, Ls, Lt, q, p = _full_block(H, Ws, Ht, Wt, rb, taus)
        D = _full_loss_dz(s, u, Ls, Lt, q, p, g[rb], taus[rb], float(rev_weight))
        dH[rb] = D @ Ws.T
        if want_dw:
            for v0 in range(0, V, v_panel):
                dW[:, v0:v0 + v_panel] += H[rb].T @ D[:, v0:v0 + v_panel]
    return dH, dW


def full_shard_terms(H, Ws_shard, Ht, Wt_shard, mask, tau, tau_rows=None):
    """What one vocabulary shard of both heads holds of full_loss_forward
    (columns c of both heads; [EKD] App. B: tensor-parallel ranks).  Per
    valid row t, with s and u the student's and teacher's scaled logits over
    c and P, Q their softmaxes restricted to c:
        lse_s_t, lse_t_t = logsumexp over c of s, of u
        e_fwd_t = sum over c of P (u - s),  e_rev_t = sum over c of Q (s - u)
    so that over a partition of the vocabulary, with L = logsumexp of the
    shards' lse and w_r = exp(lse_r - L) the shards' shares of the mass,
        KL(p||q) = sum_r w_t,r e_fwd_r - Lt + Ls,
        KL(q||p) = sum_r w_s,r e_rev_r - Ls + Lt.
    Masked rows give zeros.  Returns (lse_s, lse_t, e_fwd, e_rev), each [T]."""
    H, Ws_shard, Ht, Wt_shard = as_f64(H), as_f64(Ws_shard), as_f64(Ht), as_f64(Wt_shard)
    T = H.shape[0]
    taus = _row_values(tau_rows, T, tau)
    valid = _valid_rows(mask, T)
    out = [np.zeros(T) for _ in range(4)]
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, 64):
        rb = rows[r0:r0 + 64]
        s, u, Ls, Lt, Q, P = _full_block(H, Ws_shard, Ht, Wt_shard, rb, taus)
        out[0][rb], out[1][rb] = Ls, Lt
        out[2][rb] = (P * (u - s)).sum(axis=1)
        out[3][rb] = (Q * (s - u)).sum(axis=1)
    return tuple(out)


def full_shard_backward(H, Ws, Ht, Wt, v0, Vs, mask, tau, g, tau_rows=None, rev_weight=0.0, row_block=64):
    """One vocabulary shard's part of full_loss_backward: with dZ the whole
    heads' gradient (_full_loss_dz, whose softmaxes need every column) and
    columns c = [v0, v0 + Vs), the dH partial dZ[:, c] Ws[:, c]^T and the
    columns c of dWs, H^T dZ[:, c].  Returns (dH_partial [T, d], dWs [d, Vs])."""
    H, Ws, Ht, Wt, g = as_f64(H), as_f64(Ws), as_f64(Ht), as_f64(Wt), as_f64(g)
    T, d = H.shape
    taus = _row_values(tau_rows, T, tau)
    valid = _valid_rows(mask, T)
    dH, dW = np.zeros((T, d)), np.zeros((d, Vs))
    Wc = Ws[:, v0:v0 + Vs]
    rows = np.nonzero(valid)[0]
    for r0 in range(0, rows.size, row_block):
        rb = rows[r0:r0 + row_block]
        s, u, Ls, Lt, q, p = _full_block(H, Ws, Ht, Wt, rb, taus)
        D = _full_loss_dz(s, u, Ls, Lt, q, p, g[rb], taus[rb], float(rev_weight))[:, v0:v0 + Vs]
        dH[rb] = D @ Wc.T
        dW += H[rb].T @ D
    return dH, dW


def full_loss_rows(H, Ws, Ht, Wt, mask, tau, g, rows, tau_rows=None, rev_weight=0.0):
    """loss, lse_s, lse_t, kl_rev and dH of full_loss_* for selected rows."""
    rows = np.asarray(rows, dtype=np.int64)
    Hr, Htr = as_f64(_take_rows(H, rows)), as_f64(_take_rows(Ht, rows))
    mr, gr = _take_rows(mask, rows), _take_rows(g, rows)
    kw = dict(tau_rows=_take_rows(tau_rows, rows), rev_weight=rev_weight)
    Ws, Wt = as_f64(Ws), as_f64(Wt)
    out = full_loss_forward(Hr, Ws, Htr, Wt, mr, tau, **kw)
    dH, _ = full_loss_backward(Hr, Ws, Htr, Wt, mr, tau, gr, want_dw=False, **kw)
    return out + (dH,)
